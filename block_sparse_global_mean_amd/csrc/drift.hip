// Drift contributions of every key block to every pooled query block for fp32
// inputs (vector ALU; bf16 inputs take the matrix-core kernels of
// drift_mfma.hip), and the drift selection with swap restoration.
//
// Contributions: for pooled query i and real key token u,
//   e_u = exp(scale <qbar_i, k_u> - M_i),  M_i = max_u scale <qbar_i, k_u>,
//   contrib_ij = sum_{u in j} e_u v_u / Z_i,  Z_i = sum_u e_u,  score_ij = ||contrib_ij||,
//   zmass_ij = sum_{u in j} e_u / Z_i (optional).
// Pass 1 finds (M_i, Z_i) with an online log-sum-exp; pass 2 walks the key
// blocks and writes contrib and score. All arithmetic is fp32. The same
// kernel serves the re-rank rounds without the contributions (the expanded
// score): squared scores only, the residual r_i of a drop set, and the dot
// products <r_i, contrib_ij>, each from the contributions it forms and drops.
#include <algorithm>

#include "device_util.h"

namespace bsgm {

constexpr int kDriftRows = 8;   // pooled query rows per workgroup

// What pass 2 of k_drift_contrib produces.
enum DriftF32Mode {
  kF32Contrib = 0,   // contrib, score (and zmass)
  kF32SqNorm = 1,    // score = ||contrib_ij||^2 only
  kF32Resid = 2,     // part[row] = sum of the contributions of the counted blocks
  kF32Dot = 3        // dot[row, j] = <r_row, contrib_ij>
};

struct DriftF32Round {
  const uint32_t* kept;   // [rows, W] kept sets, or null: every block counts
  int via_kept;           // count the kept blocks, else the dropped ones
  float* part;            // [rows, 64]
  const __bf16* rsplit;   // [rows, 3, 64]: r as three bf16 terms (exact sum)
  float* dot;             // [rows, nb]
};

template <typename T>
__device__ __forceinline__ void load_row64(const T* p, float (&x)[64]) {
  constexpr int E = 16 / sizeof(T);
#pragma unroll
  for (int c = 0; c < 64 / E; ++c) {
    const uint4 raw = *reinterpret_cast<const uint4*>(p + c * E);
    const T* v = reinterpret_cast<const T*>(&raw);
#pragma unroll
    for (int e = 0; e < E; ++e) x[c * E + e] = (float)v[e];
  }
}

template <typename T, int MODE>
__global__ __launch_bounds__(256) void k_drift_contrib(const float* __restrict__ qbar,
                                                       const T* __restrict__ K,
                                                       const T* __restrict__ V,
                                                       float* __restrict__ contrib,
                                                       float* __restrict__ score,
                                                       float* __restrict__ zmass, Dims d,
                                                       DriftF32Round rd) {
  __shared__ float qs[kDriftRows][64];
  __shared__ float E[kDriftRows][128];
  __shared__ float Vs[128][65];
  __shared__ float redm[4][kDriftRows], redz[4][kDriftRows];
  __shared__ float Ms[kDriftRows], Zinv[kDriftRows];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int i0 = blockIdx.x * kDriftRows;
  const int bh = blockIdx.y;
  const size_t hoff = (size_t)bh * d.N * 64;
  for (int x = t; x < kDriftRows * 64; x += 256) {
    const int ii = i0 + x / 64;
    qs[x / 64][x % 64] = ii < d.nb ? qbar[((size_t)bh * d.nb + ii) * 64 + (x % 64)] : 0.f;
  }
  __syncthreads();

  // Pass 1: per-thread online (max, sum) over its keys, then merged.
  float m[kDriftRows], z[kDriftRows];
#pragma unroll
  for (int r = 0; r < kDriftRows; ++r) { m[r] = -INFINITY; z[r] = 0.f; }
  for (int u = t; u < d.N; u += 256) {
    if ((u % d.L) >= d.Lv) continue;
    float kv[64];
    load_row64<T>(K + hoff + (size_t)u * 64, kv);
#pragma unroll
    for (int r = 0; r < kDriftRows; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < 64; ++c) acc = fmaf(qs[r][c], kv[c], acc);
      const float l = d.scale * acc;
      if (l > m[r]) {
        z[r] = z[r] * expf(m[r] - l) + 1.f;
        m[r] = l;
      } else {
        z[r] += expf(l - m[r]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kDriftRows; ++r) {
    float mr = m[r], zr = z[r];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float mo = __shfl_xor(mr, o, 64), zo = __shfl_xor(zr, o, 64);
      const float mn = fmaxf(mr, mo);
      zr = (mn == -INFINITY) ? 0.f : zr * expf(mr - mn) + zo * expf(mo - mn);
      mr = mn;
    }
    if (lane == 0) { redm[w][r] = mr; redz[w][r] = zr; }
  }
  __syncthreads();
  if (t < kDriftRows) {
    float mr = redm[0][t], zr = redz[0][t];
    for (int q = 1; q < 4; ++q) {
      const float mo = redm[q][t], zo = redz[q][t];
      const float mn = fmaxf(mr, mo);
      zr = (mn == -INFINITY) ? 0.f : zr * expf(mr - mn) + zo * expf(mo - mn);
      mr = mn;
    }
    Ms[t] = mr;
    Zinv[t] = 1.f / zr;
  }
  __syncthreads();

  // Pass 2: per key block, weights e_u / Z into LDS, then contrib = E V.
  const int ri = t >> 5;            // output row of this thread
  const int dp = (t & 31) * 2;      // output column pair
  const int irow = min(i0 + ri, d.nb - 1);
  const size_t grow = (size_t)bh * d.nb + irow;
  const int W = (d.nb + 31) >> 5;
  float rs0 = 0.f, rs1 = 0.f;       // kF32Resid: the running sum; kF32Dot: r
  if (MODE == kF32Dot) {
    const __bf16* rp = rd.rsplit + grow * 192 + dp;
    rs0 = ((float)rp[0] + (float)rp[64]) + (float)rp[128];
    rs1 = ((float)rp[1] + (float)rp[65]) + (float)rp[129];
  }
  for (int j = 0; j < d.nb; ++j) {
    const int vlen = block_vlen(d, j);
    const size_t tok0 = (size_t)j * d.blk;
    if (t < d.blk) {
      float ew[kDriftRows];
      if (t < vlen) {
        float kv[64];
        load_row64<T>(K + hoff + (tok0 + t) * 64, kv);
#pragma unroll
        for (int r = 0; r < kDriftRows; ++r) {
          float acc = 0.f;
#pragma unroll
          for (int c = 0; c < 64; ++c) acc = fmaf(qs[r][c], kv[c], acc);
          ew[r] = expf(d.scale * acc - Ms[r]) * Zinv[r];
        }
      } else {
#pragma unroll
        for (int r = 0; r < kDriftRows; ++r) ew[r] = 0.f;
      }
#pragma unroll
      for (int r = 0; r < kDriftRows; ++r) E[r][t] = ew[r];
    }
    constexpr int EL = 16 / sizeof(T);
    for (int x = t; x < d.blk * (64 / EL); x += 256) {
      const int row = x / (64 / EL), c = x % (64 / EL);
      const uint4 raw = *reinterpret_cast<const uint4*>(V + hoff + (tok0 + row) * 64 + c * EL);
      const T* v = reinterpret_cast<const T*>(&raw);
#pragma unroll
      for (int e = 0; e < EL; ++e) Vs[row][c * EL + e] = row < vlen ? (float)v[e] : 0.f;
    }
    __syncthreads();
    float a0 = 0.f, a1 = 0.f, zs = 0.f;
    for (int u = 0; u < vlen; ++u) {
      const float e = E[ri][u];
      a0 = fmaf(e, Vs[u][dp], a0);
      a1 = fmaf(e, Vs[u][dp + 1], a1);
      zs += e;
    }
    const int ii = i0 + ri;
    if (MODE == kF32Resid) {
      const bool in = rd.kept == nullptr ||
                      ((((rd.kept[grow * W + (j >> 5)] >> (j & 31)) & 1u) != 0) ==
                       (rd.via_kept != 0));
      if (in) {
        rs0 += a0;
        rs1 += a1;
      }
    } else if (MODE == kF32Dot) {
      float dt = fmaf(a1, rs1, a0 * rs0);
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) dt += __shfl_xor(dt, o, 64);
      if (ii < d.nb && (t & 31) == 0) rd.dot[((size_t)bh * d.nb + ii) * d.nb + j] = dt;
    } else {
      float sq = a0 * a0 + a1 * a1;
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) sq += __shfl_xor(sq, o, 64);
      if (ii < d.nb) {
        if (MODE == kF32Contrib) {
          float2* dst = reinterpret_cast<float2*>(
              contrib + (((size_t)bh * d.nb + ii) * d.nb + j) * 64 + dp);
          *dst = make_float2(a0, a1);
        }
        if ((t & 31) == 0)
          score[((size_t)bh * d.nb + ii) * d.nb + j] = MODE == kF32SqNorm ? sq : sqrtf(sq);
        if ((t & 31) == 0 && zmass) zmass[((size_t)bh * d.nb + ii) * d.nb + j] = zs;
      }
    }
    __syncthreads();
  }
  if (MODE == kF32Resid && i0 + ri < d.nb)
    *reinterpret_cast<float2*>(rd.part + grow * 64 + dp) = make_float2(rs0, rs1);
}

hipError_t launch_drift_contrib(const Dims& d, int dtype, const float* qbar, const void* k,
                                const void* v, float* contrib, float* score, float* zmass,
                                hipStream_t s) {
  if (dtype != 0) return hipErrorInvalidValue;   // bf16 takes launch_drift_contrib_bf16
  dim3 grid((d.nb + kDriftRows - 1) / kDriftRows, d.B * d.H);
  hipLaunchKernelGGL((k_drift_contrib<float, kF32Contrib>), grid, dim3(256), 0, s, qbar,
                     (const float*)k, (const float*)v, contrib, score, zmass, d, DriftF32Round{});
  return hipGetLastError();
}

hipError_t launch_drift_sqnorms_f32(const Dims& d, const float* qbar, const void* k, const void* v,
                                    float* sqnorm, hipStream_t s) {
  dim3 grid((d.nb + kDriftRows - 1) / kDriftRows, d.B * d.H);
  hipLaunchKernelGGL((k_drift_contrib<float, kF32SqNorm>), grid, dim3(256), 0, s, qbar,
                     (const float*)k, (const float*)v, nullptr, sqnorm, nullptr, d,
                     DriftF32Round{});
  return hipGetLastError();
}

hipError_t launch_drift_residual_f32(const Dims& d, const float* qbar, const void* k,
                                     const void* v, const uint32_t* kept, int via_kept,
                                     float* obar, float* part, void* rsplit, float* jsq,
                                     uint32_t* best, float* jbest, int round, hipStream_t s) {
  dim3 grid((d.nb + kDriftRows - 1) / kDriftRows, d.B * d.H);
  DriftF32Round rd{kept, via_kept, part, nullptr, nullptr};
  hipLaunchKernelGGL((k_drift_contrib<float, kF32Resid>), grid, dim3(256), 0, s, qbar,
                     (const float*)k, (const float*)v, nullptr, nullptr, nullptr, d, rd);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_drift_resid(d, kept, via_kept, obar, part, 1, rsplit, jsq, best, jbest, round, s);
}

hipError_t launch_drift_dot_f32(const Dims& d, const float* qbar, const void* rsplit,
                                const void* k, const void* v, float* dot, hipStream_t s) {
  dim3 grid((d.nb + kDriftRows - 1) / kDriftRows, d.B * d.H);
  DriftF32Round rd{nullptr, 0, nullptr, (const __bf16*)rsplit, dot};
  hipLaunchKernelGGL((k_drift_contrib<float, kF32Dot>), grid, dim3(256), 0, s, qbar,
                     (const float*)k, (const float*)v, nullptr, nullptr, nullptr, d, rd);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Drift selection: one workgroup per row.
//
// Two objectives share the swap machinery. Dropped-sum drift: rows x_j = c_j,
// residual r = sum_{j in D} x_j, J = ||r||. Renormalised output shift (the
// pooled query's attention output over the kept blocks, renormalised, minus its
// dense output o = sum_j c_j): with z_j the block's normalised mass and S the
// kept set, J = ||sum_S c_j / sum_S z_j - o|| = ||u|| / Z_S where u = sum_S (c_j
// - z_j o); with rows x_j = z_j o - c_j, u = sum_D x_j + (1 - sum_j z_j) o, and
// a swap moves u exactly like r: u' = u - x_a + x_b, Z_S' = Z_S + z_a - z_b.
// The first objective ranks swaps by delta below, the second by
// (||u||^2 + delta) / Z_S'^2.
//
// With D the dropped blocks, S the kept non-forced blocks, r = sum_{j in D} c_j,
// g_j = <r, c_j> and G_ab = <c_a, c_b>, restoring a in D and dropping b in S gives
//   J^2(a, b) = ||r - c_a + c_b||^2 = ||r||^2 + delta(a, b),
//   delta(a, b) = (|c_a|^2 - 2 g_a) + (|c_b|^2 + 2 g_b) - 2 G_ab.
// A round takes the pair of least delta (ties: lower a, then lower b) and swaps
// it if delta < 0.
//
// LDS holds the contributions of D and S in slot order (D slots first, then S
// slots; forced blocks never move and are not needed). A swap exchanges the two
// slots' rows and updates r by -c_a + c_b. G over D x S does not depend on r:
// when it fits it is computed once per row into LDS, on the matrix cores with
// fp32 accuracy, and a swap refreshes one row and one column of it; g is then
// updated in place (g'_j = g_j - <c_a, c_j> + <c_b, c_j>, all of whose terms
// are old entries of G or products of the refresh). Otherwise every round
// recomputes g and the pair products on the vector ALU.
// ---------------------------------------------------------------------------
struct DriftSelArgs {
  Dims d;
  HeadBudget hb;
  int force;
  int rounds;
  int renorm;            // objective: 0 dropped-sum drift, 1 renormalised output shift
  const float* contrib;
  const float* zmass;    // renorm only: [rows, nb] normalised block masses
  int32_t* row_ptr;
  int32_t* col_idx;
  float* row_stat;
  int32_t* swap_log;
};

constexpr int kCs = 68;          // LDS row stride (floats): 16-byte aligned, rows 4 banks apart
constexpr int kTa = 3, kTb = 4;  // register tile of dot products: kTa D slots x kTb S slots
constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / 64;
// float4 registers per thread that hold a whole row of contributions: RR = 8
// for rows of up to 256 blocks, 16 up to kDriftLdsRowBlocks
// Dynamic LDS a selection workgroup may take (the static arrays need < 4 KB).
constexpr size_t kDriftSelLdsCap = 160 * 1024 - 6144;

template <typename P>
__device__ __forceinline__ float dot64(const P* x, const float* y) {
  const float4* x4 = reinterpret_cast<const float4*>(x);
  const float4* y4 = reinterpret_cast<const float4*>(y);
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int c = 0; c < 16; c += 2) {
    const float4 a0 = x4[c], b0 = y4[c], a1 = x4[c + 1], b1 = y4[c + 1];
    s0 = fmaf(a0.x, b0.x, s0); s0 = fmaf(a0.y, b0.y, s0);
    s0 = fmaf(a0.z, b0.z, s0); s0 = fmaf(a0.w, b0.w, s0);
    s1 = fmaf(a1.x, b1.x, s1); s1 = fmaf(a1.y, b1.y, s1);
    s1 = fmaf(a1.z, b1.z, s1); s1 = fmaf(a1.w, b1.w, s1);
  }
  return s0 + s1;
}

// LDS carve-up of one row (byte offsets).
struct DriftSelLds {
  size_t cs, slot, gs, keys, slot_of, zb, G, total;
};

__host__ __device__ inline DriftSelLds drift_sel_lds(int nb, int nslots, size_t gfloats) {
  DriftSelLds L;
  size_t o = 0;
  L.cs = o;      o += (size_t)nslots * kCs * 4;  // slot rows
  L.slot = o;    o += (size_t)nslots * 16;       // per slot: |c|^2, weight, block, mass
  L.gs = o;      o += (size_t)nslots * 4;        // per slot: g = <r, x>
  o = (o + 15) & ~(size_t)15;
  L.keys = o;    o += (size_t)((nb + 1) & ~1) * 8;   // priority keys by block (even count)
  L.slot_of = o; o += (size_t)nb * 4;            // slot of each block (-1: forced)
  L.zb = o;      o += (size_t)nb * 4;            // normalised block mass (renorm)
  o = (o + 15) & ~(size_t)15;
  L.G = o;       o += gfloats * 4;               // G[D slot][S slot]
  L.total = o;
  return L;
}

struct SlotRec {
  float cc;    // |x|^2
  float wgt;   // |x|^2 - 2 g (D slot) or |x|^2 + 2 g (S slot)
  int blk;     // key block in this slot
  float z;     // normalised block mass (renorm)
};

// Renormalised objective of a candidate: (||u||^2 + delta) / Z'^2 (never negative).
__device__ __forceinline__ float renorm_j2(float rr, float dlt, float zs) {
  return zs > 0.f ? fmaxf(rr + dlt, 0.f) / (zs * zs) : INFINITY;
}

// Least 64-bit key over the wave (all lanes active), on the DPP and lane-swap
// paths: every lane gets the minimum.
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_min_u64(unsigned long long x) {
  const uint32_t lo = dpp_mov_u<CTRL>((uint32_t)x), hi = dpp_mov_u<CTRL>((uint32_t)(x >> 32));
  const unsigned long long y = ((unsigned long long)hi << 32) | lo;
  return y < x ? y : x;
}
__device__ __forceinline__ unsigned long long wave_allmin_u64(unsigned long long x) {
  x = dpp_min_u64<0xB1>(x);    // quad_perm [1,0,3,2]
  x = dpp_min_u64<0x4E>(x);    // quad_perm [2,3,0,1]
  x = dpp_min_u64<0x141>(x);   // row_half_mirror
  x = dpp_min_u64<0x140>(x);   // row_mirror
  {
    const auto l = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
    const auto h = __builtin_amdgcn_permlane16_swap((uint32_t)(x >> 32), (uint32_t)(x >> 32), false, false);
    const unsigned long long u = ((unsigned long long)h[0] << 32) | l[0];
    const unsigned long long v = ((unsigned long long)h[1] << 32) | l[1];
    x = u < v ? u : v;
  }
  {
    const auto l = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
    const auto h = __builtin_amdgcn_permlane32_swap((uint32_t)(x >> 32), (uint32_t)(x >> 32), false, false);
    const unsigned long long u = ((unsigned long long)h[0] << 32) | l[0];
    const unsigned long long v = ((unsigned long long)h[1] << 32) | l[1];
    x = u < v ? u : v;
  }
  return x;
}

typedef __attribute__((ext_vector_type(2))) __bf16 sel_bf16x2;
typedef __attribute__((ext_vector_type(2))) float sel_f32x2;

// x = hi + mid + lo exactly, each a bf16 (barring subnormal residuals).
__device__ __forceinline__ void sel_split3(const float (&x)[8], bf16x8& hi, bf16x8& mid,
                                           bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const sel_f32x2 v = {x[2 * e], x[2 * e + 1]};
    const sel_bf16x2 h = __builtin_convertvector(v, sel_bf16x2);
    const sel_f32x2 r1 = v - __builtin_convertvector(h, sel_f32x2);
    const sel_bf16x2 m = __builtin_convertvector(r1, sel_bf16x2);
    const sel_f32x2 r2 = r1 - __builtin_convertvector(m, sel_f32x2);
    const sel_bf16x2 l = __builtin_convertvector(r2, sel_bf16x2);
    hi[2 * e] = h[0];
    hi[2 * e + 1] = h[1];
    mid[2 * e] = m[0];
    mid[2 * e + 1] = m[1];
    lo[2 * e] = l[0];
    lo[2 * e + 1] = l[1];
  }
}

// Head dims 32 ks + 8 (lane / 16) .. +7 of LDS slot row `row` (zeros when the
// row is past `nrows`), split in three bf16 terms: one operand fragment of
// v_mfma_f32_16x16x32_bf16 (lane l gives row or column l % 16).
__device__ __forceinline__ void sel_frag(const float* cs, int row, int nrows, int ks, int lane,
                                         bf16x8& h, bf16x8& m, bf16x8& l) {
  float x[8];
  if (row < nrows) {
    const float4* p = reinterpret_cast<const float4*>(cs + row * kCs + 32 * ks + 8 * (lane >> 4));
    const float4 u = p[0], v = p[1];
    x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
    x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = 0.f;
  }
  sel_split3(x, h, m, l);
}

template <bool CACHE, int RR>
__global__ __launch_bounds__(kSelThreads, 4) void k_select_drift(DriftSelArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char dsm[];
  const Dims& d = a.d;
  const int nb = d.nb;
  const int r = blockIdx.x;
  const int bh = r / nb, i = r - bh * nb;
  const int h = bh % d.H, b = bh / d.H;
  const int k = a.hb.keep[h];
  const int nd = nb - k, ns = k - (a.force ? d.F : 0), nsl = nd + ns;
  const DriftSelLds L = drift_sel_lds(nb, nsl, CACHE ? (size_t)nd * ns : 0);
  float* cs = reinterpret_cast<float*>(dsm + L.cs);
  SlotRec* slot = reinterpret_cast<SlotRec*>(dsm + L.slot);
  float* gs = reinterpret_cast<float*>(dsm + L.gs);
  unsigned long long* keys = reinterpret_cast<unsigned long long*>(dsm + L.keys);
  int* slot_of = reinterpret_cast<int*>(dsm + L.slot_of);
  float* zb = reinterpret_cast<float*>(dsm + L.zb);
  float* G = reinterpret_cast<float*>(dsm + L.G);
  const bool renorm = a.renorm != 0;
  __shared__ __attribute__((aligned(16))) float rv[64];
  __shared__ __attribute__((aligned(16))) float ob[64];
  __shared__ float redz[kSelWaves];
  __shared__ float part[kSelWaves][64];
  __shared__ int bks[kSelWaves];
  __shared__ unsigned long long bkey[kSelWaves];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;

  // the row, coalesced into registers: thread t holds chunk (t + 512 m) & 15 of
  // block (t + 512 m) >> 4; squared norms reduce over the 16 lanes of a block
  const float4* src = reinterpret_cast<const float4*>(
      a.contrib + ((size_t)bh * nb + i) * (size_t)nb * 64);
  float4 row[RR];
#pragma unroll
  for (int m = 0; m < RR; ++m) {
    const int x = t + kSelThreads * m;
    row[m] = x < nb * 16 ? src[x] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int m = 0; m < RR; ++m) {
    const int x = t + kSelThreads * m;
    if (kSelThreads * m < nb * 16) {
      float ss = row[m].x * row[m].x + row[m].y * row[m].y + row[m].z * row[m].z +
                 row[m].w * row[m].w;
      ss += __shfl_xor(ss, 8, 64);
      ss += __shfl_xor(ss, 4, 64);
      ss += __shfl_xor(ss, 2, 64);
      ss += __shfl_xor(ss, 1, 64);
      const int j = x >> 4;
      if ((x & 15) == 0 && j < nb) {
        const bool f = a.force && block_forced(d, j);
        const unsigned long long hi =
            f ? 0xFFFFFFFFull : (unsigned long long)orderable(sqrtf(ss));
        keys[j] = (hi << 32) | (unsigned long long)(~(uint32_t)j);
        slot_of[j] = __float_as_int(ss);   // the norm, until slots are known
      }
    }
  }
  if ((nb & 1) && t == 0) keys[nb] = 0ull;   // the even-count pad sorts below every key
  __syncthreads();
  // Initial kept set: the k keys of highest priority (forced, then norm, then
  // lower block; keys are distinct). Block j is ranked against every key by
  // threads j and j + 256 (half the keys each, two keys per LDS read) when
  // nb <= 256, else by thread j alone.
  bool kept_j = false, forced_j = false;
  float cc_j = 0.f;
  {
    const ulonglong2* k2 = reinterpret_cast<const ulonglong2*>(keys);
    const int npair = (nb + 1) >> 1;
    const bool split = nb <= kSelThreads / 2;
    const int jr = split ? (t & (kSelThreads / 2 - 1)) : t;
    const int q0 = split && t >= kSelThreads / 2 ? npair / 2 : 0;
    const int q1 = split && t < kSelThreads / 2 ? npair / 2 : npair;
    int rank = 0;
    if (jr < nb) {
      const unsigned long long kj = keys[jr];
#pragma unroll 4
      for (int q = q0; q < q1; ++q) {
        const ulonglong2 p = k2[q];
        rank += (p.x > kj ? 1 : 0) + (p.y > kj ? 1 : 0);
      }
    }
    if (split) {
      int* half = reinterpret_cast<int*>(&part[0][0]);
      if (t >= kSelThreads / 2 && jr < nb) half[jr] = rank;
      __syncthreads();
      if (t < nb) rank += half[t];
    }
    if (t < nb) {
      kept_j = rank < k;
      forced_j = a.force && block_forced(d, t);
      cc_j = __int_as_float(slot_of[t]);
    }
  }
  // slots: dropped blocks ascending, then kept non-forced blocks ascending
  {
    const bool isd = t < nb && !kept_j, iss = t < nb && kept_j && !forced_j;
    const unsigned long long md = __ballot(isd), ms = __ballot(iss);
    if (lane == 0) bkey[w] = ((unsigned long long)__popcll(md) << 32) | __popcll(ms);
    __syncthreads();
    int bd0 = 0, bs0 = 0;
    for (int q = 0; q < w; ++q) { bd0 += (int)(bkey[q] >> 32); bs0 += (int)(uint32_t)bkey[q]; }
    int sl = -1;
    if (isd) sl = bd0 + lanes_below(md);
    if (iss) sl = nd + bs0 + lanes_below(ms);
    if (t < nb) {
      slot_of[t] = sl;
      if (sl >= 0) slot[sl] = SlotRec{cc_j, 0.f, t, 0.f};
    }
  }
  __syncthreads();
  float ztot = 0.f;
  if (renorm) {
    // o = sum_j c_j (chunk c4 = t % 16 of every block this thread holds), z_j, sum_j z_j
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int m = 0; m < RR; ++m) {
      acc.x += row[m].x; acc.y += row[m].y; acc.z += row[m].z; acc.w += row[m].w;
    }
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      acc.x += __shfl_xor(acc.x, o, 64); acc.y += __shfl_xor(acc.y, o, 64);
      acc.z += __shfl_xor(acc.z, o, 64); acc.w += __shfl_xor(acc.w, o, 64);
    }
    if (lane < 16) *reinterpret_cast<float4*>(&part[w][4 * lane]) = acc;
    float zt = 0.f;
    if (t < nb) {
      zt = a.zmass[((size_t)bh * nb + i) * nb + t];
      zb[t] = zt;
    }
    zt = wave_sum(zt);
    if (lane == 0) redz[w] = zt;
    __syncthreads();
    if (t < 64) {
      float sacc = 0.f;
#pragma unroll
      for (int q = 0; q < kSelWaves; ++q) sacc += part[q][t];
      ob[t] = sacc;
    }
#pragma unroll
    for (int q = 0; q < kSelWaves; ++q) ztot += redz[q];
    __syncthreads();
  }
#pragma unroll
  for (int m = 0; m < RR; ++m) {
    const int x = t + kSelThreads * m;
    if (x < nb * 16) {
      const int sl = slot_of[x >> 4];
      if (sl >= 0) {
        float4 xv = row[m];
        if (renorm) {
          const float zj = zb[x >> 4];
          const float4 o4 = *reinterpret_cast<const float4*>(&ob[4 * (x & 15)]);
          xv = make_float4(zj * o4.x - xv.x, zj * o4.y - xv.y, zj * o4.z - xv.z, zj * o4.w - xv.w);
        }
        *reinterpret_cast<float4*>(cs + sl * kCs + 4 * (x & 15)) = xv;
      }
    }
  }
  __syncthreads();
  float z_s = 0.f;   // renorm: mass of the kept set
  if (renorm) {
    float zd = 0.f;
    for (int sl = t; sl < nsl; sl += kSelThreads) {
      const float zj = zb[slot[sl].blk];
      slot[sl].cc = dot64(cs + sl * kCs, cs + sl * kCs);
      slot[sl].z = zj;
      if (sl < nd) zd += zj;
    }
    zd = wave_sum(zd);
    if (lane == 0) redz[w] = zd;
    __syncthreads();
    zd = 0.f;
#pragma unroll
    for (int q = 0; q < kSelWaves; ++q) zd += redz[q];
    z_s = ztot - zd;
  }

  // kTa x kTb tiles of <c_a, c_b> on the vector ALU (rows too wide for the
  // cached products). Tile (ta, tb) takes D slots ta + x NTA and S slots
  // tb + y NTB, so that neighbouring lanes read neighbouring LDS rows.
  const int NTA = (nd + kTa - 1) / kTa, NTB = (ns + kTb - 1) / kTb, ntiles = NTA * NTB;
  auto tiles = [&](auto&& consume) {
    for (int tile = t; tile < ntiles; tile += kSelThreads) {
      const int ta = tile / NTB, tb = tile - ta * NTB;
      float acc[kTa][kTb];
#pragma unroll
      for (int x = 0; x < kTa; ++x)
#pragma unroll
        for (int y = 0; y < kTb; ++y) acc[x][y] = 0.f;
#pragma unroll 4
      for (int c = 0; c < 64; c += 4) {
        float4 av[kTa], bv[kTb];
#pragma unroll
        for (int x = 0; x < kTa; ++x)
          av[x] = *reinterpret_cast<const float4*>(cs + min(ta + x * NTA, nd - 1) * kCs + c);
#pragma unroll
        for (int y = 0; y < kTb; ++y)
          bv[y] = *reinterpret_cast<const float4*>(cs + (nd + min(tb + y * NTB, ns - 1)) * kCs + c);
#pragma unroll
        for (int x = 0; x < kTa; ++x)
#pragma unroll
          for (int y = 0; y < kTb; ++y) {
            acc[x][y] = fmaf(av[x].x, bv[y].x, acc[x][y]);
            acc[x][y] = fmaf(av[x].y, bv[y].y, acc[x][y]);
            acc[x][y] = fmaf(av[x].z, bv[y].z, acc[x][y]);
            acc[x][y] = fmaf(av[x].w, bv[y].w, acc[x][y]);
          }
      }
#pragma unroll
      for (int x = 0; x < kTa; ++x)
#pragma unroll
        for (int y = 0; y < kTb; ++y) {
          const int ai = ta + x * NTA, bi = tb + y * NTB;
          if (ai < nd && bi < ns) consume(ai, bi, acc[x][y]);
        }
    }
  };

  // r = sum of the dropped rows; the cached G = <x_D, x_S> on the matrix cores:
  // 16 x 16 tiles, each operand split into three bf16 terms (the six products
  // above 2^-24 relative are summed in fp32). Wave w takes a contiguous run of
  // the (S tile, D tile) pairs, S tile major, and rebuilds the S operand only
  // when its S tile changes.
  {
    float sacc = 0.f;
    for (int x = w; x < nd; x += kSelWaves) sacc += cs[x * kCs + lane];
    part[w][lane] = sacc;
  }
  if (CACHE) {
    const int NTD = (nd + 15) >> 4, NTS = (ns + 15) >> 4, np = NTD * NTS;
    const int p0 = w * np / kSelWaves, p1 = (w + 1) * np / kSelWaves;
    const int r16 = lane & 15, g4 = lane >> 4;
    int cur = -1;
    bf16x8 bh[2], bm[2], bl[2];
    for (int p = p0; p < p1; ++p) {
      const int tb = p / NTD, ta = p - tb * NTD;
      if (tb != cur) {
        cur = tb;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          sel_frag(cs + nd * kCs, 16 * tb + r16, ns, ks, lane, bh[ks], bm[ks], bl[ks]);
      }
      bf16x8 ah[2], am[2], al[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) sel_frag(cs, 16 * ta + r16, nd, ks, lane, ah[ks], am[ks], al[ks]);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[ks], bh[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[ks], bl[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am[ks], bm[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am[ks], bh[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[ks], bm[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[ks], bh[ks], acc, 0, 0, 0);
      }
      // lane l holds rows 4 (l / 16) + x of the D tile, column l % 16 of the S tile
      const int bi = 16 * tb + r16;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int ai = 16 * ta + 4 * g4 + x;
        if (ai < nd && bi < ns) G[ai * ns + bi] = acc[x];
      }
    }
  }
  __syncthreads();
  if (t < 64) {
    float sacc = 0.f;
#pragma unroll
    for (int q = 0; q < kSelWaves; ++q) sacc += part[q][t];
    rv[t] = renorm ? fmaf(1.f - ztot, ob[t], sacc) : sacc;
  }
  __syncthreads();

  // g = <r, x> and the slot weights |x|^2 - 2 g (D) or |x|^2 + 2 g (S). With
  // the cached G, later rounds update g in place: after restoring a and
  // dropping b, r' = r - x_a + x_b, so g'_j = g_j - <x_a, x_j> + <x_b, x_j>,
  // every term of which is an old entry of G or a product of the refresh.
  auto weights = [&]() {
    for (int sl = t; sl < nsl; sl += kSelThreads) {
      const float g = dot64(rv, cs + sl * kCs);
      gs[sl] = g;
      slot[sl].wgt = sl < nd ? fmaf(-2.f, g, slot[sl].cc) : fmaf(2.f, g, slot[sl].cc);
    }
  };
  weights();
  __syncthreads();

  float rr = 0.f;
  for (int round = 0;; ++round) {
    rr = wave_allsum(rv[lane] * rv[lane]);
    if (round == a.rounds) break;
    if (!CACHE && round > 0) {
      weights();
      __syncthreads();
    }

    // candidates ordered by (delta, a, b) as one 64-bit key
    unsigned long long best = ~0ull;
    if (CACHE) {
      // thread t takes S slot bi = t % ns and D slots ai = t / ns + m * (512 / ns)
      const int per = kSelThreads / max(ns, 1);
      if (ns > 0 && t < per * ns) {
        const int bi = t % ns;
        const SlotRec sb = slot[nd + bi];
        const uint32_t blo = (uint32_t)sb.blk;
#pragma unroll 4
        for (int ai = t / ns; ai < nd; ai += per) {
          const SlotRec sa = slot[ai];
          const float dlt = (sa.wgt + sb.wgt) - 2.f * G[ai * ns + bi];
          const float crit = renorm ? renorm_j2(rr, dlt, z_s + sa.z - sb.z) : dlt;
          const unsigned long long key = ((unsigned long long)orderable(crit) << 32) |
                                         ((uint32_t)sa.blk << 16) | blo;
          best = key < best ? key : best;
        }
      }
    } else {
      tiles([&](int ai, int bi, float v) {
        const SlotRec sa = slot[ai], sb = slot[nd + bi];
        const float dlt = (sa.wgt + sb.wgt) - 2.f * v;
        const float crit = renorm ? renorm_j2(rr, dlt, z_s + sa.z - sb.z) : dlt;
        const unsigned long long key = ((unsigned long long)orderable(crit) << 32) |
                                       ((uint32_t)sa.blk << 16) | (uint32_t)sb.blk;
        best = key < best ? key : best;
      });
    }
    best = wave_allmin_u64(best);
    if (lane == 0) bkey[w] = best;
    __syncthreads();
    best = bkey[0];
#pragma unroll
    for (int q = 1; q < kSelWaves; ++q) best = bkey[q] < best ? bkey[q] : best;
    const uint32_t hi = (uint32_t)(best >> 32);
    bool improves;
    if (renorm) {
      // criteria are >= 0, whose orderable keys are the float bits with the sign bit set
      const float jb = __uint_as_float(hi & 0x7FFFFFFFu);
      improves = best != ~0ull && hi >= 0x80000000u && jb < rr / (z_s * z_s);
    } else {
      // delta < 0 (strictly) exactly when its orderable key is below that of -0
      improves = best != ~0ull && hi < 0x7FFFFFFFu;
    }
    const uint32_t bab = (uint32_t)best;
    const bool do_swap = nd > 0 && ns > 0 && improves;
    const int ba = (int)(bab >> 16), bb = (int)(bab & 0xFFFFu);
    if (t == 0 && a.swap_log) {
      int32_t* lg = a.swap_log + ((size_t)r * a.rounds + round) * 2;
      lg[0] = do_swap ? ba : -1;
      lg[1] = do_swap ? bb : -1;
    }
    if (!do_swap) {
      if (a.swap_log)
        for (int q = round + 1 + t; q < a.rounds; q += kSelThreads) {
          a.swap_log[((size_t)r * a.rounds + q) * 2] = -1;
          a.swap_log[((size_t)r * a.rounds + q) * 2 + 1] = -1;
        }
      break;   // r and rr describe the final drop set
    }
    // Restore ba (D slot pa) and drop bb (S slot sb): wave 0 exchanges the two
    // slots' rows, records and g, and updates r by -x_a + x_b. No other wave
    // reads slot_of, the rows or the records until the barrier below; after it
    // ba sits in slot sb and bb in slot pa.
    if (w == 0) {
      const int pa = slot_of[ba], sb = slot_of[bb];
      const float ra = cs[pa * kCs + lane], rb = cs[sb * kCs + lane];
      rv[lane] = (rv[lane] - ra) + rb;
      cs[pa * kCs + lane] = rb;
      cs[sb * kCs + lane] = ra;
      if (lane == 0) {
        const SlotRec x = slot[pa];
        slot[pa] = slot[sb];
        slot[sb] = x;
        const float gx = gs[pa];
        gs[pa] = gs[sb];
        gs[sb] = gx;
        slot_of[ba] = sb;
        slot_of[bb] = pa;
      }
    }
    __syncthreads();
    const int pa = slot_of[bb], sbs = slot_of[ba], pb = sbs - nd;
    if (renorm) z_s += slot[sbs].z - slot[pa].z;
    if (CACHE && round + 1 < a.rounds) {
      // refresh row pa (now x_b) and column pb (now x_a) of G, and every g
      // (not after the last round, whose products nothing reads)
      for (int x = t; x < ns + nd; x += kSelThreads) {
        if (x < ns) {
          const int sl = nd + x;
          const float nw = dot64(cs + pa * kCs, cs + sl * kCs);   // <x_b, x_s>
          const float old = G[pa * ns + x];                       // <x_a, x_s>
          G[pa * ns + x] = nw;
          float g = gs[sl];
          g = x == pb ? (g - slot[sl].cc) + old : (g - old) + nw;
          gs[sl] = g;
          slot[sl].wgt = fmaf(2.f, g, slot[sl].cc);
        } else {
          const int y = x - ns;
          float g = gs[y];
          if (y == pa) {
            const float ab = dot64(cs + pa * kCs, cs + sbs * kCs);  // <x_b, x_a>
            g = (g - ab) + slot[y].cc;
          } else {
            const float nw = dot64(cs + y * kCs, cs + sbs * kCs);   // <x_y, x_a>
            const float old = G[y * ns + pb];                       // <x_y, x_b>
            G[y * ns + pb] = nw;
            g = (g - nw) + old;
          }
          gs[y] = g;
          slot[y].wgt = fmaf(-2.f, g, slot[y].cc);
        }
      }
      __syncthreads();
    }
  }
  if (t == 0 && a.row_stat) a.row_stat[r] = renorm ? sqrtf(rr) / z_s : sqrtf(rr);

  const long long base = (long long)b * a.hb.per_batch + a.hb.head_off[h] + (long long)i * k;
  if (t == 0) {
    a.row_ptr[r] = (int32_t)base;
    if (r == d.rows - 1) a.row_ptr[d.rows] = (int32_t)(base + k);
  }
  // kept blocks in ascending order: a block is kept iff it sits in an S slot or is forced
  {
    const bool f = t < nb && (slot_of[t] >= nd || slot_of[t] < 0);
    const unsigned long long m = __ballot(f);
    __syncthreads();
    if (lane == 0) bks[w] = __popcll(m);
    __syncthreads();
    int before = 0;
    for (int q = 0; q < w; ++q) before += bks[q];
    if (f) a.col_idx[base + before + lanes_below(m)] = t;
  }
}

// ---------------------------------------------------------------------------
// Best-swap drift selection for rows wider than the LDS row cache holds
// (more than 512 blocks). Same rule and swap machinery as k_select_drift; the
// row of x stays in global memory (L2) and is gathered by block, LDS holds the
// per-slot records, g, the block priorities and, when it fits, G over D x S.
// The initial top k comes from an MSB-first search for the k-th largest 32-bit
// priority (one block-wide count per bit) with ties at it taken lowest block
// first. Pair products run on the matrix cores as in k_select_drift; without
// the cached G every round recomputes them and g.
// ---------------------------------------------------------------------------
constexpr int kWideThreads = 256;
constexpr int kWideWaves = kWideThreads / 64;

struct DriftWideLds {
  size_t slot, gs, hk, slot_of, zb, G, total;
};

__host__ __device__ inline DriftWideLds drift_wide_lds(int nb, int nslots, size_t gfloats) {
  DriftWideLds L;
  size_t o = 0;
  L.slot = o;    o += (size_t)nslots * 16;       // per slot: |x|^2, weight, block, mass
  L.gs = o;      o += (size_t)nslots * 4;        // per slot: g = <r, x>
  L.hk = o;      o += (size_t)nb * 4;            // 32-bit priority of each block
  L.slot_of = o; o += (size_t)nb * 4;            // slot of each block (-1: forced)
  L.zb = o;      o += (size_t)nb * 4;            // normalised block mass (renorm)
  o = (o + 15) & ~(size_t)15;
  L.G = o;       o += gfloats * 4;               // G[D slot][S slot]
  L.total = o;
  return L;
}

// The swap rows of one selection row, read from global memory by block:
// x_j = c_j (dropped-sum drift) or z_j o - c_j (renormalised objective, o and
// z in LDS).
struct XRow {
  const float* crow;   // contributions of the row, [nb, 64]
  const float* zb;     // renorm: z_j
  const float* ob;     // renorm: o
  bool renorm;

  __device__ __forceinline__ float4 x4(int j, int c4) const {
    const float4 v = reinterpret_cast<const float4*>(crow + (size_t)j * 64)[c4];
    if (!renorm) return v;
    const float z = zb[j];
    const float4 o = reinterpret_cast<const float4*>(ob)[c4];
    return make_float4(z * o.x - v.x, z * o.y - v.y, z * o.z - v.z, z * o.w - v.w);
  }
  __device__ __forceinline__ float x1(int j, int c) const {
    const float v = crow[(size_t)j * 64 + c];
    return renorm ? zb[j] * ob[c] - v : v;
  }
  // <x_j, y> for y in LDS (four 16-byte loads in flight at a time)
  __device__ __forceinline__ float dot(int j, const float* y) const {
    const float4* y4 = reinterpret_cast<const float4*>(y);
    float s0 = 0.f, s1 = 0.f;
#pragma unroll 1
    for (int c = 0; c < 16; c += 4) {
      const float4 a0 = x4(j, c), a1 = x4(j, c + 1), a2 = x4(j, c + 2), a3 = x4(j, c + 3);
      const float4 b0 = y4[c], b1 = y4[c + 1], b2 = y4[c + 2], b3 = y4[c + 3];
      s0 = fmaf(a0.x, b0.x, s0); s0 = fmaf(a0.y, b0.y, s0);
      s0 = fmaf(a0.z, b0.z, s0); s0 = fmaf(a0.w, b0.w, s0);
      s1 = fmaf(a1.x, b1.x, s1); s1 = fmaf(a1.y, b1.y, s1);
      s1 = fmaf(a1.z, b1.z, s1); s1 = fmaf(a1.w, b1.w, s1);
      s0 = fmaf(a2.x, b2.x, s0); s0 = fmaf(a2.y, b2.y, s0);
      s0 = fmaf(a2.z, b2.z, s0); s0 = fmaf(a2.w, b2.w, s0);
      s1 = fmaf(a3.x, b3.x, s1); s1 = fmaf(a3.y, b3.y, s1);
      s1 = fmaf(a3.z, b3.z, s1); s1 = fmaf(a3.w, b3.w, s1);
    }
    return s0 + s1;
  }
  // Head dims 32 ks + 8 (lane / 16) .. +7 of x_j, split in three bf16 terms:
  // one operand fragment of v_mfma_f32_16x16x32_bf16 (lane l gives row or
  // column l % 16); zeros when j < 0.
  __device__ __forceinline__ void frag(int j, int ks, int lane, bf16x8& h, bf16x8& m,
                                       bf16x8& l) const {
    float x[8];
    if (j >= 0) {
      const int c4 = 8 * ks + 2 * (lane >> 4);
      const float4 u = x4(j, c4), v = x4(j, c4 + 1);
      x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
      x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.f;
    }
    sel_split3(x, h, m, l);
  }
};

template <bool CACHE>
__global__ __launch_bounds__(kWideThreads, 4) void k_select_drift_wide(DriftSelArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char dsm[];
  const Dims& d = a.d;
  const int nb = d.nb;
  const int r = blockIdx.x;
  const int bh = r / nb, i = r - bh * nb;
  const int h = bh % d.H, b = bh / d.H;
  const int k = a.hb.keep[h];
  const int nd = nb - k, ns = k - (a.force ? d.F : 0), nsl = nd + ns;
  const DriftWideLds L = drift_wide_lds(nb, nsl, CACHE ? (size_t)nd * ns : 0);
  SlotRec* slot = reinterpret_cast<SlotRec*>(dsm + L.slot);
  float* gs = reinterpret_cast<float*>(dsm + L.gs);
  uint32_t* hk = reinterpret_cast<uint32_t*>(dsm + L.hk);
  int* slot_of = reinterpret_cast<int*>(dsm + L.slot_of);
  float* zb = reinterpret_cast<float*>(dsm + L.zb);
  float* G = reinterpret_cast<float*>(dsm + L.G);
  const bool renorm = a.renorm != 0;
  __shared__ __attribute__((aligned(16))) float rv[64];
  __shared__ __attribute__((aligned(16))) float ob[64];
  __shared__ __attribute__((aligned(16))) float xa[64];
  __shared__ __attribute__((aligned(16))) float xb[64];
  __shared__ __attribute__((aligned(16))) float part[kWideWaves][64];
  __shared__ float redz[kWideWaves];
  __shared__ int cnt[2][3][kWideWaves];
  __shared__ unsigned long long bkey[kWideWaves];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const float* crow = a.contrib + ((size_t)bh * nb + i) * (size_t)nb * 64;
  const XRow X{crow, zb, ob, renorm};
  int pass = 0;   // alternates the count buffers between barriers

  // Squared norms and priorities: thread t takes chunk t % 16 of blocks
  // (t + 256 m) / 16 (coalesced); the 16 lanes of a block reduce by exchange.
  // Renormalised objective: also o = sum_j c_j and the masses z_j.
  {
    float4 oacc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int x = t; x < nb * 16; x += kWideThreads) {
      const float4 v = reinterpret_cast<const float4*>(crow)[x];
      float ss = v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
      ss += __shfl_xor(ss, 8, 64);
      ss += __shfl_xor(ss, 4, 64);
      ss += __shfl_xor(ss, 2, 64);
      ss += __shfl_xor(ss, 1, 64);
      const int j = x >> 4;
      if ((x & 15) == 0) {
        hk[j] = (a.force && block_forced(d, j)) ? 0xFFFFFFFFu : orderable(sqrtf(ss));
        slot_of[j] = __float_as_int(ss);   // the norm, until slots are known
      }
      oacc.x += v.x; oacc.y += v.y; oacc.z += v.z; oacc.w += v.w;
    }
    if (renorm) {
#pragma unroll
      for (int o = 16; o <= 32; o <<= 1) {
        oacc.x += __shfl_xor(oacc.x, o, 64); oacc.y += __shfl_xor(oacc.y, o, 64);
        oacc.z += __shfl_xor(oacc.z, o, 64); oacc.w += __shfl_xor(oacc.w, o, 64);
      }
      if (lane < 16) *reinterpret_cast<float4*>(&part[w][4 * lane]) = oacc;
      float zt = 0.f;
      for (int j = t; j < nb; j += kWideThreads) {
        const float zj = a.zmass[((size_t)bh * nb + i) * nb + j];
        zb[j] = zj;
        zt += zj;
      }
      zt = wave_sum(zt);
      if (lane == 0) redz[w] = zt;
    }
  }
  __syncthreads();
  float ztot = 0.f;
  if (renorm) {
    if (t < 64) {
      float sacc = 0.f;
#pragma unroll
      for (int q = 0; q < kWideWaves; ++q) sacc += part[q][t];
      ob[t] = sacc;
    }
#pragma unroll
    for (int q = 0; q < kWideWaves; ++q) ztot += redz[q];
  }

  // T: the largest priority with #{hk >= T} >= k
  uint32_t T = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    int c = 0;
    for (int j0 = 64 * w; j0 < nb; j0 += kWideThreads) {
      const int j = j0 + lane;
      c += __popcll(__ballot(j < nb && hk[j] >= cand));
    }
    if (lane == 0) cnt[pass & 1][0][w] = c;
    __syncthreads();
    int total = 0;
#pragma unroll
    for (int q = 0; q < kWideWaves; ++q) total += cnt[pass & 1][0][q];
    ++pass;
    if (total >= k) T = cand;
  }
  // kept: priority above T, or at T among the lowest blocks; slots: dropped
  // blocks ascending, then kept non-forced blocks ascending (256 blocks per
  // step, one barrier each)
  {
    int need = k, bd = 0, bs = 0;
    {
      int c = 0;
      for (int j0 = 64 * w; j0 < nb; j0 += kWideThreads) {
        const int j = j0 + lane;
        c += __popcll(__ballot(j < nb && hk[j] > T));
      }
      if (lane == 0) cnt[pass & 1][0][w] = c;
      __syncthreads();
#pragma unroll
      for (int q = 0; q < kWideWaves; ++q) need -= cnt[pass & 1][0][q];
      ++pass;
    }
    for (int base = 0; base < nb; base += kWideThreads) {
      const int j = base + 64 * w + lane;
      const bool real = j < nb;
      const uint32_t pj = real ? hk[j] : 0u;
      const bool tie = real && pj == T;
      const unsigned long long tm = __ballot(tie);
      // ties before this lane, block order: waves below, then lanes below
      if (lane == 0) cnt[pass & 1][0][w] = __popcll(tm);
      __syncthreads();
      int tb = 0, tall = 0;
#pragma unroll
      for (int q = 0; q < kWideWaves; ++q) {
        const int c = cnt[pass & 1][0][q];
        tb += q < w ? c : 0;
        tall += c;
      }
      ++pass;
      const bool kept = real && (pj > T || (tie && tb + lanes_below(tm) < need));
      const bool forced = real && a.force && block_forced(d, j);
      const bool isd = real && !kept, iss = kept && !forced;
      const unsigned long long md = __ballot(isd), ms = __ballot(iss);
      if (lane == 0) {
        cnt[pass & 1][1][w] = __popcll(md);
        cnt[pass & 1][2][w] = __popcll(ms);
      }
      __syncthreads();
      int db = 0, sb = 0, dall = 0, sall = 0;
#pragma unroll
      for (int q = 0; q < kWideWaves; ++q) {
        const int cd = cnt[pass & 1][1][q], cs2 = cnt[pass & 1][2][q];
        db += q < w ? cd : 0;
        sb += q < w ? cs2 : 0;
        dall += cd;
        sall += cs2;
      }
      ++pass;
      if (real) {
        const int sl = isd ? bd + db + lanes_below(md) : (iss ? nd + bs + sb + lanes_below(ms) : -1);
        const float cc = __int_as_float(slot_of[j]);
        slot_of[j] = sl;
        if (sl >= 0) slot[sl] = SlotRec{cc, 0.f, j, renorm ? zb[j] : 0.f};
      }
      need -= min(need, tall);
      bd += dall;
      bs += sall;
    }
  }
  __syncthreads();

  float z_s = 0.f;   // renorm: mass of the kept set
  if (renorm) {
    // |x_j|^2 of the swap rows, and the dropped mass
    float zd = 0.f;
    for (int sl = t; sl < nsl; sl += kWideThreads) {
      const int j = slot[sl].blk;
      float c2 = 0.f;
#pragma unroll 4
      for (int c = 0; c < 16; ++c) {
        const float4 x = X.x4(j, c);
        c2 = fmaf(x.x, x.x, c2); c2 = fmaf(x.y, x.y, c2);
        c2 = fmaf(x.z, x.z, c2); c2 = fmaf(x.w, x.w, c2);
      }
      slot[sl].cc = c2;
      if (sl < nd) zd += slot[sl].z;
    }
    zd = wave_sum(zd);
    if (lane == 0) redz[w] = zd;
    __syncthreads();
    zd = 0.f;
#pragma unroll
    for (int q = 0; q < kWideWaves; ++q) zd += redz[q];
    z_s = ztot - zd;
  }

  // D x S products on the matrix cores (16 x 16 x 32 tiles, operands split in
  // three bf16 terms); wave w takes a contiguous run of the (S tile, D tile)
  // pairs, S tile major, and reloads the S operand only when its tile changes.
  const int NTD = (nd + 15) >> 4, NTS = (ns + 15) >> 4, npairs = NTD * NTS;
  auto gram = [&](auto&& consume) {
    const int p0 = w * npairs / kWideWaves, p1 = (w + 1) * npairs / kWideWaves;
    const int r16 = lane & 15, g4 = lane >> 4;
    int cur = -1;
    bf16x8 bh[2], bm[2], bl[2];
    for (int p = p0; p < p1; ++p) {
      const int tb = p / NTD, ta = p - tb * NTD;
      if (tb != cur) {
        cur = tb;
        const int sb = 16 * tb + r16;
        const int jb = sb < ns ? slot[nd + sb].blk : -1;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) X.frag(jb, ks, lane, bh[ks], bm[ks], bl[ks]);
      }
      bf16x8 ah[2], am[2], al[2];
      const int sa = 16 * ta + r16;
      const int ja = sa < nd ? slot[sa].blk : -1;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) X.frag(ja, ks, lane, ah[ks], am[ks], al[ks]);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[ks], bh[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[ks], bl[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am[ks], bm[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am[ks], bh[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[ks], bm[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[ks], bh[ks], acc, 0, 0, 0);
      }
      // lane l holds D rows 4 (l / 16) + x of the tile, S column l % 16
      const int bi = 16 * tb + r16;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int ai = 16 * ta + 4 * g4 + x;
        if (ai < nd && bi < ns) consume(ai, bi, acc[x]);
      }
    }
  };

  // r = sum of the dropped rows (wave w sums the D slots w, w + 4, ..., one
  // head dim per lane), and the cached G
  {
    float sacc = 0.f;
#pragma unroll 4
    for (int sl = w; sl < nd; sl += kWideWaves) sacc += X.x1(slot[sl].blk, lane);
    part[w][lane] = sacc;
  }
  if (CACHE) gram([&](int ai, int bi, float v) { G[ai * ns + bi] = v; });
  __syncthreads();
  if (t < 64) {
    float sacc = 0.f;
#pragma unroll
    for (int q = 0; q < kWideWaves; ++q) sacc += part[q][t];
    rv[t] = renorm ? fmaf(1.f - ztot, ob[t], sacc) : sacc;
  }
  __syncthreads();

  // g = <r, x> and the slot weights |x|^2 - 2 g (D) or |x|^2 + 2 g (S)
  auto weights = [&]() {
    for (int sl = t; sl < nsl; sl += kWideThreads) {
      const float g = X.dot(slot[sl].blk, rv);
      gs[sl] = g;
      slot[sl].wgt = sl < nd ? fmaf(-2.f, g, slot[sl].cc) : fmaf(2.f, g, slot[sl].cc);
    }
  };
  weights();
  __syncthreads();

  float rr = 0.f;
  for (int round = 0;; ++round) {
    rr = wave_allsum(rv[lane] * rv[lane]);
    if (round == a.rounds) break;
    if (!CACHE && round > 0) {
      weights();
      __syncthreads();
    }

    // candidates ordered by (criterion, a, b) as one 64-bit key
    unsigned long long best = ~0ull;
    auto offer = [&](int ai, int bi, float gab) {
      const SlotRec sa = slot[ai], sb = slot[nd + bi];
      const float dlt = (sa.wgt + sb.wgt) - 2.f * gab;
      const float crit = renorm ? renorm_j2(rr, dlt, z_s + sa.z - sb.z) : dlt;
      const unsigned long long key = ((unsigned long long)orderable(crit) << 32) |
                                     ((uint32_t)sa.blk << 16) | (uint32_t)sb.blk;
      best = key < best ? key : best;
    };
    if (CACHE) {
      // thread t takes S slot bi = t % ns and D slots ai = t / ns + m * (256 / ns)
      const int per = kWideThreads / max(ns, 1);
      if (ns > 0 && ns <= kWideThreads && t < per * ns) {
        const int bi = t % ns;
#pragma unroll 4
        for (int ai = t / ns; ai < nd; ai += per) offer(ai, bi, G[ai * ns + bi]);
      } else if (ns > kWideThreads) {
        for (int x = t; x < nd * ns; x += kWideThreads) offer(x / ns, x % ns, G[x]);
      }
    } else {
      gram(offer);
    }
    best = wave_allmin_u64(best);
    if (lane == 0) bkey[w] = best;
    __syncthreads();
    best = bkey[0];
#pragma unroll
    for (int q = 1; q < kWideWaves; ++q) best = bkey[q] < best ? bkey[q] : best;
    const uint32_t hi = (uint32_t)(best >> 32);
    bool improves;
    if (renorm) {
      // criteria are >= 0, whose orderable keys are the float bits with the sign bit set
      const float jb = __uint_as_float(hi & 0x7FFFFFFFu);
      improves = best != ~0ull && hi >= 0x80000000u && jb < rr / (z_s * z_s);
    } else {
      // delta < 0 (strictly) exactly when its orderable key is below that of -0
      improves = best != ~0ull && hi < 0x7FFFFFFFu;
    }
    const uint32_t bab = (uint32_t)best;
    const bool do_swap = nd > 0 && ns > 0 && improves;
    const int ba = (int)(bab >> 16), bb = (int)(bab & 0xFFFFu);
    if (t == 0 && a.swap_log) {
      int32_t* lg = a.swap_log + ((size_t)r * a.rounds + round) * 2;
      lg[0] = do_swap ? ba : -1;
      lg[1] = do_swap ? bb : -1;
    }
    if (!do_swap) {
      if (a.swap_log)
        for (int q = round + 1 + t; q < a.rounds; q += kWideThreads) {
          a.swap_log[((size_t)r * a.rounds + q) * 2] = -1;
          a.swap_log[((size_t)r * a.rounds + q) * 2 + 1] = -1;
        }
      break;   // r and rr describe the final drop set
    }
    // Restore ba (D slot pa) and drop bb (S slot sb): wave 0 stages x_a and x_b
    // in LDS, updates r by -x_a + x_b, and exchanges the two slots' records and
    // g. No other wave reads slot_of, the records or rv until the barrier
    // below; after it ba sits in slot sb and bb in slot pa.
    if (w == 0) {
      const int pa = slot_of[ba], sb = slot_of[bb];
      const float va = X.x1(ba, lane), vb = X.x1(bb, lane);
      xa[lane] = va;
      xb[lane] = vb;
      rv[lane] = (rv[lane] - va) + vb;
      if (lane == 0) {
        const SlotRec x = slot[pa];
        slot[pa] = slot[sb];
        slot[sb] = x;
        const float gx = gs[pa];
        gs[pa] = gs[sb];
        gs[sb] = gx;
        slot_of[ba] = sb;
        slot_of[bb] = pa;
      }
    }
    __syncthreads();
    const int pa = slot_of[bb], sbs = slot_of[ba], pb = sbs - nd;
    if (renorm) z_s += slot[sbs].z - slot[pa].z;
    if (CACHE && round + 1 < a.rounds) {
      // refresh row pa (now x_b) and column pb (now x_a) of G, and every g
      // (not after the last round, whose products nothing reads)
      for (int x = t; x < ns + nd; x += kWideThreads) {
        if (x < ns) {
          const int sl = nd + x;
          const float nw = X.dot(slot[sl].blk, xb);   // <x_b, x_s>
          const float old = G[pa * ns + x];           // <x_a, x_s>
          G[pa * ns + x] = nw;
          float g = gs[sl];
          g = x == pb ? (g - slot[sl].cc) + old : (g - old) + nw;
          gs[sl] = g;
          slot[sl].wgt = fmaf(2.f, g, slot[sl].cc);
        } else {
          const int y = x - ns;
          float g = gs[y];
          if (y == pa) {
            const float ab = dot64(xb, xa);            // <x_b, x_a>
            g = (g - ab) + slot[y].cc;
          } else {
            const float nw = X.dot(slot[y].blk, xa);   // <x_y, x_a>
            const float old = G[y * ns + pb];          // <x_y, x_b>
            G[y * ns + pb] = nw;
            g = (g - nw) + old;
          }
          gs[y] = g;
          slot[y].wgt = fmaf(-2.f, g, slot[y].cc);
        }
      }
      __syncthreads();
    }
  }
  if (t == 0 && a.row_stat) a.row_stat[r] = renorm ? sqrtf(rr) / z_s : sqrtf(rr);

  const long long base0 = (long long)b * a.hb.per_batch + a.hb.head_off[h] + (long long)i * k;
  if (t == 0) {
    a.row_ptr[r] = (int32_t)base0;
    if (r == d.rows - 1) a.row_ptr[d.rows] = (int32_t)(base0 + k);
  }
  // kept blocks in ascending order: a block is kept iff it sits in an S slot or
  // is forced; 256 blocks per step
  int off = 0;
  for (int base = 0; base < nb; base += kWideThreads) {
    const int j = base + 64 * w + lane;
    const bool f = j < nb && (slot_of[j] >= nd || slot_of[j] < 0);
    const unsigned long long m = __ballot(f);
    if (lane == 0) cnt[pass & 1][0][w] = __popcll(m);
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int q = 0; q < kWideWaves; ++q) {
      const int c = cnt[pass & 1][0][q];
      before += q < w ? c : 0;
      all += c;
    }
    ++pass;
    if (f) a.col_idx[base0 + off + before + lanes_below(m)] = j;
    off += all;
  }
}

hipError_t launch_select_drift(const Dims& d, const HeadBudget& hb, int force, int rounds,
                               int objective, const float* contrib, const float* zmass,
                               int32_t* row_ptr, int32_t* col_idx, float* row_stat,
                               int32_t* swap_log, hipStream_t s) {
  DriftSelArgs a{d, hb, force, rounds, objective, contrib, zmass, row_ptr, col_idx, row_stat,
                 swap_log};
  const int nforced = force ? d.F : 0;
  size_t gmax = 0;
  int smax = 0;
  for (int h = 0; h < d.H; ++h) {
    gmax = std::max(gmax, (size_t)(d.nb - hb.keep[h]) * (size_t)(hb.keep[h] - nforced));
    smax = std::max(smax, d.nb - nforced);
  }
  if (d.nb > kDriftLdsRowBlocks) {
    // wide rows: the row stays in L2; G is cached when it fits in 64 KB
    const size_t lds_cache = drift_wide_lds(d.nb, smax, gmax).total;
    const bool cache = rounds > 0 && lds_cache <= 64 * 1024;
    const size_t lds = cache ? lds_cache : drift_wide_lds(d.nb, smax, 0).total;
    if (lds > kDriftSelLdsCap) return hipErrorInvalidValue;
    const void* fn = cache ? (const void*)k_select_drift_wide<true> : (const void*)k_select_drift_wide<false>;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(HIP_KERNEL_NAME(reinterpret_cast<void (*)(DriftSelArgs)>(const_cast<void*>(fn))),
                       dim3(d.rows), dim3(kWideThreads), lds, s, a);
    return hipGetLastError();
  }
  const size_t lds_cache = drift_sel_lds(d.nb, smax, gmax).total;
  const bool cache = rounds > 0 && lds_cache <= kDriftSelLdsCap;
  const size_t lds = cache ? lds_cache : drift_sel_lds(d.nb, smax, 0).total;
  const bool small = d.nb * 16 <= 8 * kSelThreads;
  const void* fn = cache ? (small ? (const void*)k_select_drift<true, 8> : (const void*)k_select_drift<true, 16>)
                         : (small ? (const void*)k_select_drift<false, 8> : (const void*)k_select_drift<false, 16>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(HIP_KERNEL_NAME(reinterpret_cast<void (*)(DriftSelArgs)>(const_cast<void*>(fn))),
                     dim3(d.rows), dim3(kSelThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace bsgm

namespace bsgm {

// ---------------------------------------------------------------------------
// Drift selection by re-rank rounds, dropped-sum objective ([ReSS] abstract
// and Fig. 3(c): the drop set is refined as a whole; Fig. 3(b): the initial
// set is the top drift scores; Table S3: keeping the best set seen). A round
// scores every block j against the residual of the current drop set D,
// r = sum_{D} c_j:
//   g_j = ||r_j + c_j||^2 - ||r_j||^2 = 2 <r, c_j> -/+ ||c_j||^2
// (minus when j is in D, since then r_j = r - c_j; plus otherwise), and keeps
// the forced blocks plus the top g (ties: lower block), all blocks at once.
// The initial set is the same rule with r = 0. With track-best the result is
// the set of least J = ||r|| among the initial set and every round's set
// (ties: the earlier), else the last one.
//
// One workgroup of 256 threads per row. Lane group g (16 lanes, a float4 of the
// 64-float contribution each) takes blocks g, g + 16, ...; the row is read from
// global memory (L2) once per pass. Kept sets are bitmasks in LDS.
// ---------------------------------------------------------------------------
constexpr int kRrThreads = 256;

__host__ __device__ inline size_t align_up16(size_t x) { return (x + 15) & ~(size_t)15; }

struct DriftRerankArgs {
  Dims d;
  HeadBudget hb;
  int force;
  int rounds;
  int track_best;
  const float* contrib;
  int32_t* row_ptr;
  int32_t* col_idx;
  float* row_stat;
  int32_t* set_log;   // [rows, rounds + 1, ceil(nb / 32)] or null
};

// The rank keys of the top-k search exist for rows of up to 512 blocks only.
__host__ __device__ inline size_t rank_key_bytes(int nb) { return nb <= 512 ? (size_t)nb * 8 : 0; }

__host__ __device__ inline size_t rerank_lds_bytes(int nb) {
  const size_t words = (size_t)(nb + 63) / 64 * 2;   // whole 64-block ballots
  return align_up16((size_t)nb * 4) * 2 + rank_key_bytes(nb) + 2 * words * 4;
}

// cur := the forced blocks plus the top k of score (ties: lower block), for one
// row per workgroup of kRrThreads threads (all of them call it; it ends with a
// barrier). Rows of up to 512 blocks count each block's rank against every
// key (keys: nb entries of LDS); wider rows find the k-th largest 32-bit
// priority T by an MSB-first search (one block-wide count per bit), then keep
// every block above T and the lowest blocks at T. cur: whole 64-block ballots
// of LDS; cnt: LDS scratch of the block-wide counts.
__device__ void rr_select(const Dims& d, int force, int k, const float* score,
                          unsigned long long* keys, uint32_t* cur, int (*cnt)[kRrThreads / 64]) {
  const int nb = d.nb, WP = (nb + 63) / 64 * 2;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  auto hikey = [&](int j) -> uint32_t {
    return (force && block_forced(d, j)) ? 0xFFFFFFFFu : orderable(score[j]);
  };
  int pass = 0;
  // number of blocks whose priority is at least cand (every thread; one barrier)
  auto count_ge = [&](uint32_t cand) {
    int c = 0;
    for (int j0 = 64 * w; j0 < nb; j0 += kRrThreads) {
      const int j = j0 + lane;
      c += __popcll(__ballot(j < nb && hikey(j) >= cand));
    }
    if (lane == 0) cnt[pass & 1][w] = c;
    __syncthreads();
    int total = 0;
#pragma unroll
    for (int q = 0; q < kRrThreads / 64; ++q) total += cnt[pass & 1][q];
    ++pass;
    return total;
  };
  if (nb <= 512) {
    for (int j = t; j < nb; j += kRrThreads) {
      const bool f = force && block_forced(d, j);
      const unsigned long long hi = f ? 0xFFFFFFFFull : (unsigned long long)orderable(score[j]);
      keys[j] = (hi << 32) | (unsigned long long)(~(uint32_t)j);
    }
    __syncthreads();
    for (int j0 = 64 * w; j0 < WP * 32; j0 += kRrThreads) {
      const int j = j0 + lane;
      bool in = false;
      if (j < nb) {
        const unsigned long long kj = keys[j];
        int rank = 0;
        for (int q = 0; q < nb; ++q) rank += keys[q] > kj ? 1 : 0;
        in = rank < k;
      }
      const unsigned long long m = __ballot(in);
      if (lane == 0) {
        cur[j0 >> 5] = (uint32_t)m;
        cur[(j0 >> 5) + 1] = (uint32_t)(m >> 32);
      }
    }
    __syncthreads();
    return;
  }
  uint32_t T = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    if (count_ge(cand) >= k) T = cand;
  }
  int need = k - (T == 0xFFFFFFFFu ? 0 : count_ge(T + 1u));
  for (int base = 0; base < nb; base += kRrThreads) {
    const int j0 = base + 64 * w, j = j0 + lane;
    const uint32_t hk = j < nb ? hikey(j) : 0u;
    const bool tie = j < nb && hk == T;
    const unsigned long long tm = __ballot(tie);
    if (lane == 0) cnt[pass & 1][w] = __popcll(tm);
    __syncthreads();
    int before = 0, ties = 0;
#pragma unroll
    for (int q = 0; q < kRrThreads / 64; ++q) {
      const int c = cnt[pass & 1][q];
      before += q < w ? c : 0;
      ties += c;
    }
    ++pass;
    const bool in = j < nb && (hk > T || (tie && before + lanes_below(tm) < need));
    const unsigned long long m = __ballot(in);
    if (lane == 0 && j0 < WP * 32) {
      cur[j0 >> 5] = (uint32_t)m;
      cur[(j0 >> 5) + 1] = (uint32_t)(m >> 32);
    }
    need -= min(need, ties);
  }
  __syncthreads();
}

// Row r's CSR entry (closed form: every row of head h keeps keep[h] blocks)
// and its kept blocks in ascending order, from the kept flags `out`; one wave
// walks the words 64 at a time.
__device__ void rr_emit(const Dims& d, const HeadBudget& hb, int r, const uint32_t* out,
                        int32_t* row_ptr, int32_t* col_idx, int lane) {
  const int nb = d.nb, W = (nb + 31) >> 5;
  const int bh = r / nb, i = r - bh * nb;
  const int h = bh % d.H, b = bh / d.H;
  const int k = hb.keep[h];
  const long long base = (long long)b * hb.per_batch + hb.head_off[h] + (long long)i * k;
  if (lane == 0) {
    row_ptr[r] = (int32_t)base;
    if (r == d.rows - 1) row_ptr[d.rows] = (int32_t)(base + k);
  }
  int off = 0;
  for (int x0 = 0; x0 < W; x0 += 64) {
    const int x = x0 + lane;
    const uint32_t m = x < W ? out[x] : 0u;
    const int n = __popc(m);
    int incl = n;   // inclusive scan of the counts over the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    int pos = off + incl - n;
    for (uint32_t mm = m; mm; mm &= mm - 1) col_idx[base + pos++] = 32 * x + __ffs(mm) - 1;
    off += __shfl(incl, 63, 64);
  }
}

__global__ __launch_bounds__(kRrThreads) void k_select_drift_rerank(DriftRerankArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char rsm[];
  const Dims& d = a.d;
  const int nb = d.nb, W = (nb + 31) >> 5, WP = (nb + 63) / 64 * 2;
  const int r = blockIdx.x;
  const int bh = r / nb, i = r - bh * nb;
  const int k = a.hb.keep[bh % d.H];
  float* cc = reinterpret_cast<float*>(rsm);                                   // ||c_j||^2
  float* g = reinterpret_cast<float*>(rsm + align_up16((size_t)nb * 4));      // scores
  unsigned long long* keys =
      reinterpret_cast<unsigned long long*>(rsm + 2 * align_up16((size_t)nb * 4));
  uint32_t* cur = reinterpret_cast<uint32_t*>(reinterpret_cast<unsigned char*>(keys) +
                                              rank_key_bytes(nb));   // kept flags, WP words
  uint32_t* best = cur + WP;
  __shared__ __attribute__((aligned(16))) float rv[64];
  __shared__ __attribute__((aligned(16))) float tot[64];
  __shared__ __attribute__((aligned(16))) float part[kRrThreads / 64][64];
  __shared__ float red[kRrThreads / 64];
  __shared__ int cnt[2][kRrThreads / 64];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, grp = t >> 4, c4 = t & 15;
  const float4* row =
      reinterpret_cast<const float4*>(a.contrib + ((size_t)bh * nb + i) * (size_t)nb * 64);
  auto kept = [&](const uint32_t* m, int j) { return ((m[j >> 5] >> (j & 31)) & 1u) != 0; };
  auto sum16 = [&](float s) {
    s += __shfl_xor(s, 8, 64);
    s += __shfl_xor(s, 4, 64);
    s += __shfl_xor(s, 2, 64);
    s += __shfl_xor(s, 1, 64);
    return s;
  };

  // squared norms, and the total o = sum_j c_j of the row
  {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = grp; j < nb; j += kRrThreads / 16) {
      const float4 x = row[(size_t)j * 16 + c4];
      const float s = sum16(x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w);
      if (c4 == 0) cc[j] = s;
      acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
    }
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      acc.x += __shfl_xor(acc.x, o, 64); acc.y += __shfl_xor(acc.y, o, 64);
      acc.z += __shfl_xor(acc.z, o, 64); acc.w += __shfl_xor(acc.w, o, 64);
    }
    if (lane < 16) *reinterpret_cast<float4*>(&part[w][4 * lane]) = acc;
    __syncthreads();
    if (t < 64) {
      float sacc = 0.f;
#pragma unroll
      for (int q = 0; q < kRrThreads / 64; ++q) sacc += part[q][t];
      tot[t] = sacc;
    }
  }
  __syncthreads();

  // rv := r, the sum of the dropped contributions; returns ||r||^2 (every thread).
  // When fewer blocks are kept than dropped, r = o - (sum of the kept rows), which
  // reads the smaller set.
  const bool via_kept = k < nb - k;
  auto residual = [&]() {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = grp; j < nb; j += kRrThreads / 16)
      if (kept(cur, j) == via_kept) {
        const float4 x = row[(size_t)j * 16 + c4];
        acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
      }
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      acc.x += __shfl_xor(acc.x, o, 64); acc.y += __shfl_xor(acc.y, o, 64);
      acc.z += __shfl_xor(acc.z, o, 64); acc.w += __shfl_xor(acc.w, o, 64);
    }
    if (lane < 16) *reinterpret_cast<float4*>(&part[w][4 * lane]) = acc;
    __syncthreads();
    if (t < 64) {
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < kRrThreads / 64; ++q) s += part[q][t];
      if (via_kept) s = tot[t] - s;
      rv[t] = s;
      s = wave_sum(s * s);
      if (t == 0) red[0] = s;
    }
    __syncthreads();
    return red[0];
  };
  auto log_set = [&](int round) {
    if (a.set_log)
      for (int x = t; x < W; x += kRrThreads)
        a.set_log[((size_t)r * (a.rounds + 1) + round) * W + x] = (int32_t)cur[x];
  };

  rr_select(d, a.force, k, cc, keys, cur, cnt);
  float rr = residual();
  log_set(0);
  float best_rr = rr;
  for (int x = t; x < WP; x += kRrThreads) best[x] = cur[x];
  for (int round = 1; round <= a.rounds; ++round) {
    const float4 r4 = reinterpret_cast<const float4*>(rv)[c4];
    for (int j = grp; j < nb; j += kRrThreads / 16) {
      const float4 x = row[(size_t)j * 16 + c4];
      const float s = sum16(x.x * r4.x + x.y * r4.y + x.z * r4.z + x.w * r4.w);
      if (c4 == 0) g[j] = 2.f * s + (kept(cur, j) ? cc[j] : -cc[j]);
    }
    __syncthreads();
    rr_select(d, a.force, k, g, keys, cur, cnt);
    rr = residual();
    log_set(round);
    if (rr < best_rr) {   // uniform: every thread holds the same rr and best_rr
      best_rr = rr;
      for (int x = t; x < WP; x += kRrThreads) best[x] = cur[x];
    }
  }
  __syncthreads();
  const uint32_t* out = a.track_best ? best : cur;
  if (t == 0 && a.row_stat) a.row_stat[r] = sqrtf(a.track_best ? best_rr : rr);
  if (w == 0) rr_emit(d, a.hb, r, out, a.row_ptr, a.col_idx, lane);
}

size_t drift_rerank_lds(int nb) { return rerank_lds_bytes(nb); }

hipError_t launch_select_drift_rerank(const Dims& d, const HeadBudget& hb, int force, int rounds,
                                      int track_best, const float* contrib, int32_t* row_ptr,
                                      int32_t* col_idx, float* row_stat, int32_t* set_log,
                                      hipStream_t s) {
  DriftRerankArgs a{d, hb, force, rounds, track_best, contrib, row_ptr, col_idx, row_stat,
                    set_log};
  const size_t lds = rerank_lds_bytes(d.nb);
  hipError_t e = hipFuncSetAttribute((const void*)k_select_drift_rerank,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_select_drift_rerank, dim3(d.rows), dim3(kRrThreads), lds, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Re-rank rounds in the expanded form (no contributions kept): the same rule
// as k_select_drift_rerank, with the scores assembled from per-(row, block)
// scalars that the round kernels recompute, g_j = 2 <r, c_j> -/+ ||c_j||^2.
// One workgroup per row selects the round's set into a global bitmask (rows
// wider than 2 048 blocks; k_drift_stream_step_wave below takes the others).
// ---------------------------------------------------------------------------
struct DriftStepArgs {
  Dims d;
  HeadBudget hb;
  int force;
  int rounds;
  const float* sqnorm;    // [rows, nb]: ||c_ij||^2
  const float* dot;       // [rows, nb]: <r_i, c_ij> for the previous set (round > 0)
  const uint32_t* prev;   // [rows, W]: the previous set (round > 0)
  uint32_t* next;         // [rows, W]: this round's set
  int32_t* set_log;       // [rows, rounds + 1, W] or null
};

__host__ __device__ inline size_t step_lds_bytes(int nb) {
  return align_up16((size_t)nb * 4) + rank_key_bytes(nb) + (size_t)(nb + 63) / 64 * 2 * 4;
}

size_t drift_stream_step_lds(int nb) { return step_lds_bytes(nb); }

__global__ __launch_bounds__(kRrThreads) void k_drift_stream_step(DriftStepArgs a, int round) {
  extern __shared__ __attribute__((aligned(16))) unsigned char ssm[];
  const Dims& d = a.d;
  const int nb = d.nb, W = (nb + 31) >> 5;
  const int r = blockIdx.x, t = threadIdx.x;
  const int k = a.hb.keep[(r / nb) % d.H];
  float* g = reinterpret_cast<float*>(ssm);
  unsigned long long* keys = reinterpret_cast<unsigned long long*>(ssm + align_up16((size_t)nb * 4));
  uint32_t* cur = reinterpret_cast<uint32_t*>(reinterpret_cast<unsigned char*>(keys) +
                                              rank_key_bytes(nb));
  __shared__ int cnt[2][kRrThreads / 64];
  const float* nr = a.sqnorm + (size_t)r * nb;
  if (round == 0) {
    for (int j = t; j < nb; j += kRrThreads) g[j] = nr[j];
  } else {
    const float* dt = a.dot + (size_t)r * nb;
    const uint32_t* pv = a.prev + (size_t)r * W;
    for (int j = t; j < nb; j += kRrThreads) {
      const bool in = ((pv[j >> 5] >> (j & 31)) & 1u) != 0;
      g[j] = 2.f * dt[j] + (in ? nr[j] : -nr[j]);
    }
  }
  __syncthreads();
  rr_select(d, a.force, k, g, keys, cur, cnt);
  for (int x = t; x < W; x += kRrThreads) {
    a.next[(size_t)r * W + x] = cur[x];
    if (a.set_log) a.set_log[((size_t)r * (a.rounds + 1) + round) * W + x] = (int32_t)cur[x];
  }
}

// The same step with one wave per row, for rows of up to 64 P blocks: block
// 64 p + lane's priority sits in register p of its lane, and the MSB-first
// search and the tie pass of rr_select count across the wave (lane counts and
// one wave sum per step; ballots for the ties), so no barrier is needed. It selects the same set (forced blocks first, then the highest
// g, ties to the lower block).
template <int P>
__global__ __launch_bounds__(256) void k_drift_stream_step_wave(DriftStepArgs a, int round) {
  const Dims& d = a.d;
  const int nb = d.nb, W = (nb + 31) >> 5;
  const int r = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  if (r >= d.rows) return;   // wave-uniform
  const int k = a.hb.keep[(r / nb) % d.H];
  const float* nr = a.sqnorm + (size_t)r * nb;
  const float* dt = round > 0 ? a.dot + (size_t)r * nb : nullptr;
  const uint32_t* pv = round > 0 ? a.prev + (size_t)r * W : nullptr;
  // every load unconditional (slots past the row reread its last block), so
  // that all of them are in flight at once
  float g[P];
#pragma unroll
  for (int p = 0; p < P; ++p) g[p] = nr[min(64 * p + lane, nb - 1)];
  if (round > 0) {
    float dv[P];
    uint32_t pw[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int j = min(64 * p + lane, nb - 1);
      dv[p] = dt[j];
      pw[p] = pv[j >> 5];
    }
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int j = 64 * p + lane;
      const bool in = ((pw[p] >> (j & 31)) & 1u) != 0;
      g[p] = 2.f * dv[p] + (in ? g[p] : -g[p]);
    }
  }
  uint32_t key[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int j = 64 * p + lane;
    key[p] = j >= nb ? 0u : (a.force && block_forced(d, j)) ? 0xFFFFFFFFu : orderable(g[p]);
  }
  // blocks whose priority is at least cand: a count per lane, then one wave
  // sum (exact in fp32 for up to 2^24 blocks)
  auto count_ge = [&](uint32_t cand) {
    float c = 0.f;
#pragma unroll
    for (int p = 0; p < P; ++p) c += (64 * p + lane < nb && key[p] >= cand) ? 1.f : 0.f;
    return (int)wave_allsum(c);
  };
  uint32_t T = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    if (count_ge(cand) >= k) T = cand;
  }
  int need = k - (T == 0xFFFFFFFFu ? 0 : count_ge(T + 1u));
  uint32_t* nx = a.next + (size_t)r * W;
  int32_t* lg = a.set_log ? a.set_log + ((size_t)r * (a.rounds + 1) + round) * W : nullptr;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    if (64 * p >= nb) break;   // uniform
    const bool valid = 64 * p + lane < nb;
    const bool tie = valid && key[p] == T;
    const unsigned long long tm = __ballot(tie);
    const bool in = valid && (key[p] > T || (tie && lanes_below(tm) < need));
    const unsigned long long m = __ballot(in);
    if (lane < 2 && 2 * p + lane < W) {
      const uint32_t word = lane ? (uint32_t)(m >> 32) : (uint32_t)m;
      nx[2 * p + lane] = word;
      if (lg) lg[2 * p + lane] = (int32_t)word;
    }
    need -= min(need, __popcll(tm));
  }
}

// The CSR of the final sets (one wave per row) and, when asked, J = sqrt(jsq).
struct DriftEmitArgs {
  Dims d;
  HeadBudget hb;
  const uint32_t* kept;   // [rows, W]
  const float* jsq;       // [rows]: J^2 of the kept set
  int32_t* row_ptr;
  int32_t* col_idx;
  float* row_stat;
};

__global__ __launch_bounds__(256) void k_drift_stream_emit(DriftEmitArgs a) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (r >= a.d.rows) return;
  const int W = (a.d.nb + 31) >> 5;
  if (lane == 0 && a.row_stat) a.row_stat[r] = sqrtf(a.jsq[r]);
  rr_emit(a.d, a.hb, r, a.kept + (size_t)r * W, a.row_ptr, a.col_idx, lane);
}

hipError_t launch_drift_stream_step(const Dims& d, const HeadBudget& hb, int force, int rounds,
                                    int round, const float* sqnorm, const float* dot,
                                    const uint32_t* prev, uint32_t* next, int32_t* set_log,
                                    hipStream_t s) {
  DriftStepArgs a{d, hb, force, rounds, sqnorm, dot, prev, next, set_log};
  if (d.nb <= 2048) {
    const dim3 grid((d.rows + 3) / 4);
    if (d.nb <= 256)
      hipLaunchKernelGGL(k_drift_stream_step_wave<4>, grid, dim3(256), 0, s, a, round);
    else if (d.nb <= 512)
      hipLaunchKernelGGL(k_drift_stream_step_wave<8>, grid, dim3(256), 0, s, a, round);
    else if (d.nb <= 1024)
      hipLaunchKernelGGL(k_drift_stream_step_wave<16>, grid, dim3(256), 0, s, a, round);
    else if (d.nb <= 1280)
      hipLaunchKernelGGL(k_drift_stream_step_wave<20>, grid, dim3(256), 0, s, a, round);
    else if (d.nb <= 1536)
      hipLaunchKernelGGL(k_drift_stream_step_wave<24>, grid, dim3(256), 0, s, a, round);
    else
      hipLaunchKernelGGL(k_drift_stream_step_wave<32>, grid, dim3(256), 0, s, a, round);
    return hipGetLastError();
  }
  const size_t lds = step_lds_bytes(d.nb);
  hipError_t e = hipFuncSetAttribute((const void*)k_drift_stream_step,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_drift_stream_step, dim3(d.rows), dim3(kRrThreads), lds, s, a, round);
  return hipGetLastError();
}

hipError_t launch_drift_stream_emit(const Dims& d, const HeadBudget& hb, const uint32_t* kept,
                                    const float* jsq, int32_t* row_ptr, int32_t* col_idx,
                                    float* row_stat, hipStream_t s) {
  DriftEmitArgs a{d, hb, kept, jsq, row_ptr, col_idx, row_stat};
  hipLaunchKernelGGL(k_drift_stream_emit, dim3((d.rows + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace bsgm
