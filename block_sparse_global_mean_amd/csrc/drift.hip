// Drift contributions of every key block to every pooled query block for fp32
// inputs (vector ALU; bf16 inputs take the matrix-core kernels of
// drift_mfma.hip), and the drift selection with swap restoration.
//
// Contributions: for pooled query i and real key token u,
//   e_u = exp(scale <qbar_i, k_u> - M_i),  M_i = max_u scale <qbar_i, k_u>,
//   contrib_ij = sum_{u in j} e_u v_u / Z_i,  Z_i = sum_u e_u,  score_ij = ||contrib_ij||,
//   zmass_ij = sum_{u in j} e_u / Z_i (optional).
// Pass 1 finds (M_i, Z_i) with an online log-sum-exp; pass 2 walks the key
// blocks and writes contrib and score. All arithmetic is fp32.
#include <algorithm>

#include "device_util.h"

namespace bsgm {

constexpr int kDriftRows = 8;   // pooled query rows per workgroup

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

template <typename T>
__global__ __launch_bounds__(256) void k_drift_contrib(const float* __restrict__ qbar,
                                                       const T* __restrict__ K,
                                                       const T* __restrict__ V,
                                                       float* __restrict__ contrib,
                                                       float* __restrict__ score,
                                                       float* __restrict__ zmass, Dims d) {
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
    float sq = a0 * a0 + a1 * a1;
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) sq += __shfl_xor(sq, o, 64);
    if (ii < d.nb) {
      float2* dst = reinterpret_cast<float2*>(contrib + (((size_t)bh * d.nb + ii) * d.nb + j) * 64 + dp);
      *dst = make_float2(a0, a1);
      if ((t & 31) == 0) score[((size_t)bh * d.nb + ii) * d.nb + j] = sqrtf(sq);
      if ((t & 31) == 0 && zmass) zmass[((size_t)bh * d.nb + ii) * d.nb + j] = zs;
    }
    __syncthreads();
  }
}

hipError_t launch_drift_contrib(const Dims& d, int dtype, const float* qbar, const void* k,
                                const void* v, float* contrib, float* score, float* zmass,
                                hipStream_t s) {
  if (dtype != 0) return hipErrorInvalidValue;   // bf16 takes launch_drift_contrib_bf16
  dim3 grid((d.nb + kDriftRows - 1) / kDriftRows, d.B * d.H);
  hipLaunchKernelGGL(k_drift_contrib<float>, grid, dim3(256), 0, s, qbar, (const float*)k,
                     (const float*)v, contrib, score, zmass, d);
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
// when it fits it is computed once per row into LDS and a swap refreshes one
// row and one column of it; otherwise every round recomputes the dot products.
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
// for rows of up to 256 blocks, 16 up to kDriftMaxBlocks
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
  size_t cs, slot, keys, slot_of, zb, G, total;
};

__host__ __device__ inline DriftSelLds drift_sel_lds(int nb, int nslots, size_t gfloats) {
  DriftSelLds L;
  size_t o = 0;
  L.cs = o;      o += (size_t)nslots * kCs * 4;  // slot rows
  L.slot = o;    o += (size_t)nslots * 16;       // per slot: |c|^2, weight, block, -
  L.keys = o;    o += (size_t)nb * 8;            // priority keys by block
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
  __syncthreads();
  // initial kept set: the k keys of highest priority (keys are distinct)
  bool kept_j = false, forced_j = false;
  float cc_j = 0.f;
  if (t < nb) {
    const unsigned long long kj = keys[t];
    int rank = 0;
#pragma unroll 8
    for (int q = 0; q < nb; ++q) rank += keys[q] > kj ? 1 : 0;
    kept_j = rank < k;
    forced_j = a.force && block_forced(d, t);
    cc_j = __int_as_float(slot_of[t]);
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

  // kTa x kTb tiles of <c_a, c_b>. Tile (ta, tb) takes D slots ta + x NTA and S
  // slots tb + y NTB, so that neighbouring lanes read neighbouring LDS rows.
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

  // r = sum of the dropped contributions; G once per row when cached
  {
    float s = 0.f;
    for (int x = w; x < nd; x += kSelWaves) s += cs[x * kCs + lane];
    part[w][lane] = s;
  }
  if (CACHE) tiles([&](int ai, int bi, float v) { G[ai * ns + bi] = v; });
  __syncthreads();
  if (t < 64) {
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < kSelWaves; ++q) s += part[q][t];
    rv[t] = renorm ? fmaf(1.f - ztot, ob[t], s) : s;
  }
  __syncthreads();

  float rr = 0.f;
  for (int round = 0;; ++round) {
    {
      const float x = rv[lane];
      rr = wave_sum(x * x);
    }
    if (round == a.rounds) break;

    for (int sl = t; sl < nsl; sl += kSelThreads) {
      const float g = dot64(rv, cs + sl * kCs);
      slot[sl].wgt = sl < nd ? slot[sl].cc - 2.f * g : slot[sl].cc + 2.f * g;
    }
    __syncthreads();

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
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const unsigned long long other = __shfl_xor(best, o, 64);
      best = other < best ? other : best;
    }
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
    // restore ba (D slot pa) and drop bb (S slot sb): exchange the slots' rows
    const int pa = slot_of[ba], sb = slot_of[bb], pb = sb - nd;
    if (renorm) z_s += slot[pa].z - slot[sb].z;
    __syncthreads();   // every wave is done with bkey, slot weights and G of this round
    if (t < 64) {
      const float ra = cs[pa * kCs + t], rb = cs[sb * kCs + t];
      rv[t] = (rv[t] - ra) + rb;
      cs[pa * kCs + t] = rb;
      cs[sb * kCs + t] = ra;
    } else if (t == 64) {
      const SlotRec x = slot[pa];
      slot[pa] = slot[sb];
      slot[sb] = x;
      slot_of[ba] = sb;
      slot_of[bb] = pa;
    }
    __syncthreads();
    if (CACHE)
      for (int x = t; x < ns + nd; x += kSelThreads) {
        if (x < ns) G[pa * ns + x] = dot64(cs + pa * kCs, cs + (nd + x) * kCs);
        else if (x - ns != pa) G[(x - ns) * ns + pb] = dot64(cs + (x - ns) * kCs, cs + sb * kCs);
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
