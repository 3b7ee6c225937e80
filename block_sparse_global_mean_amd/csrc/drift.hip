// Drift contributions of every key block to every pooled query block for fp32
// inputs (vector ALU; bf16 inputs take the matrix-core kernels of
// drift_mfma.hip), and the drift selection with swap restoration.
//
// Contributions: for pooled query i and real key token u,
//   e_u = exp(scale <qbar_i, k_u> - M_i),  M_i = max_u scale <qbar_i, k_u>,
//   contrib_ij = sum_{u in j} e_u v_u / Z_i,  Z_i = sum_u e_u,  score_ij = ||contrib_ij||.
// Pass 1 finds (M_i, Z_i) with an online log-sum-exp; pass 2 walks the key
// blocks and writes contrib and score. All arithmetic is fp32.
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
                                                       float* __restrict__ score, Dims d) {
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
    float a0 = 0.f, a1 = 0.f;
    for (int u = 0; u < vlen; ++u) {
      const float e = E[ri][u];
      a0 = fmaf(e, Vs[u][dp], a0);
      a1 = fmaf(e, Vs[u][dp + 1], a1);
    }
    const int ii = i0 + ri;
    float sq = a0 * a0 + a1 * a1;
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) sq += __shfl_xor(sq, o, 64);
    if (ii < d.nb) {
      float2* dst = reinterpret_cast<float2*>(contrib + (((size_t)bh * d.nb + ii) * d.nb + j) * 64 + dp);
      *dst = make_float2(a0, a1);
      if ((t & 31) == 0) score[((size_t)bh * d.nb + ii) * d.nb + j] = sqrtf(sq);
    }
    __syncthreads();
  }
}

hipError_t launch_drift_contrib(const Dims& d, int dtype, const float* qbar, const void* k,
                                const void* v, float* contrib, float* score, hipStream_t s) {
  dim3 grid((d.nb + kDriftRows - 1) / kDriftRows, d.B * d.H);
  if (dtype == 1)
    hipLaunchKernelGGL(k_drift_contrib<__bf16>, grid, dim3(256), 0, s, qbar, (const __bf16*)k,
                       (const __bf16*)v, contrib, score, d);
  else
    hipLaunchKernelGGL(k_drift_contrib<float>, grid, dim3(256), 0, s, qbar, (const float*)k,
                       (const float*)v, contrib, score, d);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Drift selection: one workgroup per row, the row's contributions in LDS.
// ---------------------------------------------------------------------------
struct DriftSelArgs {
  Dims d;
  HeadBudget hb;
  int force;
  int rounds;
  const float* contrib;
  int32_t* row_ptr;
  int32_t* col_idx;
  float* row_stat;
  int32_t* swap_log;
};

constexpr int kCs = 65;   // padded LDS row stride (floats) of a contribution vector

__device__ __forceinline__ bool better(float j2, int a, int b, float bj2, int ba, int bb) {
  return j2 < bj2 || (j2 == bj2 && (a < ba || (a == ba && b < bb)));
}

__global__ __launch_bounds__(256) void k_select_drift(DriftSelArgs a) {
  extern __shared__ float smem[];
  const Dims& d = a.d;
  const int nb = d.nb;
  float* cs = smem;                                  // [nb][kCs]
  float* cc = cs + (size_t)nb * kCs;                 // [nb] squared norms
  int* kept = reinterpret_cast<int*>(cc + nb);       // [nb]
  int* dl = kept + nb;                               // [nb] dropped list
  int* sl = dl + nb;                                 // [nb] kept non-forced list
  __shared__ float rv[64];
  __shared__ float part[4][64];
  __shared__ float redf[4];
  __shared__ int redi[4];
  __shared__ int wtot[4];
  __shared__ float bj2s[4];
  __shared__ int bas[4], bbs[4];
  __shared__ int nd_s, ns_s;

  const int r = blockIdx.x;
  const int bh = r / nb, i = r - bh * nb;
  const int h = bh % d.H, b = bh / d.H;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const float* src = a.contrib + ((size_t)bh * nb + i) * (size_t)nb * 64;
  for (int x = t; x < nb * 64; x += 256) cs[(x >> 6) * kCs + (x & 63)] = src[x];
  __syncthreads();

  // squared norms and keys (nb <= 512: two slots per thread)
  constexpr int PER = kDriftMaxBlocks / 256;
  unsigned long long key[PER];
  bool valid[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int j = t + 256 * p;
    valid[p] = j < nb;
    key[p] = 0ull;
    if (valid[p]) {
      float s = 0.f;
      for (int c = 0; c < 64; ++c) s = fmaf(cs[j * kCs + c], cs[j * kCs + c], s);
      cc[j] = s;
      const bool f = a.force && block_forced(d, j);
      const unsigned long long hi = f ? 0xFFFFFFFFull : (unsigned long long)orderable(sqrtf(s));
      key[p] = (hi << 32) | (unsigned long long)(~(uint32_t)j);
    }
  }
  const int k = a.hb.keep[h];
  unsigned long long T = 0ull;
  for (int bit = 63; bit >= 0; --bit) {
    const unsigned long long cand = T | (1ull << bit);
    int c = 0;
#pragma unroll
    for (int p = 0; p < PER; ++p) c += (valid[p] && key[p] >= cand) ? 1 : 0;
    if (block_sum_i<256>(c, redi) >= k) T = cand;
  }
#pragma unroll
  for (int p = 0; p < PER; ++p)
    if (valid[p]) kept[t + 256 * p] = key[p] >= T ? 1 : 0;
  __syncthreads();

  float rr = 0.f;
  bool stopped = false;
  for (int round = 0; round <= a.rounds; ++round) {
    // residual of the drop set: r = sum over dropped j of contrib_j
    {
      const int dd = t & 63, g = t >> 6;
      float s = 0.f;
      for (int j = g; j < nb; j += 4)
        if (!kept[j]) s += cs[j * kCs + dd];
      part[g][dd] = s;
    }
    __syncthreads();
    if (t < 64) rv[t] = (part[0][t] + part[1][t]) + (part[2][t] + part[3][t]);
    __syncthreads();
    {
      const float x = t < 64 ? rv[t] * rv[t] : 0.f;
      rr = block_sum<256>(x, redf);
    }
    if (round == a.rounds || stopped) break;

    // candidate lists, ascending: dropped blocks (to restore) and kept
    // non-forced blocks (to drop)
    {
      int nd = 0, ns = 0;
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const int j = t + 256 * p;
        const bool isd = valid[p] && !kept[j];
        const bool iss = valid[p] && kept[j] && !(a.force && block_forced(d, j));
        const unsigned long long md = __ballot(isd), ms = __ballot(iss);
        __syncthreads();
        if (lane == 0) wtot[w] = __popcll(md) | (__popcll(ms) << 16);
        __syncthreads();
        int bd = 0, bs = 0, td = 0, ts = 0;
        for (int q = 0; q < 4; ++q) {
          const int vd = wtot[q] & 0xFFFF, vs = wtot[q] >> 16;
          if (q < w) { bd += vd; bs += vs; }
          td += vd; ts += vs;
        }
        if (isd) dl[nd + bd + lanes_below(md)] = j;
        if (iss) sl[ns + bs + lanes_below(ms)] = j;
        nd += td;
        ns += ts;
      }
      if (t == 0) { nd_s = nd; ns_s = ns; }
    }
    __syncthreads();
    const int nd = nd_s, ns = ns_s;
    float best = INFINITY;
    int ba = 0x7FFFFFFF, bb = 0x7FFFFFFF;
    for (int ai = t; ai < nd; ai += 256) {
      const int aa = dl[ai];
      float u[64];
      float uu = 0.f;
#pragma unroll
      for (int c = 0; c < 64; ++c) {
        u[c] = rv[c] - cs[aa * kCs + c];
        uu = fmaf(u[c], u[c], uu);
      }
      for (int bi = 0; bi < ns; ++bi) {
        const int bbk = sl[bi];
        float dot = 0.f;
#pragma unroll
        for (int c = 0; c < 64; ++c) dot = fmaf(u[c], cs[bbk * kCs + c], dot);
        const float j2 = uu + 2.f * dot + cc[bbk];
        if (better(j2, aa, bbk, best, ba, bb)) { best = j2; ba = aa; bb = bbk; }
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ob = __shfl_xor(best, o, 64);
      const int oa = __shfl_xor(ba, o, 64), obb = __shfl_xor(bb, o, 64);
      if (better(ob, oa, obb, best, ba, bb)) { best = ob; ba = oa; bb = obb; }
    }
    if (lane == 0) { bj2s[w] = best; bas[w] = ba; bbs[w] = bb; }
    __syncthreads();
    best = bj2s[0]; ba = bas[0]; bb = bbs[0];
    for (int q = 1; q < 4; ++q)
      if (better(bj2s[q], bas[q], bbs[q], best, ba, bb)) { best = bj2s[q]; ba = bas[q]; bb = bbs[q]; }
    const bool do_swap = nd > 0 && ns > 0 && best < rr;
    if (t == 0 && a.swap_log) {
      int32_t* lg = a.swap_log + ((size_t)r * a.rounds + round) * 2;
      lg[0] = do_swap ? ba : -1;
      lg[1] = do_swap ? bb : -1;
    }
    __syncthreads();
    if (do_swap) {
      if (t == 0) { kept[ba] = 1; kept[bb] = 0; }
    } else {
      stopped = true;
      if (a.swap_log)
        for (int q = round + 1 + t; q < a.rounds; q += 256) {
          a.swap_log[((size_t)r * a.rounds + q) * 2] = -1;
          a.swap_log[((size_t)r * a.rounds + q) * 2 + 1] = -1;
        }
    }
    __syncthreads();
  }
  if (t == 0 && a.row_stat) a.row_stat[r] = sqrtf(rr);

  const long long base = (long long)b * a.hb.per_batch + a.hb.head_off[h] + (long long)i * k;
  if (t == 0) {
    a.row_ptr[r] = (int32_t)base;
    if (r == d.rows - 1) a.row_ptr[d.rows] = (int32_t)(base + k);
  }
  long long running = base;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int j = t + 256 * p;
    const bool f = valid[p] && kept[j];
    const unsigned long long m = __ballot(f);
    __syncthreads();
    if (lane == 0) wtot[w] = __popcll(m);
    __syncthreads();
    int before = 0, total = 0;
    for (int q = 0; q < 4; ++q) {
      before += (q < w) ? wtot[q] : 0;
      total += wtot[q];
    }
    if (f) a.col_idx[running + before + lanes_below(m)] = j;
    running += total;
  }
}

size_t drift_select_lds_bytes(int nb) {
  return (size_t)nb * kCs * sizeof(float) + (size_t)nb * sizeof(float) + 3 * (size_t)nb * sizeof(int);
}

hipError_t launch_select_drift(const Dims& d, const HeadBudget& hb, int force, int rounds,
                               const float* contrib, int32_t* row_ptr, int32_t* col_idx,
                               float* row_stat, int32_t* swap_log, hipStream_t s) {
  DriftSelArgs a{d, hb, force, rounds, contrib, row_ptr, col_idx, row_stat, swap_log};
  const size_t lds = drift_select_lds_bytes(d.nb);
  hipError_t e = hipFuncSetAttribute((const void*)k_select_drift,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_select_drift, dim3(d.rows), dim3(256), lds, s, a);
  return hipGetLastError();
}

}  // namespace bsgm
