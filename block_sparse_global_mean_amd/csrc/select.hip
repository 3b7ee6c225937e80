// Pooled block selection (top-k by pooled score, or cumulative pooled mass
// under a per-head cap) and CSR emission.
//
// One workgroup of 256 threads per (b, h, query block). Keys are made unique
// and totally ordered as 64-bit integers: high word = order-preserving bits of
// the pooled score (forced blocks get all ones), low word = ~j so that equal
// scores rank the lower block index first. The k-th largest key, and the
// smallest prefix reaching the mass threshold, are found exactly by an MSB-first
// bitwise search with block-wide counts, so no sort is needed.
#include "device_util.h"

namespace bsgm {

struct SelArgs {
  Dims d;
  HeadBudget hb;
  int mode;            // 0 TOPK, 1 CDF
  float tau;
  int force;
  const float* qbar;
  const float* kbar;
  int32_t* row_ptr;
  int32_t* col_idx;
  float* row_stat;
  float* scores_out;
  int32_t* counts;     // CDF: kept count per row
  uint32_t* bitmask;   // CDF: kept flags, ceil(nb/32) words per row
};

// Writes the kept flags of one row to col_idx[base...] in ascending block order.
template <int PER>
__device__ __forceinline__ void emit_ascending(const bool (&kept)[PER], int nb, long long base,
                                               int32_t* col_idx, int* wtot) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  long long running = base;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const unsigned long long m = __ballot(kept[p]);
    __syncthreads();
    if (lane == 0) wtot[w] = __popcll(m);
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      before += (q < w) ? wtot[q] : 0;
      total += wtot[q];
    }
    if (kept[p]) col_idx[running + before + lanes_below(m)] = t + 256 * p;
    running += total;
  }
}

template <int PER>
__global__ __launch_bounds__(256) void k_select_pooled(SelArgs a) {
  __shared__ float qs[64];
  __shared__ float redf[4];
  __shared__ int redi[4];
  __shared__ int wtot[4];
  const Dims& d = a.d;
  const int r = blockIdx.x;
  const int bh = r / d.nb, i = r - bh * d.nb;
  const int h = bh % d.H, b = bh / d.H;
  const int t = threadIdx.x;
  if (t < 64) qs[t] = a.qbar[((size_t)bh * d.nb + i) * 64 + t];
  __syncthreads();

  const float* kb = a.kbar + (size_t)bh * d.nb * 64;
  float S[PER], P[PER];
  unsigned long long key[PER];
  bool valid[PER];
  float mx = -INFINITY;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int j = t + 256 * p;
    valid[p] = j < d.nb;
    S[p] = -INFINITY;
    if (valid[p]) {
      const float4* kr = reinterpret_cast<const float4*>(kb + (size_t)j * 64);
      float acc = 0.f;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const float4 kv = kr[q];
        acc = fmaf(qs[4 * q + 0], kv.x, acc);
        acc = fmaf(qs[4 * q + 1], kv.y, acc);
        acc = fmaf(qs[4 * q + 2], kv.z, acc);
        acc = fmaf(qs[4 * q + 3], kv.w, acc);
      }
      S[p] = d.scale * acc;
      mx = fmaxf(mx, S[p]);
    }
  }
  mx = block_max<256>(mx, redf);
  float esum = 0.f;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    P[p] = valid[p] ? expf(S[p] - mx) : 0.f;
    esum += P[p];
  }
  const float inv = 1.f / block_sum<256>(esum, redf);
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    P[p] *= inv;
    const int j = t + 256 * p;
    if (valid[p]) {
      const bool f = a.force && block_forced(d, j);
      const unsigned long long hi = f ? 0xFFFFFFFFull : (unsigned long long)orderable(S[p]);
      key[p] = (hi << 32) | (unsigned long long)(~(uint32_t)j);
      if (a.scores_out) a.scores_out[((size_t)bh * d.nb + i) * d.nb + j] = S[p];
    } else {
      key[p] = 0ull;
    }
  }

  const int nforced = a.force ? d.F : 0;
  int k;
  if (a.mode == 1) {
    // largest key threshold T whose keys >= T hold mass >= tau
    unsigned long long T = 0ull;
    for (int bit = 63; bit >= 0; --bit) {
      const unsigned long long cand = T | (1ull << bit);
      float m = 0.f;
#pragma unroll
      for (int p = 0; p < PER; ++p) m += (valid[p] && key[p] >= cand) ? P[p] : 0.f;
      if (block_sum<256>(m, redf) >= a.tau) T = cand;
    }
    int c = 0;
#pragma unroll
    for (int p = 0; p < PER; ++p) c += (valid[p] && key[p] >= T) ? 1 : 0;
    const int n = block_sum_i<256>(c, redi);
    const int cap = a.hb.keep[h];
    k = n < cap ? n : cap;
    k = k > nforced ? k : nforced;
    k = k > 1 ? k : 1;
  } else {
    k = a.hb.keep[h];
  }
  // k-th largest key (keys are unique)
  unsigned long long T = 0ull;
  for (int bit = 63; bit >= 0; --bit) {
    const unsigned long long cand = T | (1ull << bit);
    int c = 0;
#pragma unroll
    for (int p = 0; p < PER; ++p) c += (valid[p] && key[p] >= cand) ? 1 : 0;
    if (block_sum_i<256>(c, redi) >= k) T = cand;
  }
  bool kept[PER];
  float km = 0.f;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    kept[p] = valid[p] && key[p] >= T;
    km += kept[p] ? P[p] : 0.f;
  }
  km = block_sum<256>(km, redf);
  if (t == 0 && a.row_stat) a.row_stat[r] = km;

  if (a.mode == 1) {
    const int words = (d.nb + 31) >> 5;
    const int lane = t & 63, w = t >> 6;
    if (t == 0) a.counts[r] = k;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const unsigned long long m = __ballot(kept[p]);
      const int w0 = 8 * p + 2 * w;
      if (lane == 0) {
        if (w0 < words) a.bitmask[(size_t)r * words + w0] = (uint32_t)m;
        if (w0 + 1 < words) a.bitmask[(size_t)r * words + w0 + 1] = (uint32_t)(m >> 32);
      }
    }
  } else {
    const long long base = (long long)b * a.hb.per_batch + a.hb.head_off[h] + (long long)i * k;
    if (t == 0) {
      a.row_ptr[r] = (int32_t)base;
      if (r == d.rows - 1) a.row_ptr[d.rows] = (int32_t)(base + k);
    }
    emit_ascending<PER>(kept, d.nb, base, a.col_idx, wtot);
  }
}

// Exclusive scan of per-row counts into row_ptr (one workgroup of 1024).
__global__ __launch_bounds__(1024) void k_scan_counts(const int32_t* __restrict__ counts,
                                                      int32_t* __restrict__ row_ptr, int rows) {
  __shared__ int wsum[16];
  __shared__ int wpre[16];
  __shared__ long long carry;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  if (t == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < rows; base += 1024) {
    const int idx = base + t;
    const int v = idx < rows ? counts[idx] : 0;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    if (t == 0) {
      int s = 0;
      for (int q = 0; q < 16; ++q) {
        wpre[q] = s;
        s += wsum[q];
      }
    }
    __syncthreads();
    if (idx < rows) row_ptr[idx] = (int32_t)(carry + wpre[w] + x - v);
    __syncthreads();
    if (t == 0) carry += wpre[15] + wsum[15];
    __syncthreads();
  }
  if (t == 0) row_ptr[rows] = (int32_t)carry;
}

// CSR emission from kept bitmasks: one wave per row, ascending block order.
__global__ __launch_bounds__(256) void k_emit_bitmask(const uint32_t* __restrict__ bitmask,
                                                      const int32_t* __restrict__ row_ptr,
                                                      int32_t* __restrict__ col_idx, int rows,
                                                      int nb) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int words = (nb + 31) >> 5;
  long long running = row_ptr[r];
  for (int w0 = 0; w0 < words; w0 += 64) {
    const int wi = w0 + lane;
    uint32_t bits = wi < words ? bitmask[(size_t)r * words + wi] : 0u;
    const int c = __popc(bits);
    int x = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    const int total = __shfl(x, 63, 64);
    long long pos = running + x - c;
    while (bits) {
      const int bpos = __ffs(bits) - 1;
      col_idx[pos++] = wi * 32 + bpos;
      bits &= bits - 1;
    }
    running += total;
  }
}

hipError_t launch_select_pooled(const Dims& d, const HeadBudget& hb, int mode, float tau,
                                int force, const float* qbar, const float* kbar,
                                int32_t* row_ptr, int32_t* col_idx, float* row_stat,
                                float* scores_out, int32_t* counts, uint32_t* bitmask,
                                hipStream_t s) {
  SelArgs a{d, hb, mode, tau, force, qbar, kbar, row_ptr, col_idx, row_stat, scores_out,
            counts, bitmask};
  const int per = (d.nb + 255) / 256;
  dim3 grid(d.rows), block(256);
  if (per <= 1) hipLaunchKernelGGL(k_select_pooled<1>, grid, block, 0, s, a);
  else if (per <= 2) hipLaunchKernelGGL(k_select_pooled<2>, grid, block, 0, s, a);
  else if (per <= 4) hipLaunchKernelGGL(k_select_pooled<4>, grid, block, 0, s, a);
  else if (per <= 8) hipLaunchKernelGGL(k_select_pooled<8>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(k_select_pooled<16>, grid, block, 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || mode != 1) return e;
  hipLaunchKernelGGL(k_scan_counts, dim3(1), dim3(1024), 0, s, counts, row_ptr, d.rows);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_emit_bitmask, dim3((d.rows + 3) / 4), dim3(256), 0, s, bitmask, row_ptr,
                     col_idx, d.rows, d.nb);
  return hipGetLastError();
}

}  // namespace bsgm
