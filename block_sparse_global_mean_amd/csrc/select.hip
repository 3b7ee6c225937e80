// Pooled block selection (top-k by pooled score, or cumulative pooled mass
// under a per-head cap) and CSR emission.
//
// One wave per (b, h, query block); a workgroup of four waves takes four
// consecutive query blocks of one (b, h), so each 64-key tile of pooled K is
// read from memory once per four rows and served to the waves from LDS. Lane l
// owns key blocks l, l + 64, ...; every reduction of a row is wave-local.
// Keys are made unique and totally ordered as 64-bit integers: high word =
// order-preserving bits of the pooled score (forced blocks get all ones), low
// word = ~j so that equal scores rank the lower block index first. The k-th
// largest key, and the smallest prefix reaching the mass threshold, are found
// exactly by an MSB-first bitwise search, so no sort is needed: counts come from
// ballots and masses from cross-lane sums that stay on the VALU.
#include <type_traits>

#include "pooled.h"

namespace bsgm {

struct SelArgs {
  Dims d;
  HeadBudget hb;
  int mode;            // 0 TOPK, 1 CDF, 3 VASC
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
  // VASC: per (b, h) and pair of key blocks, the contrast factor 1 + c / cbar
  // and the ranking copy of the memory; per row and pair, the summed clipped
  // demand and the number of executed children
  int npairs;
  const float* pair_fac;
  const float* mhat;
  float* pair_dem;
  float* pair_exe;
  float* demand_out;   // VASC: [rows, nb] clipped demand, or null
};

constexpr int kSelRowsPerWg = 4;
constexpr int kKtStride = 68;   // LDS row stride (floats) of the pooled-K tile

// The rows of workgroup `wg` of (b, h) = bh: query blocks 4 wg .. 4 wg + 3, one
// per wave. `kt` is 2 x 64 x kKtStride floats of LDS; t is the thread's index
// in the workgroup. No barrier follows the point where a wave without a row
// returns.
template <int PW, bool VASC>   // key blocks per lane: nb <= 64 * PW; VASC: mode 3
__device__ __forceinline__ void select_rows(const SelArgs& a, int bh, int wg,
                                            float (*kt)[64 * kKtStride], int t = threadIdx.x) {
  const Dims& d = a.d;
  const int lane = t & 63, w = t >> 6;
  const int i = wg * kSelRowsPerWg + w;
  const bool live = i < d.nb;
  const int h = bh % d.H, b = bh / d.H;
  const int r = bh * d.nb + i;

  // the pooled query row, in registers (one broadcast load per float4)
  float4 q4[16];
  {
    const float4* qr = reinterpret_cast<const float4*>(a.qbar + ((size_t)bh * d.nb + (live ? i : 0)) * 64);
#pragma unroll
    for (int c = 0; c < 16; ++c) q4[c] = qr[c];
  }

  // pooled scores S_j = scale <qbar_i, kbar_j>, 64 keys per tile; tiles are
  // double-buffered in LDS and the next one is fetched while this one is used
  const float* kb = a.kbar + (size_t)bh * d.nb * 64;
  auto fetch = [&](int p, float4 (&v)[4]) {
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int x = t + 256 * s4;          // float4 index in the tile
      const int j = 64 * p + (x >> 4);
      v[s4] = j < d.nb ? reinterpret_cast<const float4*>(kb + (size_t)j * 64)[x & 15]
                       : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  float4 nxt[4];
  fetch(0, nxt);
  float S[PW];
#pragma unroll
  for (int p = 0; p < PW; ++p) {
    S[p] = -INFINITY;
    if (64 * p >= d.nb) continue;   // uniform across the workgroup
    float* tile = kt[p & 1];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int x = t + 256 * s4;
      *reinterpret_cast<float4*>(&tile[(x >> 4) * kKtStride + 4 * (x & 15)]) = nxt[s4];
    }
    if (64 * (p + 1) < d.nb) fetch(p + 1, nxt);
    __syncthreads();   // tile p written; every wave is past tile p - 1 (the other buffer)
    if (live && 64 * p + lane < d.nb) {
      const float4* kr = reinterpret_cast<const float4*>(&tile[lane * kKtStride]);
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const float4 kv = kr[c];
        acc = fmaf(q4[c].x, kv.x, acc);
        acc = fmaf(q4[c].y, kv.y, acc);
        acc = fmaf(q4[c].z, kv.z, acc);
        acc = fmaf(q4[c].w, kv.w, acc);
      }
      S[p] = d.scale * acc;
    }
  }
  if (!live) return;   // no barrier follows

  float mx = -INFINITY;
#pragma unroll
  for (int p = 0; p < PW; ++p) mx = fmaxf(mx, S[p]);
  mx = wave_allmax(mx);
  float P[PW];
  unsigned long long key[PW];
  float esum = 0.f;
#pragma unroll
  for (int p = 0; p < PW; ++p) {
    const int j = 64 * p + lane;
    P[p] = j < d.nb ? expf(S[p] - mx) : 0.f;
    esum += P[p];
    if (j < d.nb && a.scores_out) a.scores_out[(size_t)r * d.nb + j] = S[p];
  }
  const float inv = 1.f / wave_allsum(esum);
#pragma unroll
  for (int p = 0; p < PW; ++p) P[p] *= inv;

  // ranking value: the pooled score, or for VASC the clipped value-aware
  // demand d = min(1, k a / sum a), a = P (1 + c / cbar), plus the memory copy
  float dem[VASC ? PW : 1];
  if constexpr (VASC) {
    const float* fac = a.pair_fac + (size_t)bh * a.npairs;
    float asum = 0.f;
#pragma unroll
    for (int p = 0; p < PW; ++p) {
      const int j = 64 * p + lane;
      dem[p] = j < d.nb ? P[p] * fac[j >> 1] : 0.f;
      asum += dem[p];
    }
    asum = wave_allsum(asum);
    const float kf = (float)a.hb.keep[h];
    const float* mh = a.mhat + (size_t)bh * a.npairs;
#pragma unroll
    for (int p = 0; p < PW; ++p) {
      const int j = 64 * p + lane;
      dem[p] = j < d.nb ? fminf(1.f, kf * dem[p] / asum) : 0.f;
      S[p] = j < d.nb ? dem[p] + mh[j >> 1] : 0.f;
      if (j < d.nb && a.demand_out) a.demand_out[(size_t)r * d.nb + j] = dem[p];
    }
  }
#pragma unroll
  for (int p = 0; p < PW; ++p) {
    const int j = 64 * p + lane;
    if (j < d.nb) {
      const bool f = a.force && block_forced(d, j);
      const unsigned long long hi = f ? 0xFFFFFFFFull : (unsigned long long)orderable(S[p]);
      key[p] = (hi << 32) | (unsigned long long)(~(uint32_t)j);
    } else {
      key[p] = 0ull;   // sorts below every real key, whose high word is nonzero
    }
  }

  // Both searches below end on a real key, so a bit on which every real key of
  // the row agrees is that key's bit: it starts set in T if it is a one and is
  // never tested. Only the bits that vary (a uniform set) are searched.
  uint32_t and_hi = ~0u, and_lo = ~0u, or_hi = 0u, or_lo = 0u;
#pragma unroll
  for (int p = 0; p < PW; ++p)
    if (64 * p + lane < d.nb) {
      and_hi &= (uint32_t)(key[p] >> 32);
      and_lo &= (uint32_t)key[p];
      or_hi |= (uint32_t)(key[p] >> 32);
      or_lo |= (uint32_t)key[p];
    }
  and_hi = __builtin_amdgcn_readfirstlane(wave_alland(and_hi));
  and_lo = __builtin_amdgcn_readfirstlane(wave_alland(and_lo));
  or_hi = __builtin_amdgcn_readfirstlane(wave_allor(or_hi));
  or_lo = __builtin_amdgcn_readfirstlane(wave_allor(or_lo));
  const unsigned long long common1 = ((unsigned long long)and_hi << 32) | and_lo;
  const unsigned long long vary = common1 ^ (((unsigned long long)or_hi << 32) | or_lo);

  const int nforced = a.force ? d.F : 0;
  int k;
  if (a.mode == 1) {
    // largest key threshold T whose keys >= T hold mass >= tau
    unsigned long long T = common1;
    for (unsigned long long rest = vary; rest != 0ull;) {
      const int bit = 63 - __clzll(rest);
      rest &= ~(1ull << bit);
      const unsigned long long cand = T | (1ull << bit);
      float m = 0.f;
#pragma unroll
      for (int p = 0; p < PW; ++p) m += key[p] >= cand ? P[p] : 0.f;
      if (wave_allsum(m) >= a.tau) T = cand;
    }
    int n = 0;
#pragma unroll
    for (int p = 0; p < PW; ++p) n += __popcll(__ballot(key[p] != 0ull && key[p] >= T));
    const int cap = a.hb.keep[h];
    k = n < cap ? n : cap;
    k = k > nforced ? k : nforced;
    k = k > 1 ? k : 1;
  } else {
    k = a.hb.keep[h];
  }
  // k-th largest key (keys are unique)
  unsigned long long T = common1;
  for (unsigned long long rest = vary; rest != 0ull;) {
    const int bit = 63 - __clzll(rest);
    rest &= ~(1ull << bit);
    const unsigned long long cand = T | (1ull << bit);
    int c = 0;
#pragma unroll
    for (int p = 0; p < PW; ++p) c += __popcll(__ballot(key[p] >= cand));
    if (c >= k) T = cand;
  }
  bool kept[PW];
  float km = 0.f;
#pragma unroll
  for (int p = 0; p < PW; ++p) {
    kept[p] = key[p] != 0ull && key[p] >= T;
    km += kept[p] ? P[p] : 0.f;
  }
  km = wave_allsum(km);
  if (lane == 0 && a.row_stat) a.row_stat[r] = km;

  if constexpr (VASC) {
    // pair p of tile t holds keys 64t + 2p' and 64t + 2p' + 1: lanes l and l ^ 1
#pragma unroll
    for (int p = 0; p < PW; ++p) {
      const float dv = dem[p], xv = kept[p] ? 1.f : 0.f;
      const float ds = dv + dpp_mov<0xB1>(dv), xs = xv + dpp_mov<0xB1>(xv);
      const int pair = 32 * p + (lane >> 1);
      if ((lane & 1) == 0 && pair < a.npairs) {
        a.pair_dem[(size_t)r * a.npairs + pair] = ds;
        a.pair_exe[(size_t)r * a.npairs + pair] = xs;
      }
    }
  }

  if (a.mode == 1) {
    const int words = (d.nb + 31) >> 5;
    if (lane == 0) a.counts[r] = k;
#pragma unroll
    for (int p = 0; p < PW; ++p) {
      const unsigned long long m = __ballot(kept[p]);
      if (lane == 0) {
        if (2 * p < words) a.bitmask[(size_t)r * words + 2 * p] = (uint32_t)m;
        if (2 * p + 1 < words) a.bitmask[(size_t)r * words + 2 * p + 1] = (uint32_t)(m >> 32);
      }
    }
  } else {
    const long long base = (long long)b * a.hb.per_batch + a.hb.head_off[h] + (long long)i * k;
    if (lane == 0) {
      a.row_ptr[r] = (int32_t)base;
      if (r == d.rows - 1) a.row_ptr[d.rows] = (int32_t)(base + k);
    }
    // kept blocks in ascending order: tile p, then lane
    long long running = base;
#pragma unroll
    for (int p = 0; p < PW; ++p) {
      const unsigned long long m = __ballot(kept[p]);
      if (kept[p]) a.col_idx[running + lanes_below(m)] = 64 * p + lane;
      running += __popcll(m);
    }
  }
}

template <int PW, bool VASC>
__global__ __launch_bounds__(256) void k_select_pooled(SelArgs a) {
  __shared__ __attribute__((aligned(16))) float kt[2][64 * kKtStride];
  const int wgs_per_bh = (a.d.nb + kSelRowsPerWg - 1) / kSelRowsPerWg;
  const int bh = blockIdx.x / wgs_per_bh;
  select_rows<PW, VASC>(a, bh, blockIdx.x - bh * wgs_per_bh, kt);
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
                                hipStream_t s, const VascSel* vasc) {
  SelArgs a{d, hb, mode, tau, force, qbar, kbar, row_ptr, col_idx, row_stat, scores_out,
            counts, bitmask, 0, nullptr, nullptr, nullptr, nullptr, nullptr};
  if (vasc) {
    a.npairs = vasc->npairs;
    a.pair_fac = vasc->pair_fac;
    a.mhat = vasc->mhat;
    a.pair_dem = vasc->pair_dem;
    a.pair_exe = vasc->pair_exe;
    a.demand_out = vasc->demand_out;
  }
  const int per = (d.nb + 63) / 64;
  dim3 grid(d.B * d.H * ((d.nb + kSelRowsPerWg - 1) / kSelRowsPerWg)), block(256);
  auto go = [&](auto pw) {
    constexpr int PW = decltype(pw)::value;
    if (mode == 3) hipLaunchKernelGGL((k_select_pooled<PW, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_select_pooled<PW, false>), grid, block, 0, s, a);
  };
  if (per <= 1) go(std::integral_constant<int, 1>{});
  else if (per <= 2) go(std::integral_constant<int, 2>{});
  else if (per <= 4) go(std::integral_constant<int, 4>{});
  else if (per <= 8) go(std::integral_constant<int, 8>{});
  else if (per <= 12) go(std::integral_constant<int, 12>{});
  else if (per <= 16) go(std::integral_constant<int, 16>{});
  else if (per <= 24) go(std::integral_constant<int, 24>{});
  else if (per <= 32) go(std::integral_constant<int, 32>{});
  else if (per <= 48) go(std::integral_constant<int, 48>{});
  else go(std::integral_constant<int, 64>{});
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || mode != 1) return e;
  hipLaunchKernelGGL(k_scan_counts, dim3(1), dim3(1024), 0, s, counts, row_ptr, d.rows);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_emit_bitmask, dim3((d.rows + 3) / 4), dim3(256), 0, s, bitmask, row_ptr,
                     col_idx, d.rows, d.nb);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Pooled top-k selection in one launch: the pooling of Q and K and the
// selection share one grid, and every (b, h) is pooled and selected on one XCD
// (its work queue: (b*H + h) mod the XCD count), so that the selection reads
// the pooled means through that XCD's L2 with no device-wide cache writeback
// or invalidation. The grid is persistent: a workgroup reads the XCD it runs
// on (the XCC_ID hardware register) and takes items from that XCD's queue by
// an atomic ticket until the queue is drained. A queue holds its heads'
// pooling items (item x of a head pools key blocks 4x .. 4x + 3), then their
// selection items (item x pools query blocks 4x .. 4x + 3 and selects those
// rows, as k_select_pooled), so that the query loads of one item overlap the
// selection work of others. A selection item waits until every pooling item of
// its head has published; those hold lower tickets of the same queue, so
// workgroups already running took them, and a pooling item waits on nothing:
// every wait ends. A selection item reads back the pooled queries it wrote
// itself, after its own stores are acknowledged and a barrier.
//
// Publication inside an XCD: a pooling workgroup waits until its stores are
// acknowledged by the L2 (vmcnt 0), then raises the head's count; the L1 is
// write-through and holds no line of that head's means from before (each call
// starts with clean L1s, and a CU reads a head's means only after they are
// complete), so the selecting workgroup's loads see them.
//
// The last workgroup to leave runs, in order, any queue that no workgroup
// took (an XCD with no workgroup of this grid), so the result never depends on
// where the hardware placed the workgroups, and then resets the tickets, the
// item counts and the exit count, so every call finds them zero (the caller
// zeroes them once). Its view of the counters needs no fence: each workgroup's
// last ticket fetch returned before it raised the exit count.
// ---------------------------------------------------------------------------
constexpr int kFusedSpinLimit = 1 << 22;   // waits of about 64 clocks each

// The thread index, opaque to the compiler: the items of the persistent loop
// take it afresh, so that the lane-dependent offsets of the pooling and
// selection code are not hoisted out of the loop and held in registers across
// all items (which took the kernel from about 120 to 226 registers, and from
// four workgroups per CU to two).
__device__ __forceinline__ int opaque_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// Four workgroups per CU (128 registers): the grid assumes them.
template <typename T, int PW>
__global__ __launch_bounds__(256, 4) void k_select_fused(SelArgs a, const T* __restrict__ xq,
                                                       const T* __restrict__ xk, float* qbar,
                                                       float* kbar, int32_t* sync, int nq) {
  constexpr size_t kSelLds = 2 * 64 * kKtStride * sizeof(float);
  constexpr size_t kPoolLds = kSelRowsPerWg * PoolGeom<T>::G * 65 * sizeof(float);
  __shared__ __attribute__((aligned(16))) unsigned char lds[kSelLds > kPoolLds ? kSelLds : kPoolLds];
  __shared__ int s_item, s_last;
  const Dims& d = a.d;
  const int t = threadIdx.x;
  const int nbh = d.B * d.H;
  // per (b, h): pooling items of 4 key blocks, then selection items of 4 rows
  const int kpool_per_bh = (d.nb + kSelRowsPerWg - 1) / kSelRowsPerWg;
  const int sel_per_bh = kpool_per_bh;
  int32_t* exits = sync + kFusedLine;
  int32_t* error = sync + 2 * kFusedLine;
  int32_t* done = sync + 3 * kFusedLine;   // item count of (b, h) = x at done[x * kFusedLine]
  int32_t* tickets = sync + (3 + nbh) * kFusedLine;   // queue x at tickets[x * kFusedLine]

  // runs item `item` of queue `qu`; false once the queue is drained
  auto run = [&](int qu) {
    const int nh = (nbh - qu + nq - 1) / nq;   // heads qu, qu + nq, ...
    const int npool = nh * kpool_per_bh, total = npool + nh * sel_per_bh;
    __syncthreads();   // the previous item is done with the LDS and s_item
    if (t == 0)
      s_item = __hip_atomic_fetch_add(&tickets[qu * kFusedLine], 1, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    // uniform, but read from LDS: say so, so that the item's indices and
    // addresses stay in scalar registers
    const int item = __builtin_amdgcn_readfirstlane(s_item);
    if (item >= total) return false;
    const bool kpool = item < npool;
    const int u = kpool ? item / kpool_per_bh : (item - npool) / sel_per_bh;
    const int x = kpool ? item - u * kpool_per_bh : item - npool - u * sel_per_bh;
    const int bh = qu + nq * u;
    // blocks 4x .. 4x + 3: of K for a pooling item, of Q (the rows it then
    // selects) for a selection item
    PoolUnit<T> pu[kSelRowsPerWg];
#pragma unroll
    for (int y = 0; y < kSelRowsPerWg; ++y) {
      const int j = kSelRowsPerWg * x + y;
      const bool real = j < d.nb;
      const size_t tok = ((size_t)bh * d.N + (size_t)(real ? j : 0) * d.blk) * 64;
      const size_t row = ((size_t)bh * d.nb + j) * 64;
      pu[y] = PoolUnit<T>{(kpool ? xk : xq) + tok, real ? (kpool ? kbar : qbar) + row : nullptr,
                          real ? block_vlen(d, j) : 0};
    }
    pool_units<T, kSelRowsPerWg>(pu, reinterpret_cast<float(*)[PoolGeom<T>::G][65]>(lds),
                                 opaque_tid());
    // every store of this workgroup acknowledged by the L2 before the count,
    // or before the selection reads its pooled queries back
    __builtin_amdgcn_s_waitcnt(0);
    asm volatile("" ::: "memory");
    if (!kpool && t == 0) {
      // the selection needs all of its head's pooled keys
      int spins = 0;
      while (__hip_atomic_load(&done[bh * kFusedLine], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT) < kpool_per_bh) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins == kFusedSpinLimit) {
          __hip_atomic_store(error, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
    }
    __syncthreads();
    if (kpool) {
      if (t == 0)
        __hip_atomic_fetch_add(&done[bh * kFusedLine], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      select_rows<PW, false>(a, bh, x, reinterpret_cast<float(*)[64 * kKtStride]>(lds),
                             opaque_tid());
    }
    return true;
  };

  // XCC_ID (hardware register 20, bits 3:0): the XCD this workgroup runs on
  const int xcc = (int)(__builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 15u);
  if (xcc < nq)
    while (run(xcc)) {
    }
  __syncthreads();
  if (t == 0)
    s_last = __hip_atomic_fetch_add(exits, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             (int)gridDim.x - 1;
  __syncthreads();
  if (s_last) {
    for (int qu = 0; qu < nq; ++qu)
      while (run(qu)) {
      }
    __syncthreads();
    for (int x = t; x < nbh; x += 256)
      __hip_atomic_store(&done[x * kFusedLine], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int x = t; x < kFusedMaxQueues; x += 256)
      __hip_atomic_store(&tickets[x * kFusedLine], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (t == 0) __hip_atomic_store(exits, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

hipError_t launch_select_fused(const Dims& d, const HeadBudget& hb, int dtype, int force,
                               const void* q, const void* k, float* qbar, float* kbar,
                               int32_t* sync, int32_t* row_ptr, int32_t* col_idx,
                               float* row_stat, float* scores_out, hipStream_t s) {
  SelArgs a{d, hb, 0, 0.f, force, qbar, kbar, row_ptr, col_idx, row_stat, scores_out,
            nullptr, nullptr, 0, nullptr, nullptr, nullptr, nullptr, nullptr};
  // one queue per XCD; resident workgroups: four per CU
  int dev = 0, nxcc = 1, ncu = 256;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (hipDeviceGetAttribute(&nxcc, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || nxcc < 1)
    nxcc = 1;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      ncu < 1)
    ncu = 256;
  const int nq = nxcc < kFusedMaxQueues ? nxcc : kFusedMaxQueues;
  const dim3 grid((unsigned)(4 * ncu)), block(256);
  auto go = [&](auto pw) {
    constexpr int PW = decltype(pw)::value;
    if (dtype == 1)
      hipLaunchKernelGGL((k_select_fused<__bf16, PW>), grid, block, 0, s, a,
                         static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), qbar, kbar,
                         sync, nq);
    else
      hipLaunchKernelGGL((k_select_fused<float, PW>), grid, block, 0, s, a,
                         static_cast<const float*>(q), static_cast<const float*>(k), qbar, kbar,
                         sync, nq);
  };
  const int per = (d.nb + 63) / 64;
  if (per <= 1) go(std::integral_constant<int, 1>{});
  else if (per <= 2) go(std::integral_constant<int, 2>{});
  else if (per <= 4) go(std::integral_constant<int, 4>{});
  else if (per <= 8) go(std::integral_constant<int, 8>{});
  else if (per <= 12) go(std::integral_constant<int, 12>{});
  else if (per <= 16) go(std::integral_constant<int, 16>{});
  else if (per <= 24) go(std::integral_constant<int, 24>{});
  else if (per <= 32) go(std::integral_constant<int, 32>{});
  else if (per <= 48) go(std::integral_constant<int, 48>{});
  else go(std::integral_constant<int, 64>{});
  return hipGetLastError();
}

}  // namespace bsgm
