// Block mean pooling as a device routine, shared by the pooling kernel and the
// one-launch pooled selection, and the launch of the latter.
#pragma once
#include "device_util.h"

namespace bsgm {

// Geometry of the pooling workgroup (256 threads) for element type T: each
// thread reads 16-byte chunk c of rows g, g + G, ... of a block.
template <typename T>
struct PoolGeom {
  static constexpr int E = 16 / sizeof(T);   // elements per 16-byte chunk
  static constexpr int C = 64 / E;           // chunks per 64-wide row
  static constexpr int G = 256 / C;          // row groups
  static constexpr int RMAX = 128 / G;       // rows per thread for blocks of up to 128
};

// One block of one tensor to pool: its first token, its real-token count and
// the 64 floats that receive the mean (null: nothing to pool).
template <typename T>
struct PoolUnit {
  const T* src;
  float* dst;
  int vlen;
};

// Means of U <= 4 blocks by a workgroup of 256 threads (t: the thread's index);
// part holds U x G x 65 floats of LDS. Every row of every unit is loaded before
// any is summed, so that the loads are in flight together. Per unit the sum
// runs over rows in order within a thread and over row groups in order across
// threads.
template <typename T, int U>
__device__ __forceinline__ void pool_units(const PoolUnit<T> (&u)[U],
                                           float (*part)[PoolGeom<T>::G][65],
                                           int t = threadIdx.x) {
  static_assert(U >= 1 && U <= 4, "one unit per wave of the 256-thread workgroup");
  using PG = PoolGeom<T>;
  const int c = t % PG::C, g = t / PG::C;
  uint4 raw[U][PG::RMAX];
#pragma unroll
  for (int x = 0; x < U; ++x)
#pragma unroll
    for (int k = 0; k < PG::RMAX; ++k) {
      const int r = g + k * PG::G;
      raw[x][k] = r < u[x].vlen
                      ? *reinterpret_cast<const uint4*>(u[x].src + (size_t)r * 64 + c * PG::E)
                      : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
  for (int x = 0; x < U; ++x) {
    float acc[PG::E];
#pragma unroll
    for (int e = 0; e < PG::E; ++e) acc[e] = 0.f;
#pragma unroll
    for (int k = 0; k < PG::RMAX; ++k) {
      const T* v = reinterpret_cast<const T*>(&raw[x][k]);
#pragma unroll
      for (int e = 0; e < PG::E; ++e) acc[e] += (float)v[e];
    }
#pragma unroll
    for (int e = 0; e < PG::E; ++e) part[x][g][c * PG::E + e] = acc[e];
  }
  __syncthreads();
  // unit x is reduced by wave x, one column per lane
#pragma unroll
  for (int x = 0; x < U; ++x) {
    if ((t >> 6) == x && u[x].dst) {
      const int col = t & 63;
      float s = 0.f;
#pragma unroll 8
      for (int p = 0; p < PG::G; ++p) s += part[x][p][col];
      u[x].dst[col] = s / (float)u[x].vlen;
    }
  }
}

// Pooled top-k selection in one launch (see select.hip). sync: the workspace's
// synchronisation words, zero on entry and left zero on exit.
hipError_t launch_select_fused(const Dims& d, const HeadBudget& hb, int dtype, int force,
                               const void* q, const void* k, float* qbar, float* kbar,
                               int32_t* sync, int32_t* row_ptr, int32_t* col_idx,
                               float* row_stat, float* scores_out, hipStream_t s);

// Synchronisation words of the one-launch selection, one per 128-byte line: an
// unused line, the exit count, the error flag, one pooled-item count per (b, h),
// then one ticket per XCD work queue (at most kFusedMaxQueues).
constexpr int kFusedLine = 32;
constexpr int kFusedMaxQueues = 16;
inline size_t fused_sync_words(const Dims& d) {
  return (size_t)kFusedLine * (3 + (size_t)d.B * d.H + kFusedMaxQueues);
}

}  // namespace bsgm
