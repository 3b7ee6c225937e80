// Device helpers shared by the kernels: vector types, wave/block reductions,
// order-preserving float keys, and the real-token length of a block.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "internal.h"

namespace bsgm {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;

// Real tokens of block j: padding sits at the end of each frame and block
// divides frame_len, so the real tokens are the block's first vlen tokens.
__device__ __forceinline__ int block_vlen(const Dims& d, int j) {
  int off = (j * d.blk) % d.L;
  int v = d.Lv - off;
  return v < 0 ? 0 : (v > d.blk ? d.blk : v);
}

__device__ __forceinline__ bool block_forced(const Dims& d, int j) {
  // block holding token f*L for some frame f (specials first in every frame)
  return ((j * d.blk) % d.L) == 0;
}

// Maps a float to an unsigned integer with the same order (NaN excluded).
__device__ __forceinline__ uint32_t orderable(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Block-wide reductions for NT threads (NT / 64 waves). `red` is LDS scratch
// of at least NT / 64 entries; every thread gets the result. Two barriers.
template <int NT>
__device__ __forceinline__ float block_sum(float x, float* red) {
  x = wave_sum(x);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) t += red[i];
  return t;
}
template <int NT>
__device__ __forceinline__ float block_max(float x, float* red) {
  x = wave_max(x);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  float t = red[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) t = fmaxf(t, red[i]);
  return t;
}
template <int NT>
__device__ __forceinline__ int block_sum_i(int x, int* red) {
  x = wave_sum_i(x);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) t += red[i];
  return t;
}

// Number of lanes below this one whose predicate is set, and the wave total.
__device__ __forceinline__ int lanes_below(unsigned long long mask) {
  const int lane = threadIdx.x & 63;
  unsigned long long below = lane ? (mask & ((~0ull) >> (64 - lane))) : 0ull;
  return __popcll(below);
}

// Maps a dispatch index to a work index so that the workgroups that one XCD
// (dispatch index mod 8) runs take consecutive work items: neighbouring rows
// of one head then share that XCD's L2. Bijective on [0, n).
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int per = n >> 3;
  if (bid >= per * 8) return bid;
  return (bid & 7) * per + (bid >> 3);
}

}  // namespace bsgm
