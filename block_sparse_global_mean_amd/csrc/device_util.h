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

// All-lane sum and max over a wave on the VALU cross-lane paths (DPP within a
// row of 16, then the gfx950 row and half swaps), without the LDS crossbar.
// Every lane gets bitwise the same result. All 64 lanes must be active.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_allsum(float x) {
  x += dpp_mov<0xB1>(x);    // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);    // quad_perm [2,3,0,1]
  x += dpp_mov<0x141>(x);   // row_half_mirror
  x += dpp_mov<0x140>(x);   // row_mirror
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}
__device__ __forceinline__ float wave_allmax(float x) {
  x = fmaxf(x, dpp_mov<0xB1>(x));
  x = fmaxf(x, dpp_mov<0x4E>(x));
  x = fmaxf(x, dpp_mov<0x141>(x));
  x = fmaxf(x, dpp_mov<0x140>(x));
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

// All-lane bitwise AND and OR over a wave, the same way. All 64 lanes active.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_alland(uint32_t x) {
  x &= dpp_mov_u<0xB1>(x);
  x &= dpp_mov_u<0x4E>(x);
  x &= dpp_mov_u<0x141>(x);
  x &= dpp_mov_u<0x140>(x);
  const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = p[0] & p[1];
  const auto q = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return q[0] & q[1];
}
__device__ __forceinline__ uint32_t wave_allor(uint32_t x) {
  x |= dpp_mov_u<0xB1>(x);
  x |= dpp_mov_u<0x4E>(x);
  x |= dpp_mov_u<0x141>(x);
  x |= dpp_mov_u<0x140>(x);
  const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = p[0] | p[1];
  const auto q = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return q[0] | q[1];
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

// LDS tiles of 64-wide bf16 rows (K or V, 128 bytes per key row): the
// 16-byte chunk index within a row is XOR-swizzled by swz(row).
//
// Chunk swizzle of a 128-byte key row. gfx950 LDS serves 256 bytes per
// cycle: a b128 read is served 16 lanes at a time and a b64 read 32 lanes at a
// time, and rows r and r+1 fall in different 128-byte halves. The K-operand read
// (16 rows, one logical chunk per 16 lanes) needs distinct swizzles among the even
// rows and among the odd rows of each 16-row group; the transposing V read (4
// consecutive rows x 4 chunks per 32 lanes) needs rows r and r+2 to land in
// opposite 4-chunk halves. f(r) = ((r & 2) << 1) | ((r >> 2) & 3) meets both.
__device__ __forceinline__ int swz(int row) { return ((row & 2) << 1) | ((row >> 2) & 3); }

__device__ __forceinline__ bf16x4 lds_read_tr(const unsigned char* p) {
  typedef bf16x4 __attribute__((address_space(3))) * lds_ptr;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_ptr)(p));
}

// Fragments for v_mfma_f32_32x32x16_bf16 on such tiles. Both operands give
// lane l the row or column l % 32 and the k-slots 8 (l / 32) .. +7.
//
// K fragment (operand of S^T = K X^T over head dims 16 ks .. 16 ks + 15): A-row m
// of the 32-key sub-tile t reads key row 32 t + key_perm(m), where
// m = 8a + 4h + j maps to 16 (a / 2) + 8h + 4 (a % 2) + j. Accumulator register x
// of lane l then holds key 16 (x / 8) + 8 (l / 32) + x % 8 of the sub-tile, so the
// 8 registers x = 8e .. 8e + 7 are 8 consecutive keys: exactly the k-slots that a
// lane supplies when the same keys are the contraction index of a second MFMA.
__device__ __forceinline__ int key_perm(int m) {
  return ((m >> 4) << 4) | (((m >> 2) & 1) << 3) | (((m >> 3) & 1) << 2) | (m & 3);
}

__device__ __forceinline__ bf16x8 k_frag(const unsigned char* kb, int t, int ks, int lane) {
  const int row = 32 * t + key_perm(lane & 31);
  return *reinterpret_cast<const bf16x8*>(kb + row * 128 +
                                          (((2 * ks + (lane >> 5)) ^ swz(row)) << 4));
}

// V fragment for a contraction over keys kbase .. kbase + 15: lane l gets head
// dim 32 mt + l % 32 of keys kbase + 8 (l / 32) + s, s = 0..7 (the A operand of
// O^T += V^T P^T, or equally the B operand of O += P V). Two transposing 8-byte
// reads: within each 16-lane group g, lane jj fetches 4 head dims of key row
// 8 (g / 2) + jj / 4 and of the row 4 below it.
__device__ __forceinline__ bf16x8 v_frag(const unsigned char* vb, int kbase, int mt, int lane) {
  const int g16 = lane >> 4, jj = lane & 15;
  const int row_lo = kbase + 8 * (g16 >> 1) + (jj >> 2), row_hi = row_lo + 4;
  const int byte = 64 * mt + 32 * (g16 & 1) + 8 * (jj & 3);
  const int c = byte >> 4, sub = byte & 15;
  const bf16x4 lo = lds_read_tr(vb + row_lo * 128 + ((c ^ swz(row_lo)) << 4) + sub);
  const bf16x4 hi = lds_read_tr(vb + row_hi * 128 + ((c ^ swz(row_hi)) << 4) + sub);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// One 16-byte-per-lane global->LDS copy: lane l's 16 bytes at sbase + voff (sbase a
// wave-uniform 64-bit base in SGPRs, voff the lane's byte offset) land at LDS
// byte address lds + 16*l (lds is wave-uniform; it goes to M0). Issued as an
// instruction the compiler does not see as an LDS write, so that it does not
// wait for the copy before every later LDS read; the tile ring orders it
// instead (wait_dma() and a barrier before the first read of a slot, a barrier
// between the last read of a slot and the copy that refills it).
//
// The compiler does not resolve hazards for instructions inside inline asm, and
// on gfx9-family chips a vector-memory instruction needs 5 wait states after a
// VALU instruction (v_readfirstlane, v_readlane of a spilled SGPR) writes an
// SGPR it reads, and an LDS-DMA load 1 wait state after a scalar write of M0.
// Without them it can read the old register: a stale base gives a wrong or
// unmapped source address. The s_nop 4 inside the asm covers both, whatever
// the compiler schedules in front of it.
__device__ __forceinline__ void dma16(const void* sbase, unsigned voff, unsigned lds) {
  const uint64_t b = reinterpret_cast<uint64_t>(sbase);
  const uint64_t bs = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff),
               "s"(reinterpret_cast<const void*>(bs)), "{m0}"(lds)
               : "memory");
}

// Waits until this wave's global->LDS copies have landed.
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Dispatch order of the per-(b, h, query block) attention grids. Workgroups
// are dispatched to the 8 XCDs round-robin (dispatch index mod 8). The k-th
// workgroup of XCD x takes query block x*c + k % c of head k / c, c = ceil(nb/8):
// all XCDs work on the same head at once, so one head's K and V (not eight) is
// the working set of the shared Infinity Cache, and each XCD sweeps a
// contiguous eighth of that head's query blocks, whose kept lists overlap,
// through its own L2. Returns the row (b*H + h)*nb + i, or -1 for the padding
// indices of a head (i >= nb). The grid has head_sync_grid(d) workgroups.
__device__ __forceinline__ int head_sync_row(int bid, int nb) {
  const int c = (nb + 7) >> 3;
  const int x = bid & 7, k = bid >> 3;
  const int bh = k / c, i = x * c + (k - bh * c);
  return i < nb ? bh * nb + i : -1;
}

inline int head_sync_grid(const Dims& d) { return d.B * d.H * 8 * ((d.nb + 7) / 8); }

}  // namespace bsgm
