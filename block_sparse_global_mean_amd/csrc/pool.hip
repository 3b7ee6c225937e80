// Block mean pool: the mean of Q (or K) over the real tokens of every block,
// accumulated in fp32. One workgroup per (block, b*h); HBM-bound stream.
#include "device_util.h"

namespace bsgm {

// Up to three tensors pooled by one launch (grid z selects the tensor).
struct PoolSet {
  const void* x[3];
  float* mean[3];
};

template <typename T>
__global__ __launch_bounds__(256) void k_pool(PoolSet ps, Dims d) {
  const T* __restrict__ x = static_cast<const T*>(ps.x[blockIdx.z]);
  float* __restrict__ mean = ps.mean[blockIdx.z];
  constexpr int E = 16 / sizeof(T);       // elements per 16-byte chunk
  constexpr int C = 64 / E;               // chunks per 64-wide row
  constexpr int G = 256 / C;              // row groups
  __shared__ float part[G][65];
  const int j = blockIdx.x;
  const int bh = blockIdx.y;
  const int t = threadIdx.x;
  const int c = t % C, g = t / C;
  const int vlen = block_vlen(d, j);
  const T* base = x + ((size_t)bh * d.N + (size_t)j * d.blk) * 64;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  // all of a thread's rows (at most 128 / G) are loaded before any is summed,
  // so that their loads are in flight together
  constexpr int RMAX = 128 / G;
  uint4 raw[RMAX];
#pragma unroll
  for (int k = 0; k < RMAX; ++k) {
    const int r = g + k * G;
    raw[k] = r < vlen ? *reinterpret_cast<const uint4*>(base + (size_t)r * 64 + c * E)
                      : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int k = 0; k < RMAX; ++k) {
    const T* v = reinterpret_cast<const T*>(&raw[k]);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += (float)v[e];
  }
#pragma unroll
  for (int e = 0; e < E; ++e) part[g][c * E + e] = acc[e];
  __syncthreads();
  if (t < 64) {
    float s = 0.f;
#pragma unroll 8
    for (int q = 0; q < G; ++q) s += part[q][t];
    mean[((size_t)bh * d.nb + j) * 64 + t] = s / (float)vlen;
  }
}

hipError_t launch_pool_n(const Dims& d, int dtype, int n, const void* const* xs,
                        float* const* means, hipStream_t s) {
  PoolSet ps{};
  for (int z = 0; z < n; ++z) {
    ps.x[z] = xs[z];
    ps.mean[z] = means[z];
  }
  dim3 grid(d.nb, d.B * d.H, n);
  if (dtype == 1)
    hipLaunchKernelGGL(k_pool<__bf16>, grid, dim3(256), 0, s, ps, d);
  else
    hipLaunchKernelGGL(k_pool<float>, grid, dim3(256), 0, s, ps, d);
  return hipGetLastError();
}

hipError_t launch_pool(const Dims& d, int dtype, const void* x, float* mean, hipStream_t s) {
  return launch_pool_n(d, dtype, 1, &x, &mean, s);
}

}  // namespace bsgm
