// Block mean pool: the mean of Q (or K) over the real tokens of every block,
// accumulated in fp32. One workgroup per (block, b*h); HBM-bound stream.
#include "pooled.h"

namespace bsgm {

// Up to three tensors pooled by one launch (grid z selects the tensor).
struct PoolSet {
  const void* x[3];
  float* mean[3];
};

template <typename T>
__global__ __launch_bounds__(256) void k_pool(PoolSet ps, Dims d) {
  __shared__ float part[1][PoolGeom<T>::G][65];
  const int j = blockIdx.x;
  const int bh = blockIdx.y;
  const PoolUnit<T> u[1] = {{static_cast<const T*>(ps.x[blockIdx.z]) +
                                 ((size_t)bh * d.N + (size_t)j * d.blk) * 64,
                             ps.mean[blockIdx.z] + ((size_t)bh * d.nb + j) * 64,
                             block_vlen(d, j)}};
  pool_units<T, 1>(u, part);
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
