// Value-aware selection with cross-layer pair memory ("VASC", sections 4.1-4.3
// and appendix A.1-A.5): the per-(batch, head) steps around the row kernel.
//
// Key blocks 2p and 2p + 1 form pair p; an odd last block is a singleton. Before
// selection, k_vasc_prep computes for every pair the RMS contrast of its two
// pooled value vectors, c_p = sqrt(mean_d (vbar_2p - vbar_2p+1)^2) (0 for the
// singleton), the factor 1 + c_p / cbar that scales the pair's relevance (1 when
// the mean contrast cbar is 0), and the ranking copy of the memory,
// max(0, R_p) / max_p' max(0, R_p'). The row kernel (mode 3 of k_select_pooled)
// then ranks d + copy and writes per row and pair the summed clipped demand d
// and the number of executed children. After selection, k_vasc_update adds the
// mean demand minus the mean execution over all query blocks and the pair's
// children to the raw balance R, which the caller keeps across layers.
#include "device_util.h"

namespace bsgm {

// One workgroup per (b, h).
__global__ __launch_bounds__(256) void k_vasc_prep(Dims d, int npairs, const float* __restrict__ vbar,
                                                   const float* __restrict__ memory,
                                                   float* __restrict__ pair_fac,
                                                   float* __restrict__ mhat) {
  __shared__ float red[4];
  const int bh = blockIdx.x, t = threadIdx.x;
  const float* vb = vbar + (size_t)bh * d.nb * 64;
  float* fac = pair_fac + (size_t)bh * npairs;
  const float* raw = memory + (size_t)bh * npairs;
  float csum = 0.f, top = 0.f;
  for (int p = t; p < npairs; p += 256) {
    float c = 0.f;
    if (2 * p + 1 < d.nb) {
      const float4* x = reinterpret_cast<const float4*>(vb + (size_t)(2 * p) * 64);
      const float4* y = reinterpret_cast<const float4*>(vb + (size_t)(2 * p + 1) * 64);
      float acc = 0.f;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const float4 a = x[q], b = y[q];
        acc = fmaf(a.x - b.x, a.x - b.x, acc);
        acc = fmaf(a.y - b.y, a.y - b.y, acc);
        acc = fmaf(a.z - b.z, a.z - b.z, acc);
        acc = fmaf(a.w - b.w, a.w - b.w, acc);
      }
      c = sqrtf(acc * (1.f / 64.f));
    }
    fac[p] = c;   // the contrast until the mean is known
    csum += c;
    top = fmaxf(top, raw[p]);
  }
  const float cbar = block_sum<256>(csum, red) / (float)npairs;
  top = block_max<256>(top, red);   // the largest deficit, or <= 0 if none
  for (int p = t; p < npairs; p += 256) {
    fac[p] = cbar > 0.f ? 1.f + fac[p] / cbar : 1.f;
    mhat[(size_t)bh * npairs + p] = top > 0.f ? fmaxf(raw[p], 0.f) / top : 0.f;
  }
}

// One workgroup of 16 waves per (b, h) and 64 pairs: wave w sums the rows
// i = w, w + 16, ... of its lane's pair, then wave 0 adds the 16 partial sums
// in wave order (a fixed order: the result does not depend on scheduling).
constexpr int kUpdWaves = 16;
__global__ __launch_bounds__(64 * kUpdWaves) void k_vasc_update(Dims d, int npairs,
                                                              const float* __restrict__ pair_dem,
                                                              const float* __restrict__ pair_exe,
                                                              float* __restrict__ memory) {
  __shared__ float sd[kUpdWaves][64], sx[kUpdWaves][64];
  const int chunks = (npairs + 63) / 64;
  const int bh = blockIdx.x / chunks, p0 = (blockIdx.x - bh * chunks) * 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int p = p0 + lane;
  float dem = 0.f, exe = 0.f;
  if (p < npairs) {
    const size_t base = (size_t)bh * d.nb * npairs + p;
#pragma unroll 4
    for (int i = w; i < d.nb; i += kUpdWaves) {
      dem += pair_dem[base + (size_t)i * npairs];
      exe += pair_exe[base + (size_t)i * npairs];
    }
  }
  sd[w][lane] = dem;
  sx[w][lane] = exe;
  __syncthreads();
  if (w == 0 && p < npairs) {
    float td = 0.f, tx = 0.f;
#pragma unroll
    for (int q = 0; q < kUpdWaves; ++q) {
      td += sd[q][lane];
      tx += sx[q][lane];
    }
    const float n = (float)d.nb * (2 * p + 1 < d.nb ? 2.f : 1.f);
    memory[(size_t)bh * npairs + p] += td / n - tx / n;
  }
}

hipError_t launch_vasc_prep(const Dims& d, int npairs, const float* vbar, const float* memory,
                            float* pair_fac, float* mhat, hipStream_t s) {
  hipLaunchKernelGGL(k_vasc_prep, dim3(d.B * d.H), dim3(256), 0, s, d, npairs, vbar, memory,
                     pair_fac, mhat);
  return hipGetLastError();
}

hipError_t launch_vasc_update(const Dims& d, int npairs, const float* pair_dem,
                              const float* pair_exe, float* memory, hipStream_t s) {
  const int chunks = (npairs + 63) / 64;
  hipLaunchKernelGGL(k_vasc_update, dim3(d.B * d.H * chunks), dim3(64 * kUpdWaves), 0, s, d, npairs,
                     pair_dem, pair_exe, memory);
  return hipGetLastError();
}

}  // namespace bsgm
