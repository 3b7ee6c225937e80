// Block-sparse attention forward for fp32 tensors (vector ALU path).
//
// One workgroup per (b, h, query block), one thread per query row holding its
// query and output in registers. K and V tiles of each listed key block are
// staged in LDS and read as broadcasts. Online softmax in base 2 with the
// scale folded into the query, over chunks of 16 keys.
#include "device_util.h"

namespace bsgm {

struct AttnF32Args {
  Dims d;
  const float* q;
  const float* k;
  const float* v;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  float* o;
  float* lse;
};

template <int BLK>
__global__ __launch_bounds__(BLK) void k_attn_f32(AttnF32Args a) {
  __shared__ float4 Ks[BLK * 16];
  __shared__ float4 Vs[BLK * 16];
  const Dims& d = a.d;
  const int r = head_sync_row(blockIdx.x, d.nb);
  if (r < 0) return;
  const int bh = r / d.nb, i = r - bh * d.nb;
  const int t = threadIdx.x;
  const size_t hoff = (size_t)bh * d.N * 64;
  const int qrow = i * BLK + t;
  const float c2 = d.scale * 1.4426950408889634f;
  float qv[64], o[64];
  {
    const float4* qp = reinterpret_cast<const float4*>(a.q + hoff + (size_t)qrow * 64);
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const float4 x = qp[c];
      qv[4 * c] = x.x * c2; qv[4 * c + 1] = x.y * c2; qv[4 * c + 2] = x.z * c2; qv[4 * c + 3] = x.w * c2;
    }
  }
#pragma unroll
  for (int c = 0; c < 64; ++c) o[c] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int beg = a.row_ptr[r], end = a.row_ptr[r + 1];
  for (int it = beg; it < end; ++it) {
    const int j = a.col_idx[it];
    const float4* kt = reinterpret_cast<const float4*>(a.k + hoff + (size_t)j * BLK * 64);
    const float4* vt = reinterpret_cast<const float4*>(a.v + hoff + (size_t)j * BLK * 64);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      Ks[t + BLK * s] = kt[t + BLK * s];
      Vs[t + BLK * s] = vt[t + BLK * s];
    }
    __syncthreads();
    const int vlen = block_vlen(d, j);
    for (int u0 = 0; u0 < vlen; u0 += 16) {
      float sc[16];
      float cm = -INFINITY;
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int u = u0 + x;
        float acc = -INFINITY;
        if (u < vlen) {
          acc = 0.f;
#pragma unroll
          for (int c = 0; c < 16; ++c) {
            const float4 kk = Ks[u * 16 + c];
            acc = fmaf(qv[4 * c], kk.x, acc);
            acc = fmaf(qv[4 * c + 1], kk.y, acc);
            acc = fmaf(qv[4 * c + 2], kk.z, acc);
            acc = fmaf(qv[4 * c + 3], kk.w, acc);
          }
        }
        sc[x] = acc;
        cm = fmaxf(cm, acc);
      }
      const float mn = fmaxf(m, cm);
      const float alpha = exp2f(m - mn);
      l *= alpha;
#pragma unroll
      for (int c = 0; c < 64; ++c) o[c] *= alpha;
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int u = u0 + x;
        if (u < vlen) {
          const float p = exp2f(sc[x] - mn);
          l += p;
#pragma unroll
          for (int c = 0; c < 16; ++c) {
            const float4 vv = Vs[u * 16 + c];
            o[4 * c] = fmaf(p, vv.x, o[4 * c]);
            o[4 * c + 1] = fmaf(p, vv.y, o[4 * c + 1]);
            o[4 * c + 2] = fmaf(p, vv.z, o[4 * c + 2]);
            o[4 * c + 3] = fmaf(p, vv.w, o[4 * c + 3]);
          }
        }
      }
      m = mn;
    }
  }
  const bool real_q = (qrow % d.L) < d.Lv;
  const bool any = real_q && l > 0.f;
  const float inv = any ? 1.f / l : 0.f;
  float4* op = reinterpret_cast<float4*>(a.o + hoff + (size_t)qrow * 64);
#pragma unroll
  for (int c = 0; c < 16; ++c)
    op[c] = make_float4(o[4 * c] * inv, o[4 * c + 1] * inv, o[4 * c + 2] * inv, o[4 * c + 3] * inv);
  if (a.lse)
    a.lse[(size_t)bh * d.N + qrow] = any ? (m + log2f(l)) * 0.6931471805599453f : -INFINITY;
}

hipError_t launch_attn_f32(const Dims& d, const void* q, const void* k, const void* v,
                           const int32_t* row_ptr, const int32_t* col_idx, void* o,
                           float* lse, hipStream_t s) {
  AttnF32Args a{d, (const float*)q, (const float*)k, (const float*)v, row_ptr, col_idx,
                (float*)o, lse};
  if (d.blk == 128)
    hipLaunchKernelGGL(k_attn_f32<128>, dim3(head_sync_grid(d)), dim3(128), 0, s, a);
  else
    hipLaunchKernelGGL(k_attn_f32<64>, dim3(head_sync_grid(d)), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace bsgm
