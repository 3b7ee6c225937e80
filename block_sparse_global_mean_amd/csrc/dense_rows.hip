// Dense attention of the camera and register query rows (the first ns tokens
// of every frame) over all real keys of their (b, h), bf16 inputs.
//
// The special rows of one (b, h) are gathered into groups of 128 (gathered row
// g*128 + r is token (gr / ns) * L + gr % ns with gr = g*128 + r); a group is
// one workgroup of four waves, 32 rows each, like a query block of the sparse
// kernel. The keys are split into chunks of consecutive key blocks, one
// workgroup per (b, h, group, chunk), which writes its unnormalised partial
// (O, m, l); a second kernel merges the chunks of every row and writes O and
// LSE. Per key tile the math is the sparse kernel's: S^T = K Q^T and
// O^T += V^T P^T on v_mfma_f32_32x32x16_bf16, online softmax in base 2 with a
// lazy reference maximum.
#include "device_util.h"

namespace bsgm {

struct DenseRowsArgs {
  Dims d;
  int ns;        // special tokens per frame
  int nrows;     // F * ns gathered rows per (b, h)
  int ngroups;   // ceil(nrows / 128)
  int cpc;       // key blocks per chunk
  int nchunks;   // ceil(nb / cpc)
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  float* po;     // [B*H, ngroups, nchunks, 128, 64] partial O (unnormalised)
  float* pml;    // [B*H, ngroups, nchunks, 128, 2] partial (m, l), m in raw score units
  __bf16* o;
  float* lse;
};

template <int BLK>
__global__ __launch_bounds__(256, 2) void k_dense_rows_partial(DenseRowsArgs a) {
  constexpr int NT = 256;
  constexpr int KT = BLK / 32;
  constexpr int TB = BLK * 128;
  constexpr int CPT = (BLK * 8) / NT;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * 2 * TB];

  const Dims& d = a.d;
  const int wg = blockIdx.x;
  const int c = wg % a.nchunks;
  const int tg = wg / a.nchunks;
  const int g = tg % a.ngroups, bh = tg / a.ngroups;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 31, hh = lane >> 5;
  const size_t hoff = (size_t)bh * d.N * 64;
  const __bf16* Q = a.q + hoff;
  const __bf16* K = a.k + hoff;
  const __bf16* V = a.v + hoff;
  const int gr = g * 128 + 32 * w + n;
  const bool row_ok = gr < a.nrows;
  // a wave whose 32 rows are all past the last special row only helps with the
  // tile copies (the last group of a head is usually partly empty)
  const bool wave_live = g * 128 + 32 * w < a.nrows;
  const int tok = (gr / a.ns) * d.L + gr % a.ns;

  bf16x8 qf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (row_ok) {
      qf[ks] = *reinterpret_cast<const bf16x8*>(Q + (size_t)tok * 64 + 16 * ks + 8 * hh);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[ks][e] = (__bf16)0.f;
    }
  }
  // the compiler does not see the asm copies below as vector loads: let it wait
  // for the fragment loads here, once
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) asm volatile("" : "+v"(qf[ks]));

  unsigned voff[CPT];
#pragma unroll
  for (int s2 = 0; s2 < CPT; ++s2) {
    const int q = NT * s2 + tid;
    const int row = q >> 3, pc = q & 7;
    voff[s2] = (unsigned)(row * 64 + ((pc ^ swz(row)) << 3)) * 2u;
  }
  const unsigned lds0 = (unsigned)(uintptr_t)smem + __builtin_amdgcn_readfirstlane(w) * 1024;
#define BSGM_DMA_D(BUF, J)                                                       \
  do {                                                                           \
    const __bf16* kt_ = K + (size_t)(J) * BLK * 64;                              \
    const __bf16* vt_ = V + (size_t)(J) * BLK * 64;                              \
    const unsigned kb_ = lds0 + (BUF) * 2 * TB;                                  \
    _Pragma("unroll") for (int s3 = 0; s3 < CPT; ++s3) {                         \
      dma16(kt_, voff[s3], kb_ + s3 * NT * 16);                                  \
      dma16(vt_, voff[s3], kb_ + TB + s3 * NT * 16);                             \
    }                                                                            \
  } while (0)

  f32x16 oacc[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int x = 0; x < 16; ++x) oacc[mt][x] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = d.scale * 1.4426950408889634f;
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};

  const int j0 = c * a.cpc, j1 = min(d.nb, j0 + a.cpc);
  if (j0 < j1) BSGM_DMA_D(0, j0);
  for (int j = j0; j < j1; ++j) {
    const int buf = (j - j0) & 1;
    wait_dma();
    __syncthreads();
    if (j + 1 < j1) BSGM_DMA_D(buf ^ 1, j + 1);
    if (!wave_live) continue;
    const unsigned char* kb = smem + buf * 2 * TB;
    const unsigned char* vb = kb + TB;

    f32x16 s[KT];
#pragma unroll
    for (int t = 0; t < KT; ++t) {
#pragma unroll
      for (int x = 0; x < 16; ++x) s[t][x] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_frag(kb, t, ks, lane), qf[ks], s[t], 0, 0, 0);
    }
    const int vlen = block_vlen(d, j);
    if (vlen < BLK) {
      asm volatile("" ::: "memory");
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const int key = 32 * t + 16 * (x >> 3) + 8 * hh + (x & 7);
          if (key >= vlen) s[t][x] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
      for (int x = 0; x < 16; ++x) mx = fmaxf(mx, s[t][x]);
    {
      const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                       false, false);
      mx = fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
    }
    const bool grow = (mx - m_run) * c2 > 8.f;
    if (__ballot(grow)) {
      const float m_new = grow ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c2);
      l_run *= alpha;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int x = 0; x < 16; ++x) oacc[mt][x] *= alpha;
      m_run = m_new;
    }
    const float mb = m_run * c2;
    bf16x8 pb[KT][2];
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        float pf[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) pf[x] = __builtin_amdgcn_exp2f(fmaf(s[t][8 * e + x], c2, -mb));
        const bf16x8 pv = {(__bf16)pf[0], (__bf16)pf[1], (__bf16)pf[2], (__bf16)pf[3],
                           (__bf16)pf[4], (__bf16)pf[5], (__bf16)pf[6], (__bf16)pf[7]};
        pb[t][e] = pv;
        psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pv, pv, 0, 1), ones, psum, false);
        psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pv, pv, 2, 3), ones, psum, false);
        psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pv, pv, 4, 5), ones, psum, false);
        psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pv, pv, 6, 7), ones, psum, false);
      }
    {
      const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(psum), __float_as_uint(psum),
                                                       false, false);
      psum = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
    }
    l_run += psum;
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          oacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_frag(vb, 32 * t + 16 * e, mt, lane),
                                                             pb[t][e], oacc[mt], 0, 0, 0);
  }
  wait_dma();
#undef BSGM_DMA_D

  // partial of this chunk: lane holds gathered row 32w + n, head dims
  // 32mt + 8(x/4) + 4hh + x%4
  if (!wave_live) return;
  const size_t prow = (size_t)wg * 128 + 32 * w + n;
  float* po = a.po + prow * 64;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4)
      *reinterpret_cast<float4*>(po + 32 * mt + 8 * a4 + 4 * hh) =
          make_float4(oacc[mt][4 * a4], oacc[mt][4 * a4 + 1], oacc[mt][4 * a4 + 2], oacc[mt][4 * a4 + 3]);
  if (hh == 0) *reinterpret_cast<float2*>(a.pml + prow * 2) = make_float2(m_run, l_run);
}

// One wave per gathered row: merge the chunk partials, write O (bf16) and LSE.
// Lane c takes the (m, l) of chunks c, c + 64, ...; each chunk's weight is then
// broadcast while the lanes (head dims) read the partial O rows eight at a time.
__global__ __launch_bounds__(256) void k_dense_rows_merge(DenseRowsArgs a) {
  const Dims& d = a.d;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int rows_per_bh = a.ngroups * 128;
  const int bh = wid / rows_per_bh, rr = wid - bh * rows_per_bh;
  if (bh >= d.B * d.H || rr >= a.nrows) return;
  const int g = rr >> 7, r = rr & 127;
  const float c2 = d.scale * 1.4426950408889634f;
  const size_t base = ((size_t)(bh * a.ngroups + g) * a.nchunks) * 128 + r;
  const int nc = a.nchunks;
  float m = -INFINITY;
  for (int c = lane; c < nc; c += 64) m = fmaxf(m, a.pml[(base + (size_t)c * 128) * 2]);
  m = wave_max(m);
  float l = 0.f, acc = 0.f;
  for (int c0 = 0; c0 < nc; c0 += 64) {
    float f = 0.f;
    if (c0 + lane < nc) {
      const float2 ml = *reinterpret_cast<const float2*>(a.pml + (base + (size_t)(c0 + lane) * 128) * 2);
      f = ml.y > 0.f ? __builtin_amdgcn_exp2f((ml.x - m) * c2) : 0.f;
      l += ml.y * f;
    }
    const int cn = min(64, nc - c0);
    for (int j0 = 0; j0 < cn; j0 += 8) {
      float pv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        pv[u] = j0 + u < cn ? a.po[(base + (size_t)(c0 + j0 + u) * 128) * 64 + lane] : 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u) acc = fmaf(pv[u], __shfl(f, j0 + u, 64), acc);
    }
  }
  l = wave_sum(l);
  const int tok = (rr / a.ns) * d.L + rr % a.ns;
  const size_t orow = (size_t)bh * d.N + tok;
  a.o[orow * 64 + lane] = (__bf16)(l > 0.f ? acc / l : 0.f);
  if (a.lse && lane == 0) a.lse[orow] = l > 0.f ? m * d.scale + logf(l) : -INFINITY;
}

DenseRowsPlan dense_rows_plan(const Dims& d, int ns) {
  DenseRowsPlan p;
  p.nrows = d.F * ns;
  p.ngroups = (p.nrows + 127) / 128;
  // about four workgroups per CU on 256 CUs, at least 4 key blocks per chunk
  const long long units = (long long)d.B * d.H * p.ngroups;
  int cpc = (int)((units * d.nb + 1023) / 1024);
  cpc = cpc < 4 ? 4 : cpc;
  p.cpc = cpc > d.nb ? d.nb : cpc;
  p.nchunks = (d.nb + p.cpc - 1) / p.cpc;
  const size_t parts = (size_t)d.B * d.H * p.ngroups * p.nchunks * 128;
  p.po_bytes = parts * 64 * sizeof(float);
  p.pml_bytes = parts * 2 * sizeof(float);
  return p;
}

hipError_t launch_dense_rows(const Dims& d, int ns, const void* q, const void* k, const void* v,
                             void* o, float* lse, void* ws, hipStream_t s) {
  const DenseRowsPlan p = dense_rows_plan(d, ns);
  float* po = static_cast<float*>(ws);
  float* pml = reinterpret_cast<float*>(static_cast<char*>(ws) + align256(p.po_bytes));
  DenseRowsArgs a{d, ns, p.nrows, p.ngroups, p.cpc, p.nchunks, (const __bf16*)q, (const __bf16*)k,
                  (const __bf16*)v, po, pml, (__bf16*)o, lse};
  const int grid = d.B * d.H * p.ngroups * p.nchunks;
  if (d.blk == 128)
    hipLaunchKernelGGL(k_dense_rows_partial<128>, dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_dense_rows_partial<64>, dim3(grid), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int waves = d.B * d.H * p.ngroups * 128;
  hipLaunchKernelGGL(k_dense_rows_merge, dim3((waves + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace bsgm
