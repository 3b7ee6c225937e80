// Drift contributions on the matrix cores, for bf16 K and V.
//
// For pooled query i (fp32 mean of Q over the real tokens of block i) and real
// key token u: l_iu = scale <qbar_i, k_u>; with M_i = max_u l_iu and
// Z_i = sum_u exp(l_iu - M_i),
//   contrib_ij = sum_{u in j} exp(l_iu - M_i) v_u / Z_i,   score_ij = ||contrib_ij||,
//   zmass_ij = sum_{u in j} exp(l_iu - M_i) / Z_i (optional).
//
// Both contractions run as v_mfma_f32_32x32x16_bf16 with fp32 accuracy: the
// fp32 operand (qbar in the logits, the weights in the value sum) is split into
// three bf16 terms whose sum is exactly the fp32 value (8 + 8 + 8 significant
// bits), and K and V are bf16 already, so every product is exact and only the
// fp32 accumulation rounds. Three launches:
//   k_drift_stats   per (query row i, key block j): block max m_ij and
//                   z_ij = sum_{u in j} exp(l_iu - m_ij);
//   k_drift_norm    per row: M_i = max_j m_ij, Z_i = sum_j z_ij exp(m_ij - M_i);
//   k_drift_contrib per (i, j): the weights exp(l_iu - M_i) / Z_i, then
//                   contrib = weights x V and its norm.
// A workgroup owns two key blocks of one (b, h), stages their K (and V) tiles
// in LDS once, and its four waves take the 32-row query tiles x key blocks.
#include "device_util.h"

namespace bsgm {

struct DriftMfmaArgs {
  Dims d;
  const float* qbar;     // [B*H*nb, 64]
  const __bf16* k;       // [B, H, N, 64]
  const __bf16* v;
  float2* stats;         // [B*H*nb, nb]: (m_ij, z_ij)
  float2* mz;            // [B*H*nb]: (M_i * log2(e), 1 / Z_i)
  float* contrib;        // [B*H*nb, nb, 64]
  float* score;          // [B*H*nb, nb]
  float* zmass;          // [B*H*nb, nb] or null: sum over the block of exp(l - M) / Z
};

constexpr int kDriftBlocksPerWg = 2;
constexpr float kLog2e = 1.4426950408889634f;

// x = hi + mid + lo exactly, each a bf16 (barring subnormal residuals).
__device__ __forceinline__ void split3(const float (&x)[8], bf16x8& hi, bf16x8& mid, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 h = (__bf16)x[e];
    const float r1 = x[e] - (float)h;
    const __bf16 m = (__bf16)r1;
    const float r2 = r1 - (float)m;
    hi[e] = h;
    mid[e] = m;
    lo[e] = (__bf16)r2;
  }
}

// Copies BLK key rows (128 bytes each) of `src` into a swizzled LDS tile.
template <int BLK, int NT>
__device__ __forceinline__ void stage_tile(unsigned char* dst, const __bf16* src) {
#pragma unroll
  for (int q = threadIdx.x; q < BLK * 8; q += NT) {
    const int row = q >> 3, pc = q & 7;
    *reinterpret_cast<uint4*>(dst + row * 128 + ((pc ^ swz(row)) << 4)) =
        *reinterpret_cast<const uint4*>(src + (size_t)row * 64 + pc * 8);
  }
}

// B operand of S^T = K Qbar^T for the query tile starting at row i0: lane l holds
// query i0 + l % 32 and head dims 16 ks + 8 (l / 32) .. +7, split in three terms.
__device__ __forceinline__ void load_qbar(const float* qbar_bh, int nb, int i0, int lane,
                                          bf16x8 (&qh)[4], bf16x8 (&qm)[4], bf16x8 (&ql)[4]) {
  const int i = i0 + (lane & 31);
  const bool ok = i < nb;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    float x[8];
    if (ok) {
      const float4* p = reinterpret_cast<const float4*>(qbar_bh + (size_t)i * 64 + 16 * ks +
                                                        8 * (lane >> 5));
      const float4 a = p[0], b = p[1];
      x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
      x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.f;
    }
    split3(x, qh[ks], qm[ks], ql[ks]);
  }
}

// Raw dot products <qbar_i, k_u> of the 32 keys of sub-tile t (register x of
// lane l: key 16 (x / 8) + 8 (l / 32) + x % 8, query l % 32).
__device__ __forceinline__ f32x16 qk_tile(const unsigned char* kb, int t, int lane,
                                          const bf16x8 (&qh)[4], const bf16x8 (&qm)[4],
                                          const bf16x8 (&ql)[4]) {
  f32x16 s;
#pragma unroll
  for (int x = 0; x < 16; ++x) s[x] = 0.f;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const bf16x8 ka = k_frag(kb, t, ks, lane);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, ql[ks], s, 0, 0, 0);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qm[ks], s, 0, 0, 0);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qh[ks], s, 0, 0, 0);
  }
  return s;
}

__device__ __forceinline__ int tile_key(int t, int x, int lane) {
  return 32 * t + 16 * (x >> 3) + 8 * (lane >> 5) + (x & 7);
}

template <int BLK>
__global__ __launch_bounds__(256, 4) void k_drift_stats(DriftMfmaArgs a) {
  constexpr int KT = BLK / 32, TB = BLK * 128;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kDriftBlocksPerWg * TB];
  const Dims& d = a.d;
  const int bh = blockIdx.y, j0 = kDriftBlocksPerWg * blockIdx.x;
  const int nj = min(kDriftBlocksPerWg, d.nb - j0);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const size_t hoff = (size_t)bh * d.N * 64;
  for (int jj = 0; jj < nj; ++jj)
    stage_tile<BLK, 256>(smem + jj * TB, a.k + hoff + (size_t)(j0 + jj) * BLK * 64);
  __syncthreads();

  const float* qbar_bh = a.qbar + (size_t)bh * d.nb * 64;
  const int nrt = (d.nb + 31) / 32;
  for (int u = w; u < nrt * nj; u += 4) {
    const int rt = u / nj, jj = u - rt * nj, j = j0 + jj;
    bf16x8 qh[4], qm[4], ql[4];
    load_qbar(qbar_bh, d.nb, 32 * rt, lane, qh, qm, ql);
    const int vlen = block_vlen(d, j);
    // one 32-key sub-tile at a time, merged online: (mx, z) over the real keys
    const float c2 = d.scale * kLog2e;
    float mx = -INFINITY, z = 0.f;
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      if (32 * t >= vlen) break;   // uniform: the remaining sub-tiles are padding
      const f32x16 s = qk_tile(smem + jj * TB, t, lane, qh, qm, ql);
      float mt = -INFINITY;
#pragma unroll
      for (int x = 0; x < 16; ++x)
        if (tile_key(t, x, lane) < vlen) mt = fmaxf(mt, s[x]);
      {
        const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt),
                                                         false, false);
        mt = fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
      }
      const float mb = mt * c2;
      float zt = 0.f;
#pragma unroll
      for (int x = 0; x < 16; ++x)
        if (tile_key(t, x, lane) < vlen) zt += __builtin_amdgcn_exp2f(fmaf(s[x], c2, -mb));
      {
        const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(zt), __float_as_uint(zt),
                                                         false, false);
        zt = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
      }
      // every sub-tile before vlen holds a real key, so mt is finite
      const float mn = fmaxf(mx, mt);
      z = z * __builtin_amdgcn_exp2f((mx - mn) * c2) + zt * __builtin_amdgcn_exp2f((mt - mn) * c2);
      mx = mn;
    }
    const int i = 32 * rt + (lane & 31);
    if (lane < 32 && i < d.nb)
      a.stats[((size_t)bh * d.nb + i) * d.nb + j] = make_float2(mx * d.scale, z);
  }
}

// One wave per pooled query row.
__global__ __launch_bounds__(256) void k_drift_norm(DriftMfmaArgs a) {
  const Dims& d = a.d;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (r >= d.rows) return;
  const float2* st = a.stats + (size_t)r * d.nb;
  float m = -INFINITY;
  for (int j = lane; j < d.nb; j += 64) m = fmaxf(m, st[j].x);
  m = wave_max(m);
  float z = 0.f;
  for (int j = lane; j < d.nb; j += 64) {
    const float2 e = st[j];
    z += e.y * expf(e.x - m);
  }
  z = wave_sum(z);
  if (lane == 0) a.mz[r] = make_float2(m * kLog2e, 1.f / z);
}

template <int BLK>
__global__ __launch_bounds__(256, 2) void k_drift_contrib_mfma(DriftMfmaArgs a) {
  constexpr int KT = BLK / 32, TB = BLK * 128;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kDriftBlocksPerWg * 2 * TB];
  const Dims& d = a.d;
  const int bh = blockIdx.y, j0 = kDriftBlocksPerWg * blockIdx.x;
  const int nj = min(kDriftBlocksPerWg, d.nb - j0);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n = lane & 31, hh = lane >> 5;
  const size_t hoff = (size_t)bh * d.N * 64;
  for (int jj = 0; jj < nj; ++jj) {
    stage_tile<BLK, 256>(smem + (2 * jj) * TB, a.k + hoff + (size_t)(j0 + jj) * BLK * 64);
    stage_tile<BLK, 256>(smem + (2 * jj + 1) * TB, a.v + hoff + (size_t)(j0 + jj) * BLK * 64);
  }
  __syncthreads();

  const float* qbar_bh = a.qbar + (size_t)bh * d.nb * 64;
  const float c2 = d.scale * kLog2e;
  const int nrt = (d.nb + 31) / 32;
  for (int u = w; u < nrt * nj; u += 4) {
    const int rt = u / nj, jj = u - rt * nj, j = j0 + jj;
    const unsigned char* kb = smem + (2 * jj) * TB;
    const unsigned char* vb = kb + TB;
    const int i = 32 * rt + n;
    bf16x8 qh[4], qm[4], ql[4];
    load_qbar(qbar_bh, d.nb, 32 * rt, lane, qh, qm, ql);
    const float2 mz = i < d.nb ? a.mz[(size_t)bh * d.nb + i] : make_float2(0.f, 0.f);
    const int vlen = block_vlen(d, j);

    // c[mt]: rows = queries 8 (x / 4) + 4 (l / 32) + x % 4 of the tile, column =
    // head dim 32 mt + l % 32.
    f32x16 c[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int x = 0; x < 16; ++x) c[mt][x] = 0.f;
    float wsum = 0.f;
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      const f32x16 s = qk_tile(kb, t, lane, qh, qm, ql);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        float p[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const float wgt = __builtin_amdgcn_exp2f(fmaf(s[8 * e + x], c2, -mz.x)) * mz.y;
          p[x] = tile_key(t, 8 * e + x, lane) < vlen ? wgt : 0.f;
          wsum += p[x];
        }
        bf16x8 ph, pm, pl;
        split3(p, ph, pm, pl);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const bf16x8 vf = v_frag(vb, 32 * t + 16 * e, mt, lane);
          c[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pl, vf, c[mt], 0, 0, 0);
          c[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pm, vf, c[mt], 0, 0, 0);
          c[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ph, vf, c[mt], 0, 0, 0);
        }
      }
    }

    // contrib rows: lanes 0-31 write 128 contiguous bytes of one query row,
    // lanes 32-63 those of the row 4 below.
    float* out = a.contrib + (((size_t)bh * d.nb) * d.nb + j) * 64;
    const size_t rs = (size_t)d.nb * 64;
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const int qi = 32 * rt + 8 * (x >> 2) + 4 * hh + (x & 3);
      if (qi < d.nb) {
        out[qi * rs + n] = c[0][x];
        out[qi * rs + 32 + n] = c[1][x];
      }
    }

    // score: sum of squares over the 64 head dims (32 lanes x 2 tiles) of each
    // of the 16 rows a lane holds. Halving exchanges leave lane n with the
    // total of row x = 8 b4 + 4 b3 + 2 b2 + b1 (b_k = bit k of n).
    float v[16];
#pragma unroll
    for (int x = 0; x < 16; ++x) v[x] = c[0][x] * c[0][x] + c[1][x] * c[1][x];
#pragma unroll
    for (int step = 0; step < 4; ++step) {
      const int msk = 16 >> step, half = 8 >> step;
      const bool up = (n & msk) != 0;
#pragma unroll
      for (int k2 = 0; k2 < half; ++k2) {
        const float send = up ? v[k2] : v[k2 + half];
        const float keep = up ? v[k2 + half] : v[k2];
        v[k2] = keep + __shfl_xor(send, msk, 64);
      }
    }
    v[0] += __shfl_xor(v[0], 1, 64);
    const int xr = (((n >> 4) & 1) << 3) | (((n >> 3) & 1) << 2) | (((n >> 2) & 1) << 1) |
                   ((n >> 1) & 1);
    const int qi = 32 * rt + 8 * (xr >> 2) + 4 * hh + (xr & 3);
    if ((n & 1) == 0 && qi < d.nb)
      a.score[((size_t)bh * d.nb + qi) * d.nb + j] = sqrtf(v[0]);
    if (a.zmass) {
      const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(wsum), __float_as_uint(wsum),
                                                       false, false);
      const float zt = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
      if (hh == 0 && i < d.nb) a.zmass[((size_t)bh * d.nb + i) * d.nb + j] = zt;
    }
  }
}

hipError_t launch_drift_contrib_bf16(const Dims& d, const float* qbar, const void* k,
                                     const void* v, float2* stats, float2* mz, float* contrib,
                                     float* score, float* zmass, hipStream_t s) {
  DriftMfmaArgs a{d, qbar, (const __bf16*)k, (const __bf16*)v, stats, mz, contrib, score, zmass};
  const dim3 grid((d.nb + kDriftBlocksPerWg - 1) / kDriftBlocksPerWg, d.B * d.H);
  if (d.blk == 128)
    hipLaunchKernelGGL(k_drift_stats<128>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_drift_stats<64>, grid, dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_drift_norm, dim3((d.rows + 3) / 4), dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (d.blk == 128)
    hipLaunchKernelGGL(k_drift_contrib_mfma<128>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_drift_contrib_mfma<64>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace bsgm
