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
// fp32 accumulation rounds. Four launches:
//   k_qbar_split    qbar as its three bf16 terms, once per row;
//   k_drift_stats   per (query row i, key block j): block max m_ij and
//                   z_ij = sum_{u in j} exp(l_iu - m_ij);
//   k_drift_norm    per row: M_i = max_j m_ij, Z_i = sum_j z_ij exp(m_ij - M_i);
//   k_drift_contrib per (i, j): the weights exp(l_iu - M_i) / Z_i, then
//                   contrib = weights x V and its norm.
// In the second and fourth, one wave owns one key block of one (b, h) and a run
// of 32-row query tiles: it loads the block's K fragments into registers once
// (and, for the value sums, its V tile into a private LDS slice), then walks
// its query tiles with no barrier, so the launches need no workgroup-wide
// staging and the waves of a CU run independently.
#include <algorithm>

#include "device_util.h"

namespace bsgm {

struct DriftMfmaArgs {
  Dims d;
  const float* qbar;     // [B*H*nb, 64]
  __bf16* qsplit;        // [B*H*nb, 3, 64]: qbar as hi, mid, lo bf16 terms
  const __bf16* k;       // [B, H, N, 64]
  const __bf16* v;
  float2* stats;         // [B*H*nb, nb]: (m_ij, z_ij)
  float2* mz;            // [B*H*nb]: (M_i log2(e) + log2(Z_i), 1 / Z_i): the weights are
                         // exp2(l_iu log2(e) - mz.x)
  float* contrib;        // [B*H*nb, nb, 64]
  float* score;          // [B*H*nb, nb]
  float* zmass;          // [B*H*nb, nb] or null: sum over the block of exp(l - M) / Z
};

constexpr float kLog2e = 1.4426950408889634f;

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;

// x = hi + mid + lo exactly, each a bf16 (barring subnormal residuals): hi is x
// rounded to bf16, mid the rounded remainder, lo what is left (at most 8
// significant bits, so exact). Pairs of values convert in one instruction.
__device__ __forceinline__ void split3(const float (&x)[8], bf16x8& hi, bf16x8& mid, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const f32x2 v = {x[2 * e], x[2 * e + 1]};
    const bf16x2 h = __builtin_convertvector(v, bf16x2);
    const f32x2 r1 = v - __builtin_convertvector(h, f32x2);
    const bf16x2 m = __builtin_convertvector(r1, bf16x2);
    const f32x2 r2 = r1 - __builtin_convertvector(m, f32x2);
    const bf16x2 l = __builtin_convertvector(r2, bf16x2);
    hi[2 * e] = h[0];
    hi[2 * e + 1] = h[1];
    mid[2 * e] = m[0];
    mid[2 * e + 1] = m[1];
    lo[2 * e] = l[0];
    lo[2 * e + 1] = l[1];
  }
}

// qsplit rows: thread (row, c) splits head dims 8c .. 8c + 7 of qbar once, for
// both per-(i, j) kernels.
__global__ __launch_bounds__(256) void k_qbar_split(DriftMfmaArgs a) {
  const int x = blockIdx.x * 256 + threadIdx.x;
  if (x >= a.d.rows * 8) return;
  const int row = x >> 3, c = x & 7;
  const float4* p = reinterpret_cast<const float4*>(a.qbar + (size_t)row * 64 + 8 * c);
  const float4 u = p[0], w = p[1];
  const float v[8] = {u.x, u.y, u.z, u.w, w.x, w.y, w.z, w.w};
  bf16x8 h, m, l;
  split3(v, h, m, l);
  bf16x8* o = reinterpret_cast<bf16x8*>(a.qsplit + (size_t)row * 192 + 8 * c);
  o[0] = h;
  o[8] = m;
  o[16] = l;
}

// Row fragments of sub-tile t of a block of 64-wide bf16 rows (K, or V as the
// A operand of V R^T), straight from global memory into registers: for
// head-dim step ks, lane l holds the 8 head dims 16 ks + 8 (l / 32) .. +7 of
// row 32 t + key_perm(l % 32) (the A operand of S^T = K Qbar^T, the layout
// k_frag reads from an LDS tile).
__device__ __forceinline__ void load_row_frags(const __bf16* blk, int t, int lane, bf16x8 (&f)[4]) {
  const __bf16* rowp = blk + (size_t)(32 * t + key_perm(lane & 31)) * 64 + 8 * (lane >> 5);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) f[ks] = *reinterpret_cast<const bf16x8*>(rowp + 16 * ks);
}

template <int KT>
__device__ __forceinline__ void load_k_frags(const __bf16* kblk, int lane, bf16x8 (&kf)[KT][4]) {
#pragma unroll
  for (int t = 0; t < KT; ++t) load_row_frags(kblk, t, lane, kf[t]);
}

// B operand of S^T = K Qbar^T for the query tile starting at row i0: lane l holds
// query i0 + l % 32 and head dims 16 ks + 8 (l / 32) .. +7, as three bf16 terms.
__device__ __forceinline__ void load_qsplit(const __bf16* qs_bh, int nb, int i0, int lane,
                                            bf16x8 (&qh)[4], bf16x8 (&qm)[4], bf16x8 (&ql)[4]) {
  const int i = i0 + (lane & 31);
  if (i < nb) {
    const __bf16* p = qs_bh + (size_t)i * 192 + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      qh[ks] = *reinterpret_cast<const bf16x8*>(p + 16 * ks);
      qm[ks] = *reinterpret_cast<const bf16x8*>(p + 64 + 16 * ks);
      ql[ks] = *reinterpret_cast<const bf16x8*>(p + 128 + 16 * ks);
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qh[ks][e] = (__bf16)0.f;
        qm[ks][e] = (__bf16)0.f;
        ql[ks][e] = (__bf16)0.f;
      }
    }
  }
}

// Raw dot products <qbar_i, k_u> of the 32 keys of sub-tile t (register x of
// lane l: key 16 (x / 8) + 8 (l / 32) + x % 8, query l % 32).
__device__ __forceinline__ f32x16 qk_tile(const bf16x8 (&kt)[4], const bf16x8 (&qh)[4],
                                          const bf16x8 (&qm)[4], const bf16x8 (&ql)[4]) {
  f32x16 s;
#pragma unroll
  for (int x = 0; x < 16; ++x) s[x] = 0.f;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt[ks], ql[ks], s, 0, 0, 0);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt[ks], qm[ks], s, 0, 0, 0);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt[ks], qh[ks], s, 0, 0, 0);
  }
  return s;
}

__device__ __forceinline__ int tile_key(int t, int x, int lane) {
  return 32 * t + 16 * (x >> 3) + 8 * (lane >> 5) + (x & 7);
}

// Work split of the two per-(i, j) kernels: one wave per (b, h, key block, run
// of `rtpw` consecutive 32-row query tiles), so that a wave loads its key block
// once and keeps it for all its query tiles. Waves are numbered
// ((b*H + h) * nb + j) * nsplit + s; there is no barrier, and a wave past the
// last item returns at once.
struct WaveItem {
  int bh, j, rt0, rt1;
};

__device__ __forceinline__ bool wave_item(const Dims& d, int rtpw, WaveItem& it) {
  const int nrt = (d.nb + 31) / 32, nsplit = (nrt + rtpw - 1) / rtpw;
  // wave-uniform (the compiler cannot tell from threadIdx), so that every
  // index and address derived from it lives in scalar registers
  const int gw = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (gw >= d.B * d.H * d.nb * nsplit) return false;
  const int s = gw % nsplit, bj = gw / nsplit;
  it.bh = bj / d.nb;
  it.j = bj - it.bh * d.nb;
  it.rt0 = s * rtpw;
  it.rt1 = min(nrt, it.rt0 + rtpw);
  return true;
}

// Sets the scores of the padding keys of sub-tile t to -inf, when the sub-tile
// straddles the end of the real keys (a wave-uniform test).
__device__ __forceinline__ void mask_padding(f32x16& s, int t, int vlen, int lane) {
  if (32 * t + 32 > vlen) {
#pragma unroll
    for (int x = 0; x < 16; ++x) s[x] = tile_key(t, x, lane) < vlen ? s[x] : -INFINITY;
  }
}

// (m_ij, z_ij) of one 32-row query tile against the wave's key block. FULL:
// the block has no padding keys; the products of the next 32-key sub-tile are
// then issued before this sub-tile's softmax work, in one branch-free block,
// so that the two overlap.
template <int KT, bool FULL>
__device__ __forceinline__ void stats_tile(const DriftMfmaArgs& a, const WaveItem& it, int rt,
                                           int vlen, int lane, const bf16x8 (&kf)[KT][4]) {
  const Dims& d = a.d;
  bf16x8 qh[4], qm[4], ql[4];
  load_qsplit(a.qsplit + (size_t)it.bh * d.nb * 192, d.nb, 32 * rt, lane, qh, qm, ql);
  const float c2 = d.scale * kLog2e;
  // one 32-key sub-tile at a time, merged online: (mx, z) over the real keys
  float mx = -INFINITY, z = 0.f;
  f32x16 s = qk_tile(kf[0], qh, qm, ql);
#pragma unroll
  for (int t = 0; t < KT; ++t) {
    if (!FULL && 32 * t >= vlen) break;   // uniform: the remaining sub-tiles are padding
    f32x16 sn;
    if (FULL && t + 1 < KT) sn = qk_tile(kf[t + 1], qh, qm, ql);
    if (!FULL) {
      if (t > 0) s = qk_tile(kf[t], qh, qm, ql);
      mask_padding(s, t, vlen, lane);
    }
    float mt = s[0];
#pragma unroll
    for (int x = 1; x < 16; ++x) mt = fmaxf(mt, s[x]);
    {
      const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt),
                                                       false, false);
      mt = fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
    }
    const float mb = mt * c2;
    float zt = 0.f;
#pragma unroll
    for (int x = 0; x < 16; ++x) zt += __builtin_amdgcn_exp2f(fmaf(s[x], c2, -mb));
    {
      const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(zt), __float_as_uint(zt),
                                                       false, false);
      zt = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
    }
    // every sub-tile before vlen holds a real key, so mt is finite
    const float mn = fmaxf(mx, mt);
    z = z * __builtin_amdgcn_exp2f((mx - mn) * c2) + zt * __builtin_amdgcn_exp2f((mt - mn) * c2);
    mx = mn;
    if (FULL && t + 1 < KT) s = sn;
  }
  const int i = 32 * rt + (lane & 31);
  if (lane < 32 && i < d.nb)
    a.stats[((size_t)it.bh * d.nb + i) * d.nb + it.j] = make_float2(mx * d.scale, z);
}

template <int BLK>
__global__ __launch_bounds__(256, 3) void k_drift_stats(DriftMfmaArgs a, int rtpw) {
  constexpr int KT = BLK / 32;
  const Dims& d = a.d;
  WaveItem it;
  if (!wave_item(d, rtpw, it)) return;
  const int lane = threadIdx.x & 63;
  bf16x8 kf[KT][4];
  load_k_frags<KT>(a.k + ((size_t)it.bh * d.N + (size_t)it.j * BLK) * 64, lane, kf);
  const int vlen = block_vlen(d, it.j);
  if (vlen == BLK)
    for (int rt = it.rt0; rt < it.rt1; ++rt) stats_tile<KT, true>(a, it, rt, vlen, lane, kf);
  else
    for (int rt = it.rt0; rt < it.rt1; ++rt) stats_tile<KT, false>(a, it, rt, vlen, lane, kf);
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
  // 1/Z folded into the exponent: a rounding of log2(Z) scales every weight of
  // the row by the same factor (2^-24 relative per unit of log2(Z))
  if (lane == 0) a.mz[r] = make_float2(fmaf(m, kLog2e, log2f(z)), 1.f / z);
}

// c += W V over the wave's key block (V tile in LDS at vb) for one 32-row
// query tile, with weights W_iu = exp2(s_iu c2 - mzx) (lane l's query is l % 32;
// mzx = +inf leaves its row unchanged). c[mt]: rows = queries
// 8 (x / 4) + 4 (l / 32) + x % 4 of the tile, column = head dim 32 mt + l % 32.
// ZM: wsum collects the lane's weights. FULL: the block has no padding keys,
// and the score products of the next sub-tile are issued before this
// sub-tile's weights, as in stats_tile. Otherwise sub-tiles that hold only
// padding keys (weights all zero) are skipped.
template <int KT, bool ZM, bool FULL>
__device__ __forceinline__ void weigh_values(const bf16x8 (&kf)[KT][4], const unsigned char* vb,
                                             const bf16x8 (&qh)[4], const bf16x8 (&qm)[4],
                                             const bf16x8 (&ql)[4], float mzx, float c2,
                                             int vlen, int lane, f32x16 (&c)[2], float& wsum) {
  f32x16 s = qk_tile(kf[0], qh, qm, ql);
#pragma unroll
  for (int t = 0; t < KT; ++t) {
    if (!FULL && 32 * t >= vlen) break;   // uniform: the remaining sub-tiles are padding
    f32x16 sn;
    if (FULL && t + 1 < KT) sn = qk_tile(kf[t + 1], qh, qm, ql);
    if (!FULL) {
      if (t > 0) s = qk_tile(kf[t], qh, qm, ql);
      mask_padding(s, t, vlen, lane);   // exp2(-inf) = 0: padding keys weigh nothing
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      float p[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        p[x] = __builtin_amdgcn_exp2f(fmaf(s[8 * e + x], c2, -mzx));
        if (ZM) wsum += p[x];
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
    if (FULL && t + 1 < KT) s = sn;
  }
}

// contrib, score (and zmass when ZM) of one 32-row query tile against the
// wave's key block, whose V tile sits in LDS at vb. NC: no contributions are
// written, and score receives the squared norm ||contrib_ij||^2 instead.
template <int KT, bool ZM, bool FULL, bool NC>
__device__ __forceinline__ void contrib_tile(const DriftMfmaArgs& a, const WaveItem& it, int rt,
                                             int vlen, int lane, const bf16x8 (&kf)[KT][4],
                                             const unsigned char* vb) {
  const Dims& d = a.d;
  const int n = lane & 31, hh = lane >> 5;
  const int i = 32 * rt + n;
  const int j = it.j, bh = it.bh;
  bf16x8 qh[4], qm[4], ql[4];
  load_qsplit(a.qsplit + (size_t)bh * d.nb * 192, d.nb, 32 * rt, lane, qh, qm, ql);
  const float2 mz = i < d.nb ? a.mz[(size_t)bh * d.nb + i] : make_float2(0.f, 0.f);
  const float c2 = d.scale * kLog2e;

  f32x16 c[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int x = 0; x < 16; ++x) c[mt][x] = 0.f;
  float wsum = 0.f;
  weigh_values<KT, ZM, FULL>(kf, vb, qh, qm, ql, i < d.nb ? mz.x : INFINITY, c2, vlen, lane, c,
                            wsum);

  // contrib rows: lanes 0-31 write 128 contiguous bytes of one query row,
  // lanes 32-63 those of the row 4 below. Raw buffer stores off a wave-uniform
  // resource at (b, h, row tile, j): the lane's byte offset in a VGPR, the
  // row's (a multiple of the row pitch) in an SGPR, so no store needs address
  // arithmetic. The tile spans under 32 * nb * 256 bytes.
  if (!NC) {
    const uint32_t rsb = (uint32_t)d.nb * 256u;   // bytes between query rows
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        a.contrib + (((size_t)bh * d.nb + 32 * rt) * d.nb + j) * 64, 0, (int)(32u * rsb), 0x00020000);
    const uint32_t off0 = (uint32_t)(4 * hh) * rsb + (uint32_t)n * 4u;
    if (32 * rt + 32 <= d.nb) {
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int so = (8 * (x >> 2) + (x & 3)) * (int)rsb;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(c[0][x]), rs, (int)off0, so, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(c[1][x]), rs, (int)off0 + 128, so, 0);
      }
    } else {
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int rr = 8 * (x >> 2) + (x & 3);
        if (32 * rt + 4 * hh + rr < d.nb) {
          const int so = rr * (int)rsb;
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(c[0][x]), rs, (int)off0, so, 0);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(c[1][x]), rs, (int)off0 + 128, so, 0);
        }
      }
    }
  }

  // score: sum of squares over the 64 head dims (32 lanes x 2 tiles) of each
  // of the 16 rows a lane holds, with one fixed contraction so that the
  // rounding does not depend on instruction scheduling. Halving exchanges
  // leave lane n with the total of row x = 8 b4 + 4 b3 + 2 b2 + b1 (b_k = bit
  // k of n).
  float v[16];
#pragma unroll
  for (int x = 0; x < 16; ++x) v[x] = fmaf(c[0][x], c[0][x], c[1][x] * c[1][x]);
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
    a.score[((size_t)bh * d.nb + qi) * d.nb + j] = NC ? v[0] : sqrtf(v[0]);
  if (ZM) {
    const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(wsum), __float_as_uint(wsum),
                                                     false, false);
    const float zt = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
    if (hh == 0 && i < d.nb) a.zmass[((size_t)bh * d.nb + i) * d.nb + j] = zt;
  }
}

// Each wave transposes its block's V through a private LDS tile (swizzled
// 128-byte rows, read back with the transposing LDS reads of v_frag) and keeps
// its K fragments in registers.
template <int BLK>
__device__ __forceinline__ void stage_v(const __bf16* src, int lane, unsigned char* vb) {
#pragma unroll
  for (int m = 0; m < BLK / 8; ++m) {
    const int q = lane + 64 * m, row = q >> 3, pc = q & 7;
    *reinterpret_cast<uint4*>(vb + row * 128 + ((pc ^ swz(row)) << 4)) =
        *reinterpret_cast<const uint4*>(src + (size_t)row * 64 + pc * 8);
  }
}

template <int BLK, bool ZM, bool NC>
__global__ __launch_bounds__(256, 2) void k_drift_contrib_mfma(DriftMfmaArgs a, int rtpw) {
  constexpr int KT = BLK / 32, TB = BLK * 128;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[4 * TB];
  const Dims& d = a.d;
  WaveItem it;
  if (!wave_item(d, rtpw, it)) return;
  const int lane = threadIdx.x & 63;
  unsigned char* vb = smem + (threadIdx.x >> 6) * TB;
  const size_t tok0 = (size_t)it.bh * d.N + (size_t)it.j * BLK;
  stage_v<BLK>(a.v + tok0 * 64, lane, vb);
  bf16x8 kf[KT][4];
  load_k_frags<KT>(a.k + tok0 * 64, lane, kf);
  const int vlen = block_vlen(d, it.j);
  // (the pipelined form needs 16 more registers than the zmass variant has)
  if (vlen == BLK && !ZM)
    for (int rt = it.rt0; rt < it.rt1; ++rt)
      contrib_tile<KT, ZM, true, NC>(a, it, rt, vlen, lane, kf, vb);
  else
    for (int rt = it.rt0; rt < it.rt1; ++rt)
      contrib_tile<KT, ZM, false, NC>(a, it, rt, vlen, lane, kf, vb);
}

// ---------------------------------------------------------------------------
// Re-rank rounds in the expanded form, without the contributions. With
// r_i = sum_{j in D_i} contrib_ij the residual of row i's drop set D_i, a
// round scores block j by 2 <r_i, contrib_ij> -/+ ||contrib_ij||^2, and
//   <r_i, contrib_ij> = sum_{u in j} w_iu <v_u, r_i>,   w_iu = exp(l_iu - M_i) / Z_i,
// so each round needs r_i (a weighted value sum over the dropped blocks) and
// then one scalar per (i, j), both recomputed from qbar, K, V and (M_i, Z_i).
// Nothing of size rows x nb x 64 is kept.
// ---------------------------------------------------------------------------
struct DriftRoundArgs {
  const uint32_t* kept;   // [rows, W]: the round's kept set (bit j % 32 of word j / 32),
                          // or null: every block counts (the total o_i = sum_j contrib_ij)
  int via_kept;           // sum the kept blocks and take r = o - that sum
  float* obar;            // [rows, 64]: o_i
  float* part;            // [rows, ngroups, 64]: per group of key blocks, the partial sum
  int ngroups;
  __bf16* rsplit;         // [rows, 3, 64]: r as hi, mid, lo bf16 terms
  float* dot;             // [rows, nb]: <r_i, contrib_ij>
};

// Per row (one wave): the sum of the group partials in group order. Without
// kept sets that is o_i, stored as such. Otherwise r (o_i minus the sum with
// via_kept), its three bf16 terms for the dot products, and J^2 = ||r||^2;
// with best, also the kept set of least J so far (round 0 starts it; ties
// keep the earlier set).
__global__ __launch_bounds__(256) void k_drift_resid(DriftRoundArgs r, int rows, int W, int round,
                                                     float* jsq, uint32_t* best, float* jbest) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float* p = r.part + (size_t)row * r.ngroups * 64 + lane;
  float x = 0.f;
  for (int g = 0; g < r.ngroups; ++g) x += p[(size_t)g * 64];
  if (!r.kept) {
    r.obar[(size_t)row * 64 + lane] = x;
    return;
  }
  if (r.via_kept) x = r.obar[(size_t)row * 64 + lane] - x;
  const __bf16 h = (__bf16)x;
  const float r1 = x - (float)h;
  const __bf16 m = (__bf16)r1;
  const __bf16 l = (__bf16)(r1 - (float)m);
  __bf16* o = r.rsplit + (size_t)row * 192 + lane;
  o[0] = h;
  o[64] = m;
  o[128] = l;
  const float j2 = wave_sum(x * x);   // bitwise the same in every lane
  if (lane == 0) jsq[row] = j2;
  if (best) {
    const bool take = round == 0 || j2 < jbest[row];
    if (take) {
      if (lane == 0) jbest[row] = j2;
      for (int w = lane; w < W; w += 64) best[(size_t)row * W + w] = r.kept[(size_t)row * W + w];
    }
  }
}

// ---------------------------------------------------------------------------
// The two round passes, row-stationary. A workgroup of WV waves owns WV
// consecutive 32-row query tiles of one (b, h) (wave w takes tile WV * rg + w;
// waves past the last tile only help to stage) and a range of key blocks. Each
// wave keeps its tile's bf16 terms of qbar (and of r) in registers for the
// whole range, and every key block's K and V tiles are staged once in LDS for
// all WV waves, instead of once per wave as in the contribution kernel (whose
// waves each own a key block and walk query tiles). Staging is double-buffered
// through registers: the next block's global loads are issued before the
// waves work on the current block and land in the other LDS buffer after it,
// so one barrier per block orders both buffers. A (row, block) pair takes the
// products of the contribution kernel in the same order, and a row's partial
// sum adds its counted blocks in ascending order, so the results do not depend
// on the grid.
// ---------------------------------------------------------------------------
constexpr int kRsMaskWords = 128;   // counted-block bitmask of a range: up to 4096 blocks

// Register stage of one block's K and V tiles (BLK * 128 bytes each) over the
// 64 * WV threads of the workgroup: thread x holds 16-byte chunks x, x + 64 WV,
// ... of each tile. Chunk c of a tile is row c / 8, head dims 8 (c % 8) .. +7,
// stored at the swizzled LDS place that k_frag and v_frag read.
template <int BLK, int WV>
struct RsStage {
  static constexpr int TB = BLK * 128, CT = BLK * 8, NT = 64 * WV;
  static constexpr int PT = (CT + NT - 1) / NT;
  static constexpr bool EVEN = CT % NT == 0;
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  u32x4 rk[PT], rv[PT];
  // every element is loaded (a thread past the last chunk reloads the last
  // one), so that no element keeps a value from an earlier load
  __device__ __forceinline__ void load(const __bf16* k, const __bf16* v, int x) {
#pragma unroll
    for (int p = 0; p < PT; ++p) {
      const int c = EVEN ? x + NT * p : min(x + NT * p, CT - 1);
      rk[p] = *reinterpret_cast<const u32x4*>(k + (size_t)c * 8);
      rv[p] = *reinterpret_cast<const u32x4*>(v + (size_t)c * 8);
    }
  }
  __device__ __forceinline__ void store(unsigned char* kb, int x) const {
#pragma unroll
    for (int p = 0; p < PT; ++p) {
      const int c = x + NT * p, row = c >> 3, pc = c & 7;
      if (EVEN || c < CT) {
        const int off = row * 128 + ((pc ^ swz(row)) << 4);
        *reinterpret_cast<u32x4*>(kb + off) = rk[p];
        *reinterpret_cast<u32x4*>(kb + TB + off) = rv[p];
      }
    }
  }
};

// First block j' >= j of [.., j1) whose bit is set in the LDS mask (word w
// covers blocks 32 (wb + w) .. +31); j1 if none. Every thread gets the same.
__device__ __forceinline__ int rs_next(const uint32_t* um, int wb, int j, int j1) {
  while (j < j1) {
    const uint32_t m = um[(j >> 5) - wb] >> (j & 31);
    if (m) return min(j + (int)__builtin_ctz(m), j1);
    j = (j | 31) + 1;
  }
  return j1;
}

// c += W V over one staged block (K tile at kb, V tile at vb), K fragments read
// from LDS per 32-key sub-tile; the sub-tile work of weigh_values without the
// pipelined form.
template <int KT>
__device__ __forceinline__ void weigh_values_lds(const unsigned char* kb, const unsigned char* vb,
                                                 const bf16x8 (&qh)[4], const bf16x8 (&qm)[4],
                                                 const bf16x8 (&ql)[4], float mzx, float c2,
                                                 int vlen, int lane, f32x16 (&c)[2]) {
#pragma unroll
  for (int t = 0; t < KT; ++t) {
    if (32 * t >= vlen) break;   // uniform: the remaining sub-tiles are padding
    bf16x8 kt[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kt[ks] = k_frag(kb, t, ks, lane);
    f32x16 s = qk_tile(kt, qh, qm, ql);
    mask_padding(s, t, vlen, lane);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      float p[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) p[x] = __builtin_amdgcn_exp2f(fmaf(s[8 * e + x], c2, -mzx));
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
}

// Residual partial sums: workgroup (b, h, row group rg, key group g) sums W V
// over the blocks [g nb / G, (g + 1) nb / G) that its rows count, the weights of
// a row for which a block does not count set to zero. A block counts where it
// is dropped, or with via_kept where it is kept (the smaller set when fewer
// blocks are kept than dropped; the kept sets of neighbouring rows overlap).
// A block is staged when some row of the workgroup counts it, and a wave adds
// it when some row of its tile does. Grid: B * H * ceil(nrt / WV) * ngroups.
template <int BLK, int WV>
__global__ __launch_bounds__(64 * WV, 2) void k_drift_dropsum(DriftMfmaArgs a, DriftRoundArgs r) {
  constexpr int KT = BLK / 32, TB = BLK * 128;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2][2 * TB];
  __shared__ uint32_t umask[kRsMaskWords];
  const Dims& d = a.d;
  const int nrt = (d.nb + 31) / 32, ngr = (nrt + WV - 1) / WV, G = r.ngroups, W = (d.nb + 31) >> 5;
  const int g = blockIdx.x % G, rg = (blockIdx.x / G) % ngr, bh = blockIdx.x / (G * ngr);
  const int j0 = (int)((long long)g * d.nb / G), j1 = (int)((long long)(g + 1) * d.nb / G);
  const int x = threadIdx.x, lane = x & 63, n = lane & 31, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(x >> 6);
  const int rt = rg * WV + w, i = 32 * rt + n;
  const uint32_t inv = r.via_kept ? 0u : 0xFFFFFFFFu;   // counted: kept bits, or dropped bits
  const int wb = j0 >> 5;
  // the blocks that some row of the workgroup counts
  if (r.kept) {
    const int nw = ((j1 - 1) >> 5) - wb + 1, row0 = 32 * WV * rg;
    const int nrows = min(32 * WV, d.nb - row0);
    for (int y = x; y < nw; y += 64 * WV) umask[y] = 0u;
    __syncthreads();
    const uint32_t* kr = r.kept + ((size_t)bh * d.nb + row0) * W + wb;
    for (int y = x; y < nrows * nw; y += 64 * WV) {
      const int q = y / nw, wi = y - q * nw;
      const uint32_t word = kr[(size_t)q * W + wi] ^ inv;
      if (word) atomicOr(&umask[wi], word);
    }
    __syncthreads();
  }
  auto next = [&](int j) { return r.kept ? rs_next(umask, wb, j, j1) : j; };
  const size_t tokb = (size_t)bh * d.N;
  RsStage<BLK, WV> st;
  int j = next(j0);
  if (j < j1) {
    st.load(a.k + (tokb + (size_t)j * BLK) * 64, a.v + (tokb + (size_t)j * BLK) * 64, x);
    st.store(smem[0], x);
  }
  bf16x8 qh[4], qm[4], ql[4];
  load_qsplit(a.qsplit + (size_t)bh * d.nb * 192, d.nb, 32 * rt, lane, qh, qm, ql);
  const bool live = i < d.nb;
  const float mzx_row = live ? a.mz[(size_t)bh * d.nb + i].x : INFINITY;
  const float c2 = d.scale * kLog2e;
  const uint32_t* krow = r.kept ? r.kept + ((size_t)bh * d.nb + min(i, d.nb - 1)) * W : nullptr;
  // the row's counted bits of the word holding the current block
  uint32_t wcur = (krow && j < j1) ? krow[j >> 5] ^ inv : 0xFFFFFFFFu;
  f32x16 c[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int e = 0; e < 16; ++e) c[mt][e] = 0.f;
  __syncthreads();
  int cur = 0;
  // The stage is loaded and stored in every pass (the last block's pass
  // reloads that block into the idle buffer), so that no stage value lives
  // across a pass.
  while (j < j1) {
    const int jn = next(j + 1), jl = jn < j1 ? jn : j;
    // the next block's word first, then its tiles: both land before the store
    uint32_t wnext = wcur;
    if (krow && jn < j1 && (jn >> 5) != (j >> 5)) wnext = krow[jn >> 5] ^ inv;
    st.load(a.k + (tokb + (size_t)jl * BLK) * 64, a.v + (tokb + (size_t)jl * BLK) * 64, x);
    const bool drop = live && ((wcur >> (j & 31)) & 1u) != 0;
    if (__ballot(drop) != 0ull)   // uniform
      weigh_values_lds<KT>(smem[cur], smem[cur] + TB, qh, qm, ql, drop ? mzx_row : INFINITY, c2,
                           block_vlen(d, j), lane, c);
    st.store(smem[cur ^ 1], x);
    if (jn >= j1) break;
    __syncthreads();
    cur ^= 1;
    j = jn;
    wcur = wnext;
  }
  if (rt >= nrt) return;
  float* prow = r.part + (((size_t)bh * d.nb + 32 * rt) * G + g) * 64;
  const size_t rs = (size_t)G * 64;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int q = 8 * (e >> 2) + 4 * hh + (e & 3);
    if (32 * rt + q < d.nb) {
      prow[q * rs + n] = c[0][e];
      prow[q * rs + 32 + n] = c[1][e];
    }
  }
}

// <r_i, contrib_ij> for every block of a range: workgroup (b, h, row group rg,
// range g of ngroups equal ranges). Per block and query tile, X = V R^T on the
// matrix cores (V rows as the A operand, read from LDS as K fragments are; r as
// three bf16 terms, so the products are exact; X has the layout of S^T), then
// the weighted sum sum_u w_iu X_ui over the block's real keys.
template <int BLK, int WV>
__global__ __launch_bounds__(64 * WV, 2) void k_drift_dot(DriftMfmaArgs a, DriftRoundArgs r) {
  constexpr int KT = BLK / 32, TB = BLK * 128;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2][2 * TB];
  const Dims& d = a.d;
  const int nrt = (d.nb + 31) / 32, ngr = (nrt + WV - 1) / WV, G = r.ngroups;
  const int g = blockIdx.x % G, rg = (blockIdx.x / G) % ngr, bh = blockIdx.x / (G * ngr);
  const int j0 = (int)((long long)g * d.nb / G), j1 = (int)((long long)(g + 1) * d.nb / G);
  const int x = threadIdx.x, lane = x & 63;
  const int w = __builtin_amdgcn_readfirstlane(x >> 6);
  const int rt = rg * WV + w, i = 32 * rt + (lane & 31);
  const size_t tokb = (size_t)bh * d.N;
  RsStage<BLK, WV> st;
  if (j0 < j1) {
    st.load(a.k + (tokb + (size_t)j0 * BLK) * 64, a.v + (tokb + (size_t)j0 * BLK) * 64, x);
    st.store(smem[0], x);
  }
  bf16x8 qh[4], qm[4], ql[4], rh[4], rm[4], rl[4];
  load_qsplit(a.qsplit + (size_t)bh * d.nb * 192, d.nb, 32 * rt, lane, qh, qm, ql);
  load_qsplit(r.rsplit + (size_t)bh * d.nb * 192, d.nb, 32 * rt, lane, rh, rm, rl);
  const float mzx = i < d.nb ? a.mz[(size_t)bh * d.nb + i].x : INFINITY;
  const float c2 = d.scale * kLog2e;
  float* drow = r.dot + ((size_t)bh * d.nb + min(i, d.nb - 1)) * d.nb;
  const bool busy = rt < nrt;
  __syncthreads();
  int cur = 0;
  for (int j = j0; j < j1; ++j) {
    // loaded and stored in every pass, as in k_drift_dropsum
    const int jl = min(j + 1, j1 - 1);
    st.load(a.k + (tokb + (size_t)jl * BLK) * 64, a.v + (tokb + (size_t)jl * BLK) * 64, x);
    if (busy) {
      const unsigned char* kb = smem[cur];
      const unsigned char* vb = smem[cur] + TB;
      const int vlen = block_vlen(d, j);
      float acc = 0.f;
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        if (32 * t >= vlen) break;   // uniform: the remaining sub-tiles are padding
        bf16x8 kt[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kt[ks] = k_frag(kb, t, ks, lane);
        f32x16 s = qk_tile(kt, qh, qm, ql);
        mask_padding(s, t, vlen, lane);   // weight 0 for padding keys
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kt[ks] = k_frag(vb, t, ks, lane);
        const f32x16 xv = qk_tile(kt, rh, rm, rl);
#pragma unroll
        for (int e = 0; e < 16; ++e)
          acc = fmaf(__builtin_amdgcn_exp2f(fmaf(s[e], c2, -mzx)), xv[e], acc);
      }
      const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc), __float_as_uint(acc),
                                                       false, false);
      const float tot = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
      if (lane < 32 && i < d.nb) drow[j] = tot;
    }
    st.store(smem[cur ^ 1], x);
    if (j + 1 >= j1) break;
    __syncthreads();
    cur ^= 1;
  }
}

// Query tiles per wave for `slots` resident waves on the chip: among the
// choices of least makespan (query tiles per slot, counting whole rounds of
// resident waves), the most tiles per wave, which loads each key block the
// fewest times.
static int tiles_per_wave(const Dims& d, int slots) {
  const int nrt = (d.nb + 31) / 32;
  const long long bjs = (long long)d.B * d.H * d.nb;
  long long best_span = -1;
  int best = nrt;
  for (int r = nrt; r >= 1; --r) {
    const long long waves = bjs * ((nrt + r - 1) / r);
    const long long span = ((waves + slots - 1) / slots) * r;
    if (best_span < 0 || span < best_span) {
      best_span = span;
      best = r;
    }
  }
  return best;
}

static int compute_units() {
  static int cu = 0;
  if (cu == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cu = n;
    else
      cu = 256;
  }
  return cu;
}

// qbar's split terms, the per-(i, j) statistics and the per-row (M_i, Z_i).
static hipError_t launch_drift_stats(const DriftMfmaArgs& a, hipStream_t s) {
  const Dims& d = a.d;
  const int nrt = (d.nb + 31) / 32;
  const long long bjs = (long long)d.B * d.H * d.nb;
  hipLaunchKernelGGL(k_qbar_split, dim3((d.rows * 8 + 255) / 256), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    // stats: 3 waves per SIMD
    const int r = tiles_per_wave(d, compute_units() * 12);
    const long long waves = bjs * ((nrt + r - 1) / r);
    const dim3 grid((unsigned)((waves + 3) / 4));
    if (d.blk == 128)
      hipLaunchKernelGGL(k_drift_stats<128>, grid, dim3(256), 0, s, a, r);
    else
      hipLaunchKernelGGL(k_drift_stats<64>, grid, dim3(256), 0, s, a, r);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_drift_norm, dim3((d.rows + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Grid of a per-(b, h, key block, run of query tiles) kernel at `slots`
// resident waves; r receives the run length.
static dim3 wave_grid(const Dims& d, int slots, int& r) {
  const int nrt = (d.nb + 31) / 32;
  r = tiles_per_wave(d, slots);
  const long long waves = (long long)d.B * d.H * d.nb * ((nrt + r - 1) / r);
  return dim3((unsigned)((waves + 3) / 4));
}

template <bool ZM, bool NC>
static void launch_contrib(const DriftMfmaArgs& a, hipStream_t s) {
  // contributions: 2 waves per SIMD
  int r = 0;
  const dim3 grid = wave_grid(a.d, compute_units() * 8, r);
  if (a.d.blk == 128)
    hipLaunchKernelGGL((k_drift_contrib_mfma<128, ZM, NC>), grid, dim3(256), 0, s, a, r);
  else
    hipLaunchKernelGGL((k_drift_contrib_mfma<64, ZM, NC>), grid, dim3(256), 0, s, a, r);
}

hipError_t launch_drift_contrib_bf16(const Dims& d, const float* qbar, void* qsplit, const void* k,
                                     const void* v, float2* stats, float2* mz, float* contrib,
                                     float* score, float* zmass, hipStream_t s) {
  DriftMfmaArgs a{d, qbar, (__bf16*)qsplit, (const __bf16*)k, (const __bf16*)v, stats, mz, contrib,
                  score, zmass};
  hipError_t e = launch_drift_stats(a, s);
  if (e != hipSuccess) return e;
  if (zmass) launch_contrib<true, false>(a, s);
  else launch_contrib<false, false>(a, s);
  return hipGetLastError();
}

hipError_t launch_drift_sqnorms_bf16(const Dims& d, const float* qbar, void* qsplit, const void* k,
                                     const void* v, float2* stats, float2* mz, float* sqnorm,
                                     hipStream_t s) {
  DriftMfmaArgs a{d, qbar, (__bf16*)qsplit, (const __bf16*)k, (const __bf16*)v, stats, mz, nullptr,
                  sqnorm, nullptr};
  hipError_t e = launch_drift_stats(a, s);
  if (e != hipSuccess) return e;
  launch_contrib<false, true>(a, s);
  return hipGetLastError();
}

int drift_round_groups_max(const Dims& d) { return d.nb < 16 ? d.nb : 16; }

// Waves per workgroup of the row-stationary passes: the query tiles of a
// (b, h) in equal groups of three or four (four, some idle, for rows of at
// most 64 blocks: fewer waves would hold a whole block's stage each).
static int rs_waves(const Dims& d) {
  const int nrt = (d.nb + 31) / 32;
  const int ngr = (nrt + 3) / 4;
  const int wv = (nrt + ngr - 1) / ngr;
  return wv < 3 ? 4 : wv;
}

// Least group count whose ranges fit the counted-block mask (4096 blocks,
// less one word for a range that starts inside a word). At most
// drift_round_groups_max for every row width the streamed selection accepts.
static int rs_min_groups(const Dims& d) {
  const int span = 32 * (kRsMaskWords - 1);
  return (d.nb + span - 1) / span;
}

// Ranges of key blocks per row group in the dot pass: 16 (measured best on 176-
// and 1100-block rows against 4 to 64), one block each on narrower rows.
static int rs_dot_ranges(const Dims& d) { return std::min(16, d.nb); }

template <bool DROPSUM, int BLK, int WV>
static void launch_rs_k(const DriftMfmaArgs& a, const DriftRoundArgs& r, dim3 grid, hipStream_t s) {
  if (DROPSUM)
    hipLaunchKernelGGL((k_drift_dropsum<BLK, WV>), grid, dim3(64 * WV), 0, s, a, r);
  else
    hipLaunchKernelGGL((k_drift_dot<BLK, WV>), grid, dim3(64 * WV), 0, s, a, r);
}

template <bool DROPSUM, int BLK>
static void launch_rs_b(const DriftMfmaArgs& a, const DriftRoundArgs& r, hipStream_t s) {
  const Dims& d = a.d;
  const int nrt = (d.nb + 31) / 32, wv = rs_waves(d), ngr = (nrt + wv - 1) / wv;
  const dim3 grid((unsigned)((long long)d.B * d.H * ngr * r.ngroups));
  if (wv == 3) launch_rs_k<DROPSUM, BLK, 3>(a, r, grid, s);
  else launch_rs_k<DROPSUM, BLK, 4>(a, r, grid, s);
}

template <bool DROPSUM>
static void launch_rs(const DriftMfmaArgs& a, const DriftRoundArgs& r, hipStream_t s) {
  if (a.d.blk == 128) launch_rs_b<DROPSUM, 128>(a, r, s);
  else launch_rs_b<DROPSUM, 64>(a, r, s);
}

hipError_t launch_drift_residual_bf16(const Dims& d, const void* qsplit, const void* k,
                                      const void* v, const float2* mz, const uint32_t* kept,
                                      int via_kept, float* obar, float* part, void* rsplit,
                                      float* jsq, uint32_t* best, float* jbest, int round,
                                      hipStream_t s) {
  DriftMfmaArgs a{d, nullptr, (__bf16*)qsplit, (const __bf16*)k, (const __bf16*)v, nullptr,
                  const_cast<float2*>(mz), nullptr, nullptr, nullptr};
  // as many key groups as part holds (16 measured best on 176- and 1100-block rows)
  const int G = drift_round_groups_max(d);
  if (G < rs_min_groups(d)) return hipErrorInvalidValue;   // rows too wide for the mask
  DriftRoundArgs r{kept, via_kept, obar, part, G, (__bf16*)rsplit, nullptr};
  launch_rs<true>(a, r, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_drift_resid, dim3((d.rows + 3) / 4), dim3(256), 0, s, r, d.rows,
                     (d.nb + 31) >> 5, round, jsq, best, jbest);
  return hipGetLastError();
}

hipError_t launch_drift_resid(const Dims& d, const uint32_t* kept, int via_kept, float* obar,
                              float* part, int ngroups, void* rsplit, float* jsq, uint32_t* best,
                              float* jbest, int round, hipStream_t s) {
  DriftRoundArgs r{kept, via_kept, obar, part, ngroups, (__bf16*)rsplit, nullptr};
  hipLaunchKernelGGL(k_drift_resid, dim3((d.rows + 3) / 4), dim3(256), 0, s, r, d.rows,
                     (d.nb + 31) >> 5, round, jsq, best, jbest);
  return hipGetLastError();
}

hipError_t launch_drift_dot_bf16(const Dims& d, const void* qsplit, const void* rsplit,
                                 const void* k, const void* v, const float2* mz, float* dot,
                                 hipStream_t s) {
  DriftMfmaArgs a{d, nullptr, (__bf16*)qsplit, (const __bf16*)k, (const __bf16*)v, nullptr,
                  const_cast<float2*>(mz), nullptr, nullptr, nullptr};
  DriftRoundArgs r{nullptr, 0, nullptr, nullptr, rs_dot_ranges(d), (__bf16*)rsplit, dot};
  launch_rs<false>(a, r, s);
  return hipGetLastError();
}

}  // namespace bsgm
