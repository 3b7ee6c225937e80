// Block-sparse flash-attention forward, bf16 inputs, fp32 accumulation, for
// gfx950 (CDNA4) with 64-wide waves and bf16 MFMA.
//
// Work split: one workgroup per (b, h, query block) with BLK/32 waves; each
// wave owns 32 query rows. The workgroup walks the CSR list of its row in
// ascending key-block order; K and V tiles (BLK x 64 bf16) are staged in LDS,
// double-buffered, with the next tile's global loads issued before the
// current tile's math.
//
// Math per key tile, per wave (online softmax, exp2 with the scale folded in):
//   S^T = K Q^T      v_mfma_f32_32x32x16_bf16, A = K rows from LDS, B = Q in VGPRs
//   P   = exp2(S*c - m*c)  rounded to bf16 in registers
//   O^T += V^T P^T   v_mfma_f32_32x32x16_bf16, A = V^T via ds_read_b64_tr_b16, B = P
// Computing the transposes puts one query per lane pair (lanes l and l^32), so
// row max/sum need only in-lane work plus one v_permlane32_swap, and P feeds the
// second MFMA straight from registers. The K rows that feed the first MFMA are
// permuted (pi below) so that each lane's P registers hold 8 consecutive keys,
// the k-slot order that the second MFMA expects.
//
// LDS tiles are row-major (128 B per key row) with the 16-byte chunk index
// XOR-swizzled by swz(row), which keeps both the 16-byte K reads and the 8-byte
// transposing V reads free of bank conflicts within each access phase.
#include "device_util.h"

namespace bsgm {

struct AttnArgs {
  Dims d;
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  __bf16* o;
  float* lse;
};

__device__ __forceinline__ int swz(int row) { return ((row & 3) << 1) | ((row >> 3) & 1); }

__device__ __forceinline__ bf16x4 lds_read_tr(const unsigned char* p) {
  typedef bf16x4 __attribute__((address_space(3))) * lds_ptr;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_ptr)(p));
}

template <int BLK>
__global__ __launch_bounds__(BLK * 2, 2) void k_attn_bf16(AttnArgs a) {
  constexpr int NT = BLK * 2;          // threads (BLK/32 waves)
  constexpr int KT = BLK / 32;         // 32-key sub-tiles per key block
  constexpr int TB = BLK * 128;        // bytes of one K or V tile
  constexpr int CPT = (BLK * 8) / NT;  // 16-byte chunks per thread per tile
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * 2 * TB];

  const Dims& d = a.d;
  const int r = xcd_remap(blockIdx.x, d.rows);
  const int bh = r / d.nb, i = r - bh * d.nb;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 31, hh = lane >> 5;
  const size_t hoff = (size_t)bh * d.N * 64;
  const __bf16* Q = a.q + hoff;
  const __bf16* K = a.k + hoff;
  const __bf16* V = a.v + hoff;
  const int beg = a.row_ptr[r], end = a.row_ptr[r + 1];
  const int qrow = i * BLK + 32 * w + n;

  // B operand of S^T = K Q^T: column n = query, k-slots 8*hh.. = head dims.
  bf16x8 qf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    qf[ks] = *reinterpret_cast<const bf16x8*>(Q + (size_t)qrow * 64 + 16 * ks + 8 * hh);

  // Key row that A-operand lane row m reads: pi(m) with m = 8a + 4h + j maps to
  // 16(a/2) + 8h + 4(a%2) + j, so accumulator register x of lane l holds key
  // 16(x/8) + 8(l/32) + x%8 of the 32-key sub-tile.
  const int pim = ((n >> 4) << 4) | (((n >> 2) & 1) << 3) | (((n >> 3) & 1) << 2) | (n & 3);

  // Tile chunk c of this thread: key row cid/8, 16-byte column cid%8, with
  // cid = tid + NT*s; the LDS offset applies the chunk swizzle.
  int goff[CPT], soff[CPT];
#pragma unroll
  for (int s = 0; s < CPT; ++s) {
    const int cid = tid + NT * s;
    const int row = cid >> 3, c = cid & 7;
    goff[s] = cid * 8;
    soff[s] = row * 128 + ((c ^ swz(row)) << 4);
  }
  uint4 kreg0, kreg1, kreg2, kreg3, vreg0, vreg1, vreg2, vreg3;
  static_assert(CPT == 4, "four chunks per thread per tile");
#define BSGM_GLOAD(J)                                                   \
  do {                                                                  \
    const __bf16* kt_ = K + (size_t)(J) * BLK * 64;                     \
    const __bf16* vt_ = V + (size_t)(J) * BLK * 64;                     \
    kreg0 = *reinterpret_cast<const uint4*>(kt_ + goff[0]);             \
    kreg1 = *reinterpret_cast<const uint4*>(kt_ + goff[1]);             \
    kreg2 = *reinterpret_cast<const uint4*>(kt_ + goff[2]);             \
    kreg3 = *reinterpret_cast<const uint4*>(kt_ + goff[3]);             \
    vreg0 = *reinterpret_cast<const uint4*>(vt_ + goff[0]);             \
    vreg1 = *reinterpret_cast<const uint4*>(vt_ + goff[1]);             \
    vreg2 = *reinterpret_cast<const uint4*>(vt_ + goff[2]);             \
    vreg3 = *reinterpret_cast<const uint4*>(vt_ + goff[3]);             \
  } while (0)
#define BSGM_SWRITE(BUF)                                                \
  do {                                                                  \
    unsigned char* kb_ = smem + (BUF) * 2 * TB;                         \
    unsigned char* vb_ = kb_ + TB;                                      \
    *reinterpret_cast<uint4*>(kb_ + soff[0]) = kreg0;                   \
    *reinterpret_cast<uint4*>(kb_ + soff[1]) = kreg1;                   \
    *reinterpret_cast<uint4*>(kb_ + soff[2]) = kreg2;                   \
    *reinterpret_cast<uint4*>(kb_ + soff[3]) = kreg3;                   \
    *reinterpret_cast<uint4*>(vb_ + soff[0]) = vreg0;                   \
    *reinterpret_cast<uint4*>(vb_ + soff[1]) = vreg1;                   \
    *reinterpret_cast<uint4*>(vb_ + soff[2]) = vreg2;                   \
    *reinterpret_cast<uint4*>(vb_ + soff[3]) = vreg3;                   \
  } while (0)

  // Lane-constant parts of the transposing V read: within each 16-lane group g,
  // lane jj fetches 4 head dims of key row 8*(g/2) + jj/4 (+4 for the upper half).
  const int g16 = lane >> 4, jj = lane & 15;
  const int vrow0 = 8 * (g16 >> 1) + (jj >> 2);
  const int vbyte = 32 * (g16 & 1) + 8 * (jj & 3);

  f32x16 oacc[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int x = 0; x < 16; ++x) oacc[mt][x] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = d.scale * 1.4426950408889634f;

  if (beg < end) {
    BSGM_GLOAD(a.col_idx[beg]);
    BSGM_SWRITE(0);
  }
  __syncthreads();

  for (int it = beg; it < end; ++it) {
    const int buf = (it - beg) & 1;
    const int j = a.col_idx[it];
    const bool has_next = it + 1 < end;
    if (has_next) BSGM_GLOAD(a.col_idx[it + 1]);
    const unsigned char* kb = smem + buf * 2 * TB;
    const unsigned char* vb = kb + TB;

    f32x16 s[KT];
#pragma unroll
    for (int t = 0; t < KT; ++t) {
#pragma unroll
      for (int x = 0; x < 16; ++x) s[t][x] = 0.f;
      const int row = 32 * t + pim;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 ka =
            *reinterpret_cast<const bf16x8*>(kb + row * 128 + (((2 * ks + hh) ^ swz(row)) << 4));
        s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s[t], 0, 0, 0);
      }
    }

    const int vlen = block_vlen(d, j);
    if (vlen < BLK) {
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
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c2);
    const float mb = m_new * c2;

    bf16x8 pb[KT][2];
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[t][8 * e + x], c2, -mb));
          psum += p;
          pb[t][e][x] = (__bf16)p;
        }
    {
      const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(psum), __float_as_uint(psum),
                                                       false, false);
      psum = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int x = 0; x < 16; ++x) oacc[mt][x] *= alpha;

#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int kbase = 32 * t + 16 * e;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const int row_lo = kbase + vrow0, row_hi = row_lo + 4;
          const int byte = 64 * mt + vbyte;
          const int c = byte >> 4, sub = byte & 15;
          const bf16x4 lo = lds_read_tr(vb + row_lo * 128 + ((c ^ swz(row_lo)) << 4) + sub);
          const bf16x4 hi = lds_read_tr(vb + row_hi * 128 + ((c ^ swz(row_hi)) << 4) + sub);
          const bf16x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          oacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[t][e], oacc[mt], 0, 0, 0);
        }
      }

    if (has_next) BSGM_SWRITE(buf ^ 1);
    __syncthreads();
  }

  // Output: lane holds query qrow and head dims 32mt + 8(x/4) + 4hh + x%4.
  const bool real_q = (qrow % d.L) < d.Lv;
  const bool any = real_q && l_run > 0.f;
  const float inv = any ? 1.f / l_run : 0.f;
  __bf16* orow = a.o + hoff + (size_t)qrow * 64;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      bf16x4 ov;
#pragma unroll
      for (int x = 0; x < 4; ++x) ov[x] = (__bf16)(oacc[mt][4 * a4 + x] * inv);
      *reinterpret_cast<bf16x4*>(orow + 32 * mt + 8 * a4 + 4 * hh) = ov;
    }
  if (a.lse && hh == 0)
    a.lse[(size_t)bh * d.N + qrow] = any ? m_run * d.scale + logf(l_run) : -INFINITY;
}

hipError_t launch_attn_bf16(const Dims& d, const void* q, const void* k, const void* v,
                            const int32_t* row_ptr, const int32_t* col_idx, void* o,
                            float* lse, hipStream_t s) {
  AttnArgs a{d, (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, row_ptr, col_idx,
             (__bf16*)o, lse};
  if (d.blk == 128)
    hipLaunchKernelGGL(k_attn_bf16<128>, dim3(d.rows), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_attn_bf16<64>, dim3(d.rows), dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace bsgm
