// Block-sparse flash-attention forward, bf16 inputs, fp32 accumulation, for
// gfx950 (CDNA4) with 64-wide waves and matrix cores.
//
// Work split: one workgroup per (b, h, query block) with BLK/32 waves; each
// wave owns 32 query rows. The workgroup walks the CSR list of its row in
// ascending key-block order; K and V tiles (BLK x 64, 2 bytes per element) are
// staged in LDS, double-buffered: right after the barrier that opens a tile, the
// waves issue direct global->LDS copies of the next tile into the other buffer,
// which land while the current tile's math runs. The row's column list is kept
// in an LDS ring, entry x packing the block of tile x + 1 (whose copy tile x
// issues) with the number of real keys of tile x, so the loop reads one LDS word
// and no global memory besides the tiles per tile.
//
// Logits, in one of two forms:
//  - fp16 (with a workspace): k_k_to_f16 first copies K to fp16, and each wave
//    holds its queries as fp16(q * scale * log2 e). The first product then
//    yields base-2 logits, and its accumulator starts at -m, so
//    P = exp2(accumulator) takes no per-score arithmetic. The fp16 copy of a
//    bf16 value x is exact for |x| >= 2^-17 (fp16 keeps 11 significant bits
//    down to 2^-14 and steps of 2^-24 below); smaller values move by at most
//    2^-25. The scaled query keeps 11 significant bits (relative error 2^-12)
//    above 2^-14 and an absolute error of at most 2^-25 below. The form is
//    used only where every |k| of the listed key blocks and every
//    |q * scale * log2 e| of the query block is below 2^7, so that the two
//    absolute terms add at most 64 * 2^7 * 2^-25 = 2^-12 each to a base-2
//    logit: its error is at most 2^-12 * sum_d |q_d c k_d| + 2^-11, plus the
//    fp32 accumulation. A query block outside that range, or one of whose
//    listed key blocks is, is flagged and left to the bf16 form, which a
//    second launch runs for the flagged rows only.
//  - bf16: S = K Q^T on the bf16 inputs, P = exp2(S c - m c), c = scale log2 e.
// Softmax keeps a reference maximum m per query row instead of a running one:
// m is the maximum of the row's first tile, and it moves (O and l rescaled)
// only when a later tile would make some P exceed 2^64, which is detected from
// the tile's row sum (no per-tile maximum). P that large is still far inside
// the fp32 and bf16 ranges, and the softmax is the same for any reference. The
// row sum is taken from the bf16-rounded P, the values that enter the second
// MFMA.
//
// Math per key tile, per wave:
//   S^T = K Q^T      v_mfma_f32_32x32x16_{f16,bf16}, A = K rows from LDS, B = Q in VGPRs
//   P   = exp2(...)  rounded to bf16 in registers
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
#include <type_traits>

#include "device_util.h"

namespace bsgm {

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;

struct AttnArgs {
  Dims d;
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  __bf16* o;
  float* lse;
  const _Float16* kh;   // fp16 form: K in fp16
  const int32_t* kbad;  // fp16 form: per (b, h, key block), nonzero if some |k| >= kF16FormMax
  int32_t* redo;        // per row: the fp16 form writes 1 (left to the bf16 form) or 0;
                        // the bf16 form, when given it, runs only the rows marked 1
};

// Magnitude bound of K and of q * scale * log2 e in the fp16 form (larger,
// infinite or NaN values flag their block). It caps what the fp16 rounding
// below 2^-14 (absolute, at most 2^-25 per element) can add to a logit.
constexpr float kF16FormMax = 128.f;

// fp16 copy of K, one workgroup per (b, h, key block), and the block's range flag.
template <int BLK>
__global__ __launch_bounds__(256) void k_k_to_f16(const __bf16* __restrict__ k,
                                                  _Float16* __restrict__ kh,
                                                  int32_t* __restrict__ kbad) {
  constexpr int V8 = BLK * 64 / 8;   // 8-element vectors per block
  const size_t base = (size_t)blockIdx.x * V8;
  int out = 0;
#pragma unroll
  for (int x = threadIdx.x; x < V8; x += 256) {
    const bf16x8 v = reinterpret_cast<const bf16x8*>(k)[base + x];
    f16x8 h;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float f = (float)v[e];
      out |= !(fabsf(f) < kF16FormMax);
      h[e] = (_Float16)f;
    }
    reinterpret_cast<f16x8*>(kh)[base + x] = h;
  }
  out = __syncthreads_or(out);
  if (threadIdx.x == 0) kbad[blockIdx.x] = out != 0;
}

template <int BLK, bool F16>
__global__ __launch_bounds__(BLK * 2, 2) void k_attn_bf16(AttnArgs a) {
  constexpr int NT = BLK * 2;          // threads (BLK/32 waves)
  constexpr int KT = BLK / 32;         // 32-key sub-tiles per key block
  constexpr int TB = BLK * 128;        // bytes of one K or V tile
  constexpr int CPT = (BLK * 8) / NT;  // 16-byte chunks per thread per tile
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * 2 * TB];
  constexpr int CB = 1024;
  __shared__ int colbuf[CB];

  const Dims& d = a.d;
  const int r = head_sync_row(blockIdx.x, d.nb);
  if (r < 0) return;
  if constexpr (!F16) {
    if (a.redo && a.redo[r] == 0) return;
  }
  const int bh = r / d.nb, i = r - bh * d.nb;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 31, hh = lane >> 5;
  const size_t hoff = (size_t)bh * d.N * 64;
  const __bf16* Q = a.q + hoff;
  const unsigned char* Kb = F16 ? reinterpret_cast<const unsigned char*>(a.kh + hoff)
                                : reinterpret_cast<const unsigned char*>(a.k + hoff);
  const unsigned char* Vb = reinterpret_cast<const unsigned char*>(a.v + hoff);
  const int beg = a.row_ptr[r], end = a.row_ptr[r + 1];
  const int qrow = i * BLK + 32 * w + n;
  const float c2 = d.scale * 1.4426950408889634f;

  // B operand of S^T = K Q^T: column n = query, k-slots 8*hh.. = head dims.
  typedef std::conditional_t<F16, f16x8, bf16x8> qvec;
  qvec qf[4];
  int bad = 0;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const bf16x8 qb = *reinterpret_cast<const bf16x8*>(Q + (size_t)qrow * 64 + 16 * ks + 8 * hh);
    if constexpr (F16) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float f = (float)qb[e] * c2;
        bad |= !(fabsf(f) < kF16FormMax);
        qf[ks][e] = (_Float16)f;
      }
    } else {
      qf[ks] = qb;
    }
  }

  // Key row that A-operand lane row m reads: pi(m) with m = 8a + 4h + j maps to
  // 16(a/2) + 8h + 4(a%2) + j, so accumulator register x of lane l holds key
  // 16(x/8) + 8(l/32) + x%8 of the 32-key sub-tile.
  const int pim = key_perm(n);

  unsigned voff[CPT];
#pragma unroll
  for (int s3 = 0; s3 < CPT; ++s3) {
    const int q = NT * s3 + tid;
    const int row = q >> 3, pc = q & 7;
    voff[s3] = (unsigned)(row * 128 + ((pc ^ swz(row)) << 4));
  }
  const unsigned lds0 = (unsigned)(uintptr_t)smem + __builtin_amdgcn_readfirstlane(w) * 1024;
  auto dma = [&](int buf, int j) {
    const unsigned char* kt = Kb + (size_t)j * TB;
    const unsigned char* vt = Vb + (size_t)j * TB;
    const unsigned kb = lds0 + buf * 2 * TB;
#pragma unroll
    for (int s3 = 0; s3 < CPT; ++s3) {
      dma16(kt, voff[s3], kb + s3 * NT * 16);
      dma16(vt, voff[s3], kb + TB + s3 * NT * 16);
    }
  };

  // Lane-constant parts of the transposing V read: within each 16-lane group g,
  // lane jj fetches 4 head dims of key row 8*(g/2) + jj/4 (+4 for the upper half).
  const int g16 = lane >> 4, jj = lane & 15;
  const int vrow0 = 8 * (g16 >> 1) + (jj >> 2);
  const int vbyte = 32 * (g16 & 1) + 8 * (jj & 3);

  const int nt = end - beg;
  // entry x: the next tile's block (for its copy) and this tile's real-key count
  auto entry = [&](int x) {
    const int c = a.col_idx[beg + x];
    const int cn = x + 1 < nt ? a.col_idx[beg + x + 1] : 0;
    return (cn << 7) | (block_vlen(d, c) - 1);
  };
  for (int x = tid; x < min(nt, CB); x += NT) colbuf[x] = entry(x);

  if constexpr (F16) {
    // The fp16 form needs every scaled query of the block and every value of
    // every listed key block below kF16FormMax in magnitude; otherwise the row
    // is left to the bf16 form.
    for (int x = tid; x < nt; x += NT) bad |= a.kbad[(size_t)bh * d.nb + a.col_idx[beg + x]];
    __shared__ int vote[NT / 64];
    const bool wave_bad = __ballot(bad) != 0ull;
    if (lane == 0) vote[w] = wave_bad;
    __syncthreads();
    int any = 0;
#pragma unroll
    for (int q = 0; q < NT / 64; ++q) any |= vote[q];
    any = __builtin_amdgcn_readfirstlane(any);
    if (tid == 0) a.redo[r] = any != 0;
    if (any) return;
  }

  f32x16 oacc[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int x = 0; x < 16; ++x) oacc[mt][x] = 0.f;
  // m_run: the reference maximum in the product's units (raw <q,k> for bf16,
  // base-2 logits for fp16); sc converts them to base-2 units.
  float m_run = -INFINITY, l_run = 0.f;
  const float sc = F16 ? 1.f : c2;
  f32x16 cinit;   // fp16 form: the start -m of every score accumulator
#pragma unroll
  for (int x = 0; x < 16; ++x) cinit[x] = -m_run;

  if (nt > 0) dma(0, a.col_idx[beg]);

  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};

  for (int it = beg; it < end; ++it) {
    const int jt = it - beg;
    const int buf = jt & 1;
    wait_dma();
    __syncthreads();
    if ((jt & (CB / 2 - 1)) == 0 && jt > 0 && jt + CB / 2 < nt)
      for (int x = jt + CB / 2 + tid; x < min(nt, jt + CB); x += NT) colbuf[x & (CB - 1)] = entry(x);
    const int ecur = __builtin_amdgcn_readfirstlane(colbuf[jt & (CB - 1)]);
    if (it + 1 < end) dma(buf ^ 1, ecur >> 7);
    const unsigned char* kb = smem + buf * 2 * TB;
    const unsigned char* vb = kb + TB;
    const int vlen = (ecur & 127) + 1;

    // Scores of the tile; SHIFTED (fp16 form only): accumulators start at -m.
    auto scores = [&](f32x16 (&s)[KT], auto shifted_tag) {
      constexpr bool SHIFTED = decltype(shifted_tag)::value;
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        const int row = 32 * t + pim;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const unsigned char* p = kb + row * 128 + (((2 * ks + hh) ^ swz(row)) << 4);
          f32x16 c;
          if (ks == 0) {
#pragma unroll
            for (int x = 0; x < 16; ++x) c[x] = 0.f;
            if constexpr (SHIFTED) c = cinit;
          } else {
            c = s[t];
          }
          if constexpr (F16)
            s[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(*reinterpret_cast<const f16x8*>(p),
                                                          qf[ks], c, 0, 0, 0);
          else
            s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(p),
                                                           qf[ks], c, 0, 0, 0);
        }
      }
      if (vlen < BLK) {
        // the real keys are a prefix: sub-tiles past it are masked whole, and
        // only the one that straddles its end compares key by key
#pragma unroll
        for (int t = 0; t < KT; ++t) {
          if (32 * t >= vlen) {
#pragma unroll
            for (int x = 0; x < 16; ++x) s[t][x] = -INFINITY;
          } else if (32 * t + 32 > vlen) {
#pragma unroll
            for (int x = 0; x < 16; ++x) {
              const int key = 32 * t + 16 * (x >> 3) + 8 * hh + (x & 7);
              if (key >= vlen) s[t][x] = -INFINITY;
            }
          }
        }
      }
    };
    f32x16 s[KT];

    bf16x8 pb[KT][2];
    // P and its row sum: from shifted scores P = exp2(s), else exp2(s sc - m sc).
    auto soft = [&](const f32x16 (&s)[KT], auto shifted_tag) {
      constexpr bool SHIFTED = decltype(shifted_tag)::value;
      const float mb = m_run * sc;
      float ps4[4] = {0.f, 0.f, 0.f, 0.f};   // four independent sum chains
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          float pf[8];
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            const float z = s[t][8 * e + x];
            pf[x] = __builtin_amdgcn_exp2f(SHIFTED ? z : (F16 ? z - mb : fmaf(z, sc, -mb)));
          }
          const bf16x8 pv = {(__bf16)pf[0], (__bf16)pf[1], (__bf16)pf[2], (__bf16)pf[3],
                             (__bf16)pf[4], (__bf16)pf[5], (__bf16)pf[6], (__bf16)pf[7]};
          pb[t][e] = pv;
          ps4[0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pv, pv, 0, 1), ones, ps4[0], false);
          ps4[1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pv, pv, 2, 3), ones, ps4[1], false);
          ps4[2] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pv, pv, 4, 5), ones, ps4[2], false);
          ps4[3] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pv, pv, 6, 7), ones, ps4[3], false);
        }
      const float psum = (ps4[0] + ps4[1]) + (ps4[2] + ps4[3]);
      const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(psum), __float_as_uint(psum),
                                                       false, false);
      return __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
    };
    // The reference m stays while every P of the row is at most 2^64 (far from
    // the fp32 and bf16 range limits). A row whose sum passes that moves m to
    // the maximum of this tile's scores, recomputed from the K tile still in
    // LDS. The first tile, which has no reference yet (m = -inf), takes that
    // path directly.
    float psum = INFINITY;
    if (jt > 0) {
      scores(s, std::integral_constant<bool, F16>{});
      psum = soft(s, std::integral_constant<bool, F16>{});
    }
    if (__ballot(!(psum <= 1.8446744e19f))) {
      const bool big = !(psum <= 1.8446744e19f);
      scores(s, std::false_type{});
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int x = 0; x < 16; ++x) mx = fmaxf(mx, s[t][x]);
      const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                       false, false);
      mx = fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
      const float m_new = big ? fmaxf(m_run, mx) : m_run;
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * sc);
      l_run *= alpha;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int x = 0; x < 16; ++x) oacc[mt][x] *= alpha;
      m_run = m_new;
      if constexpr (F16) {
#pragma unroll
        for (int x = 0; x < 16; ++x) cinit[x] = -m_run;
      }
      psum = soft(s, std::false_type{});
    }
    l_run += psum;

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
  }
  wait_dma();

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
  // natural-log units: m_run * scale (bf16 form) or m_run * ln 2 (base-2 logits)
  const float mnat = F16 ? m_run * 0.6931471805599453f : m_run * d.scale;
  if (a.lse && hh == 0) a.lse[(size_t)bh * d.N + qrow] = any ? mnat + logf(l_run) : -INFINITY;
}

// Parts of the workspace: the fp16 copy of K, then a range flag per (b, h, key
// block), then a fallback flag per row (each part 256-byte aligned).
struct AttnWs {
  _Float16* kh;
  int32_t* kbad;
  int32_t* redo;
};
static AttnWs attn_ws(const Dims& d, void* ws) {
  unsigned char* p = static_cast<unsigned char*>(ws);
  AttnWs w;
  w.kh = reinterpret_cast<_Float16*>(p);
  p += align256((size_t)d.B * d.H * d.N * 64 * 2);
  w.kbad = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)d.rows * 4);
  w.redo = reinterpret_cast<int32_t*>(p);
  return w;
}

hipError_t launch_attn_prepare(const Dims& d, const void* k, void* ws, hipStream_t s) {
  const AttnWs w = attn_ws(d, ws);
  if (d.blk == 128)
    hipLaunchKernelGGL(k_k_to_f16<128>, dim3(d.rows), dim3(256), 0, s, (const __bf16*)k, w.kh,
                       w.kbad);
  else
    hipLaunchKernelGGL(k_k_to_f16<64>, dim3(d.rows), dim3(256), 0, s, (const __bf16*)k, w.kh,
                       w.kbad);
  return hipGetLastError();
}

template <int BLK>
static hipError_t launch_blk(const Dims& d, AttnArgs a, void* ws, bool k_ready, hipStream_t s) {
  const dim3 grid(head_sync_grid(d)), block(BLK * 2);
  if (ws) {
    const AttnWs w = attn_ws(d, ws);
    a.kh = w.kh;
    a.kbad = w.kbad;
    a.redo = w.redo;
    if (!k_ready) {
      const hipError_t e = launch_attn_prepare(d, a.k, ws, s);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((k_attn_bf16<BLK, true>), grid, block, 0, s, a);
  }
  // all rows without a workspace; else only the rows the fp16 form left over
  hipLaunchKernelGGL((k_attn_bf16<BLK, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attn_bf16(const Dims& d, const void* q, const void* k, const void* v,
                            const int32_t* row_ptr, const int32_t* col_idx, void* o,
                            float* lse, void* ws, hipStream_t s, bool k_ready) {
  AttnArgs a{d, (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, row_ptr, col_idx,
             (__bf16*)o, lse, nullptr, nullptr, nullptr};
  return d.blk == 128 ? launch_blk<128>(d, a, ws, k_ready, s)
                      : launch_blk<64>(d, a, ws, k_ready, s);
}

}  // namespace bsgm
