// C-ABI host layer: argument validation, workspace layout, dispatch to the
// kernel launchers. Everything is enqueued on the caller's stream; nothing is
// allocated and nothing synchronises.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/bsgm.h"
#include "internal.h"
#include "pooled.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return BSGM_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(BSGM_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Validates a layout and fills the kernel view. Returns BSGM_OK or an error.
int check_layout(const bsgm_layout* L, bsgm::Dims* d) {
  if (!L) return fail(BSGM_E_ARG, "layout is NULL");
  if (L->batch < 1 || L->heads < 1 || L->frames < 1 || L->frame_len < 1)
    return fail(BSGM_E_ARG, "batch, heads, frames and frame_len must be >= 1");
  if (L->frame_valid < 1 || L->frame_valid > L->frame_len)
    return fail(BSGM_E_ARG, "frame_valid must be in [1, frame_len]");
  if (!(std::isfinite(L->scale) && L->scale > 0.f))
    return fail(BSGM_E_ARG, "scale must be finite and > 0");
  if (L->dtype != BSGM_F32 && L->dtype != BSGM_BF16)
    return fail(BSGM_E_ARG, "dtype must be BSGM_F32 or BSGM_BF16");
  if (L->head_dim != 64) return fail(BSGM_E_UNSUPPORTED, "head_dim must be 64 (got %d)", L->head_dim);
  if (L->block != 64 && L->block != 128)
    return fail(BSGM_E_UNSUPPORTED, "block must be 64 or 128 (got %d)", L->block);
  if (L->frame_len % L->block != 0)
    return fail(BSGM_E_UNSUPPORTED, "frame_len (%d) must be a multiple of block (%d)", L->frame_len,
                L->block);
  if (L->frame_len - L->frame_valid >= L->block)
    return fail(BSGM_E_UNSUPPORTED,
                "padding per frame (%d) must be shorter than a block (%d): no empty blocks",
                L->frame_len - L->frame_valid, L->block);
  if (L->heads > bsgm::kMaxHeads)
    return fail(BSGM_E_UNSUPPORTED, "heads must be <= %d", bsgm::kMaxHeads);
  const long long N = (long long)L->frames * L->frame_len;
  const long long nb = N / L->block;
  const long long rows = (long long)L->batch * L->heads * nb;
  if (N > (1LL << 30) || rows >= (1LL << 31) - 1)
    return fail(BSGM_E_UNSUPPORTED, "layout too large (tokens %lld, rows %lld)", N, rows);
  d->B = L->batch;
  d->H = L->heads;
  d->D = L->head_dim;
  d->F = L->frames;
  d->L = L->frame_len;
  d->Lv = L->frame_valid;
  d->blk = L->block;
  d->N = (int)N;
  d->nb = (int)nb;
  d->rows = (int)rows;
  d->scale = L->scale;
  return BSGM_OK;
}

using bsgm::align256;

struct WsLayout {
  size_t qbar, kbar, counts, bitmask, stats, mz, qsplit, vbar, fac, mhat, pdem, pexe, total;
};

int vasc_pairs(const bsgm::Dims& d) { return (d.nb + 1) / 2; }

// Workspace of the one-launch selection: its synchronisation words first (the
// part that must be zero), then the pooled Q and K.
struct FusedWs {
  size_t sync, qbar, kbar, total;
};

FusedWs fused_ws_layout(const bsgm::Dims& d) {
  FusedWs w{};
  const size_t pooled = (size_t)d.rows * 64 * sizeof(float);
  w.sync = 0;
  w.qbar = align256(bsgm::fused_sync_words(d) * sizeof(int32_t));
  w.kbar = w.qbar + align256(pooled);
  w.total = w.kbar + align256(pooled);
  return w;
}

WsLayout ws_layout(const bsgm::Dims& d, int mode) {
  WsLayout w{};
  const size_t pooled = (size_t)d.rows * 64 * sizeof(float);
  size_t off = 0;
  w.qbar = off;
  off += align256(pooled);
  if (mode == BSGM_SEL_TOPK || mode == BSGM_SEL_CDF || mode == BSGM_SEL_VASC) {
    w.kbar = off;
    off += align256(pooled);
  }
  if (mode == BSGM_SEL_VASC) {
    const size_t np = (size_t)vasc_pairs(d);
    w.vbar = off;
    off += align256(pooled);
    w.fac = off;
    off += align256((size_t)d.B * d.H * np * sizeof(float));
    w.mhat = off;
    off += align256((size_t)d.B * d.H * np * sizeof(float));
    w.pdem = off;
    off += align256((size_t)d.rows * np * sizeof(float));
    w.pexe = off;
    off += align256((size_t)d.rows * np * sizeof(float));
  }
  if (mode == BSGM_SEL_DRIFT) {
    w.stats = off;
    off += align256((size_t)d.rows * d.nb * 2 * sizeof(float));
    w.mz = off;
    off += align256((size_t)d.rows * 2 * sizeof(float));
    w.qsplit = off;   // bf16 hi, mid, lo terms of qbar
    off += align256((size_t)d.rows * 3 * 64 * 2);
  }
  if (mode == BSGM_SEL_CDF) {
    w.counts = off;
    off += align256((size_t)d.rows * sizeof(int32_t));
    w.bitmask = off;
    off += align256((size_t)d.rows * ((d.nb + 31) / 32) * sizeof(uint32_t));
  }
  w.total = off;
  return w;
}

// Workspace of the streamed (expanded-form) re-rank drift selection. The
// squared scores and the per-round dot products reuse the statistics' bytes,
// which are dead once (M_i, Z_i) are formed.
struct StreamWs {
  size_t qbar, qsplit, stats, mz, obar, part, rsplit, jsq, jbest, m0, m1, best, total;
};

StreamWs stream_ws_layout(const bsgm::Dims& d) {
  StreamWs w{};
  const size_t rows = (size_t)d.rows, words = (size_t)((d.nb + 31) / 32);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  w.qbar = take(rows * 64 * sizeof(float));
  w.qsplit = take(rows * 3 * 64 * 2);
  w.stats = take(rows * d.nb * 2 * sizeof(float));   // later: ||c||^2, then <r, c>
  w.mz = take(rows * 2 * sizeof(float));
  w.obar = take(rows * 64 * sizeof(float));
  w.part = take(rows * bsgm::drift_round_groups_max(d) * 64 * sizeof(float));
  w.rsplit = take(rows * 3 * 64 * 2);
  w.jsq = take(rows * sizeof(float));
  w.jbest = take(rows * sizeof(float));
  w.m0 = take(rows * words * 4);
  w.m1 = take(rows * words * 4);
  w.best = take(rows * words * 4);
  w.total = off;
  return w;
}

// Checks the per-head budgets and fills the closed-form CSR offsets.
int check_budget(const bsgm::Dims& d, const bsgm_select_params* P, bsgm::HeadBudget* hb) {
  if (!P) return fail(BSGM_E_ARG, "params is NULL");
  if (!P->keep_per_head) return fail(BSGM_E_ARG, "keep_per_head is NULL");
  const int nforced = P->force_frame_first_block ? d.F : 0;
  long long off = 0;
  for (int h = 0; h < d.H; ++h) {
    const int k = P->keep_per_head[h];
    if (k < 1 || k > d.nb)
      return fail(BSGM_E_ARG, "keep_per_head[%d] = %d outside [1, %d]", h, k, d.nb);
    if (k < nforced)
      return fail(BSGM_E_ARG, "keep_per_head[%d] = %d is below the %d forced blocks", h, k, nforced);
    hb->keep[h] = k;
    hb->head_off[h] = off;
    off += (long long)d.nb * k;
  }
  hb->per_batch = off;
  return BSGM_OK;
}

// Checks of the TOPK / CDF arguments shared by the pooled selection entry points.
int check_pooled_select(const bsgm::Dims& d, const bsgm_select_params* params, const void* q,
                        const void* k) {
  if (!q || !k) return fail(BSGM_E_ARG, "TOPK and CDF need q and k");
  if (params->mode == BSGM_SEL_CDF && !(params->cdf_tau > 0.f && params->cdf_tau <= 1.f))
    return fail(BSGM_E_ARG, "cdf_tau must be in (0, 1]");
  if (d.nb > bsgm::kSelectMaxBlocks)
    return fail(BSGM_E_UNSUPPORTED, "pooled selection supports at most %d blocks per row",
                bsgm::kSelectMaxBlocks);
  return BSGM_OK;
}

// Pools Q and K into the workspace and selects (TOPK or CDF) from the means.
int run_pooled_select(const bsgm::Dims& d, const bsgm::HeadBudget& hb, int dtype,
                      const bsgm_select_params* params, const void* q, const void* k,
                      int32_t* row_ptr, int32_t* col_idx, float* row_stat, float* scores_out,
                      void* ws, const WsLayout& w, hipStream_t s) {
  const int mode = params->mode;
  char* base = static_cast<char*>(ws);
  float* qbar = reinterpret_cast<float*>(base + w.qbar);
  float* kbar = reinterpret_cast<float*>(base + w.kbar);
  int32_t* counts = mode == BSGM_SEL_CDF ? reinterpret_cast<int32_t*>(base + w.counts) : nullptr;
  uint32_t* bitmask =
      mode == BSGM_SEL_CDF ? reinterpret_cast<uint32_t*>(base + w.bitmask) : nullptr;
  const void* xs[2] = {q, k};
  float* means[2] = {qbar, kbar};
  hipError_t e = bsgm::launch_pool_n(d, dtype, 2, xs, means, s);
  if (e != hipSuccess) return hip_fail(e, "pool launch");
  e = bsgm::launch_select_pooled(d, hb, mode, params->cdf_tau,
                                 params->force_frame_first_block ? 1 : 0, qbar, kbar, row_ptr,
                                 col_idx, row_stat, scores_out, counts, bitmask, s);
  if (e != hipSuccess) return hip_fail(e, "select launch");
  return ok();
}

}  // namespace

extern "C" {

int32_t bsgm_version(void) { return 10600; }

const char* bsgm_last_error(void) { return g_err.c_str(); }

size_t bsgm_workspace_bytes(const bsgm_layout* layout, int32_t mode) {
  bsgm::Dims d;
  if (check_layout(layout, &d) != BSGM_OK) return 0;
  if (mode != BSGM_SEL_TOPK && mode != BSGM_SEL_CDF && mode != BSGM_SEL_DRIFT &&
      mode != BSGM_SEL_VASC) {
    fail(BSGM_E_ARG, "unknown selection mode %d", mode);
    return 0;
  }
  ok();
  return ws_layout(d, mode).total;
}

int64_t bsgm_col_capacity(const bsgm_layout* layout, const bsgm_select_params* params) {
  bsgm::Dims d;
  if (check_layout(layout, &d) != BSGM_OK) return -1;
  bsgm::HeadBudget hb;
  if (check_budget(d, params, &hb) != BSGM_OK) return -1;
  ok();
  return (int64_t)d.B * hb.per_batch;
}

int bsgm_pool_blocks(const bsgm_layout* layout, const void* x, float* mean, void* stream) {
  bsgm::Dims d;
  int st = check_layout(layout, &d);
  if (st != BSGM_OK) return st;
  if (!x || !mean) return fail(BSGM_E_ARG, "x and mean must be non-NULL");
  hipError_t e = bsgm::launch_pool(d, layout->dtype, x, mean, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "pool launch");
  return ok();
}

int bsgm_pool_blocks2(const bsgm_layout* layout, const void* x0, float* mean0, const void* x1,
                      float* mean1, void* stream) {
  bsgm::Dims d;
  int st = check_layout(layout, &d);
  if (st != BSGM_OK) return st;
  if (!x0 || !mean0 || !x1 || !mean1) return fail(BSGM_E_ARG, "x0, mean0, x1 and mean1 must be non-NULL");
  const void* xs[2] = {x0, x1};
  float* means[2] = {mean0, mean1};
  hipError_t e = bsgm::launch_pool_n(d, layout->dtype, 2, xs, means, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "pool launch");
  return ok();
}

int bsgm_drift_scores(const bsgm_layout* layout, const void* q, const void* k, const void* v,
                      float* contrib, float* score, float* zmass, void* ws, size_t ws_bytes,
                      void* stream) {
  bsgm::Dims d;
  int st = check_layout(layout, &d);
  if (st != BSGM_OK) return st;
  if (!q || !k || !v || !contrib || !score || !ws)
    return fail(BSGM_E_ARG, "q, k, v, contrib, score and ws must be non-NULL");
  const WsLayout w = ws_layout(d, BSGM_SEL_DRIFT);
  if (ws_bytes < w.total)
    return fail(BSGM_E_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, w.total);
  float* qbar = reinterpret_cast<float*>(static_cast<char*>(ws) + w.qbar);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = bsgm::launch_pool(d, layout->dtype, q, qbar, s);
  if (e != hipSuccess) return hip_fail(e, "pool launch");
  if (layout->dtype == BSGM_BF16) {
    char* base = static_cast<char*>(ws);
    e = bsgm::launch_drift_contrib_bf16(d, qbar, base + w.qsplit, k, v,
                                        reinterpret_cast<float2*>(base + w.stats),
                                        reinterpret_cast<float2*>(base + w.mz), contrib, score,
                                        zmass, s);
  } else {
    e = bsgm::launch_drift_contrib(d, layout->dtype, qbar, k, v, contrib, score, zmass, s);
  }
  if (e != hipSuccess) return hip_fail(e, "drift launch");
  return ok();
}

size_t bsgm_drift_streamed_workspace_bytes(const bsgm_layout* layout) {
  bsgm::Dims d;
  if (check_layout(layout, &d) != BSGM_OK) return 0;
  ok();
  return stream_ws_layout(d).total;
}

int bsgm_select_drift_streamed(const bsgm_layout* layout, const bsgm_select_params* params,
                               const void* q, const void* k, const void* v, int32_t* row_ptr,
                               int32_t* col_idx, int64_t col_capacity, float* row_stat,
                               int32_t* set_log, void* ws, size_t ws_bytes, void* stream) {
  bsgm::Dims d;
  int st = check_layout(layout, &d);
  if (st != BSGM_OK) return st;
  bsgm::HeadBudget hb;
  st = check_budget(d, params, &hb);
  if (st != BSGM_OK) return st;
  if (params->mode != BSGM_SEL_DRIFT)
    return fail(BSGM_E_ARG, "streamed drift selection takes mode BSGM_SEL_DRIFT (got %d)",
                params->mode);
  if (params->restoration != BSGM_RESTORE_RERANK &&
      params->restoration != BSGM_RESTORE_RERANK_TRACK_BEST)
    return fail(BSGM_E_UNSUPPORTED, "streamed drift selection takes the re-rank restoration rules");
  if (params->drift_objective != BSGM_DRIFT_DROPPED_SUM)
    return fail(BSGM_E_UNSUPPORTED, "streamed drift selection takes the dropped-sum objective");
  if (params->swap_rounds < 0) return fail(BSGM_E_ARG, "swap_rounds must be >= 0");
  if (bsgm::drift_stream_step_lds(d.nb) > bsgm::kMaxRowLds)
    return fail(BSGM_E_UNSUPPORTED, "streamed drift selection: a row of %d blocks needs %zu bytes of LDS",
                d.nb, bsgm::drift_stream_step_lds(d.nb));
  if (!q || !k || !v || !row_ptr || !col_idx || !ws)
    return fail(BSGM_E_ARG, "q, k, v, row_ptr, col_idx and ws must be non-NULL");
  const long long need = (long long)d.B * hb.per_batch;
  if (need > 0x7FFFFFFFLL)
    return fail(BSGM_E_UNSUPPORTED, "worst-case nnz %lld does not fit int32 CSR", need);
  if (col_capacity < need)
    return fail(BSGM_E_CAPACITY, "col_capacity %lld below worst-case nnz %lld",
                (long long)col_capacity, need);
  const StreamWs w = stream_ws_layout(d);
  if (ws_bytes < w.total)
    return fail(BSGM_E_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, w.total);
  char* base = static_cast<char*>(ws);
  float* qbar = reinterpret_cast<float*>(base + w.qbar);
  float2* mz = reinterpret_cast<float2*>(base + w.mz);
  float* sqnorm = reinterpret_cast<float*>(base + w.stats);
  float* dot = sqnorm + (size_t)d.rows * d.nb;
  float* part = reinterpret_cast<float*>(base + w.part);
  float* obar = reinterpret_cast<float*>(base + w.obar);
  float* jsq = reinterpret_cast<float*>(base + w.jsq);
  float* jbest = reinterpret_cast<float*>(base + w.jbest);
  uint32_t* masks[2] = {reinterpret_cast<uint32_t*>(base + w.m0),
                        reinterpret_cast<uint32_t*>(base + w.m1)};
  const bool tb = params->restoration == BSGM_RESTORE_RERANK_TRACK_BEST;
  uint32_t* best = tb ? reinterpret_cast<uint32_t*>(base + w.best) : nullptr;
  const int force = params->force_frame_first_block ? 1 : 0, R = params->swap_rounds;
  hipStream_t s = (hipStream_t)stream;

  // bf16 K and V take the matrix-core passes, fp32 the vector-ALU ones
  const bool f32 = layout->dtype == BSGM_F32;
  void* rsplit = base + w.rsplit;
  auto residual = [&](const uint32_t* kept, int vk, int round, uint32_t* bst) {
    return f32 ? bsgm::launch_drift_residual_f32(d, qbar, k, v, kept, vk, obar, part, rsplit, jsq,
                                                 bst, jbest, round, s)
               : bsgm::launch_drift_residual_bf16(d, base + w.qsplit, k, v, mz, kept, vk, obar,
                                                  part, rsplit, jsq, bst, jbest, round, s);
  };
  auto dots = [&]() {
    return f32 ? bsgm::launch_drift_dot_f32(d, qbar, rsplit, k, v, dot, s)
               : bsgm::launch_drift_dot_bf16(d, base + w.qsplit, rsplit, k, v, mz, dot, s);
  };

  hipError_t e = bsgm::launch_pool(d, layout->dtype, q, qbar, s);
  if (e != hipSuccess) return hip_fail(e, "pool launch");
  e = f32 ? bsgm::launch_drift_sqnorms_f32(d, qbar, k, v, sqnorm, s)
          : bsgm::launch_drift_sqnorms_bf16(d, qbar, base + w.qsplit, k, v,
                                            reinterpret_cast<float2*>(base + w.stats), mz, sqnorm,
                                            s);
  if (e != hipSuccess) return hip_fail(e, "drift score launch");
  e = bsgm::launch_drift_stream_step(d, hb, force, R, 0, sqnorm, nullptr, nullptr, masks[0],
                                     set_log, s);
  if (e != hipSuccess) return hip_fail(e, "drift step launch");
  // with fewer blocks kept than dropped in every head, r = o - (sum of the kept
  // blocks): the rounds then weigh the smaller set, after one pass for o
  bool via_kept = true;
  for (int h = 0; h < d.H; ++h) via_kept = via_kept && hb.keep[h] < d.nb - hb.keep[h];
  if (via_kept && (R > 0 || tb || row_stat)) {
    e = residual(nullptr, 0, 0, nullptr);
    if (e != hipSuccess) return hip_fail(e, "drift total launch");
  }
  const int vk = via_kept ? 1 : 0;
  int c = 0;
  for (int round = 1; round <= R; ++round, c ^= 1) {
    e = residual(masks[c], vk, round - 1, best);
    if (e != hipSuccess) return hip_fail(e, "drift residual launch");
    e = dots();
    if (e != hipSuccess) return hip_fail(e, "drift dot launch");
    e = bsgm::launch_drift_stream_step(d, hb, force, R, round, sqnorm, dot, masks[c],
                                       masks[c ^ 1], set_log, s);
    if (e != hipSuccess) return hip_fail(e, "drift step launch");
  }
  // J of the last set: the track-best comparison and row_stat need it
  if (tb || row_stat) {
    e = residual(masks[c], vk, R, best);
    if (e != hipSuccess) return hip_fail(e, "drift residual launch");
  }
  e = bsgm::launch_drift_stream_emit(d, hb, tb ? best : masks[c], tb ? jbest : jsq, row_ptr,
                                     col_idx, row_stat, s);
  if (e != hipSuccess) return hip_fail(e, "drift emit launch");
  return ok();
}

size_t bsgm_special_rows_workspace_bytes(const bsgm_layout* layout, int32_t n_special) {
  bsgm::Dims d;
  if (check_layout(layout, &d) != BSGM_OK) return 0;
  if (n_special < 1 || n_special > d.Lv) {
    fail(BSGM_E_ARG, "n_special = %d outside [1, frame_valid = %d]", n_special, d.Lv);
    return 0;
  }
  ok();
  const bsgm::DenseRowsPlan p = bsgm::dense_rows_plan(d, n_special);
  return align256(p.po_bytes) + align256(p.pml_bytes);
}

int bsgm_special_rows_dense_fwd(const bsgm_layout* layout, const void* q, const void* k,
                                const void* v, int32_t n_special, void* o, float* lse, void* ws,
                                size_t ws_bytes, void* stream) {
  bsgm::Dims d;
  int st = check_layout(layout, &d);
  if (st != BSGM_OK) return st;
  if (layout->dtype != BSGM_BF16)
    return fail(BSGM_E_UNSUPPORTED, "special rows: dtype must be BSGM_BF16");
  if (!q || !k || !v || !o || !ws) return fail(BSGM_E_ARG, "q, k, v, o and ws must be non-NULL");
  if (n_special < 1 || n_special > d.Lv)
    return fail(BSGM_E_ARG, "n_special = %d outside [1, frame_valid = %d]", n_special, d.Lv);
  const bsgm::DenseRowsPlan p = bsgm::dense_rows_plan(d, n_special);
  const size_t need = align256(p.po_bytes) + align256(p.pml_bytes);
  if (ws_bytes < need) return fail(BSGM_E_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  hipError_t e = bsgm::launch_dense_rows(d, n_special, q, k, v, o, lse, ws, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "special rows launch");
  return ok();
}

int bsgm_select_blocks(const bsgm_layout* layout, const bsgm_select_params* params,
                       const void* q, const void* k, const float* contrib, const float* zmass,
                       int32_t* row_ptr,
                       int32_t* col_idx, int64_t col_capacity, float* row_stat,
                       float* scores_out, int32_t* swap_log, void* ws, size_t ws_bytes,
                       void* stream) {
  bsgm::Dims d;
  int st = check_layout(layout, &d);
  if (st != BSGM_OK) return st;
  bsgm::HeadBudget hb;
  st = check_budget(d, params, &hb);
  if (st != BSGM_OK) return st;
  const int mode = params->mode;
  if (mode == BSGM_SEL_VASC)
    return fail(BSGM_E_ARG, "VASC selection carries memory: use bsgm_vasc_select_blocks");
  if (mode != BSGM_SEL_TOPK && mode != BSGM_SEL_CDF && mode != BSGM_SEL_DRIFT)
    return fail(BSGM_E_ARG, "unknown selection mode %d", mode);
  if (!row_ptr || !col_idx) return fail(BSGM_E_ARG, "row_ptr and col_idx must be non-NULL");
  const long long need = (long long)d.B * hb.per_batch;
  if (need > 0x7FFFFFFFLL)
    return fail(BSGM_E_UNSUPPORTED, "worst-case nnz %lld does not fit int32 CSR", need);
  if (col_capacity < need)
    return fail(BSGM_E_CAPACITY, "col_capacity %lld below worst-case nnz %lld",
                (long long)col_capacity, need);
  hipStream_t s = (hipStream_t)stream;
  if (mode == BSGM_SEL_DRIFT) {
    if (!contrib) return fail(BSGM_E_ARG, "DRIFT needs contrib");
    if (params->swap_rounds < 0) return fail(BSGM_E_ARG, "swap_rounds must be >= 0");
    if (params->drift_objective != BSGM_DRIFT_DROPPED_SUM &&
        params->drift_objective != BSGM_DRIFT_RENORMALISED)
      return fail(BSGM_E_ARG, "unknown drift objective %d", params->drift_objective);
    if (params->drift_objective == BSGM_DRIFT_RENORMALISED && !zmass)
      return fail(BSGM_E_ARG, "the renormalised drift objective needs zmass");
    if (params->restoration != BSGM_RESTORE_BEST_SWAP &&
        params->restoration != BSGM_RESTORE_RERANK &&
        params->restoration != BSGM_RESTORE_RERANK_TRACK_BEST)
      return fail(BSGM_E_ARG, "unknown restoration rule %d", params->restoration);
    if (params->restoration != BSGM_RESTORE_BEST_SWAP) {
      if (params->drift_objective != BSGM_DRIFT_DROPPED_SUM)
        return fail(BSGM_E_UNSUPPORTED, "re-rank restoration takes the dropped-sum objective");
      if (bsgm::drift_rerank_lds(d.nb) > bsgm::kMaxRowLds)
        return fail(BSGM_E_UNSUPPORTED, "re-rank selection: a row of %d blocks needs %zu bytes of LDS",
                    d.nb, bsgm::drift_rerank_lds(d.nb));
      hipError_t e = bsgm::launch_select_drift_rerank(
          d, hb, params->force_frame_first_block ? 1 : 0, params->swap_rounds,
          params->restoration == BSGM_RESTORE_RERANK_TRACK_BEST ? 1 : 0, contrib, row_ptr,
          col_idx, row_stat, swap_log, s);
      if (e != hipSuccess) return hip_fail(e, "drift re-rank select launch");
      return ok();
    }
    if (d.nb > bsgm::kDriftMaxBlocks)
      return fail(BSGM_E_UNSUPPORTED, "DRIFT supports at most %d blocks per row (got %d)",
                  bsgm::kDriftMaxBlocks, d.nb);
    if (swap_log && params->swap_rounds == 0) swap_log = nullptr;
    hipError_t e = bsgm::launch_select_drift(d, hb, params->force_frame_first_block ? 1 : 0,
                                             params->swap_rounds, params->drift_objective, contrib,
                                             zmass, row_ptr, col_idx, row_stat, swap_log, s);
    if (e != hipSuccess) return hip_fail(e, "drift select launch");
    return ok();
  }
  st = check_pooled_select(d, params, q, k);
  if (st != BSGM_OK) return st;
  if (!ws) return fail(BSGM_E_ARG, "ws must be non-NULL");
  const WsLayout w = ws_layout(d, mode);
  if (ws_bytes < w.total)
    return fail(BSGM_E_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, w.total);
  return run_pooled_select(d, hb, layout->dtype, params, q, k, row_ptr, col_idx, row_stat,
                           scores_out, ws, w, s);
}

int bsgm_select_blocks_pooled(const bsgm_layout* layout, const bsgm_select_params* params,
                              const float* qbar, const float* kbar, int32_t* row_ptr,
                              int32_t* col_idx, int64_t col_capacity, float* row_stat,
                              float* scores_out, void* ws, size_t ws_bytes, void* stream) {
  bsgm::Dims d;
  int st = check_layout(layout, &d);
  if (st != BSGM_OK) return st;
  bsgm::HeadBudget hb;
  st = check_budget(d, params, &hb);
  if (st != BSGM_OK) return st;
  const int mode = params->mode;
  if (mode != BSGM_SEL_TOPK && mode != BSGM_SEL_CDF)
    return fail(BSGM_E_UNSUPPORTED, "selection from pooled means takes TOPK or CDF (got mode %d)",
                mode);
  if (!qbar || !kbar) return fail(BSGM_E_ARG, "qbar and kbar must be non-NULL");
  if (!row_ptr || !col_idx) return fail(BSGM_E_ARG, "row_ptr and col_idx must be non-NULL");
  const long long need = (long long)d.B * hb.per_batch;
  if (need > 0x7FFFFFFFLL)
    return fail(BSGM_E_UNSUPPORTED, "worst-case nnz %lld does not fit int32 CSR", need);
  if (col_capacity < need)
    return fail(BSGM_E_CAPACITY, "col_capacity %lld below worst-case nnz %lld",
                (long long)col_capacity, need);
  if (mode == BSGM_SEL_CDF && !(params->cdf_tau > 0.f && params->cdf_tau <= 1.f))
    return fail(BSGM_E_ARG, "cdf_tau must be in (0, 1]");
  if (d.nb > bsgm::kSelectMaxBlocks)
    return fail(BSGM_E_UNSUPPORTED, "pooled selection supports at most %d blocks per row",
                bsgm::kSelectMaxBlocks);
  int32_t* counts = nullptr;
  uint32_t* bitmask = nullptr;
  if (mode == BSGM_SEL_CDF) {
    if (!ws) return fail(BSGM_E_ARG, "CDF needs ws");
    const WsLayout w = ws_layout(d, mode);
    if (ws_bytes < w.total)
      return fail(BSGM_E_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, w.total);
    counts = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + w.counts);
    bitmask = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + w.bitmask);
  }
  hipError_t e = bsgm::launch_select_pooled(d, hb, mode, params->cdf_tau,
                                            params->force_frame_first_block ? 1 : 0, qbar, kbar,
                                            row_ptr, col_idx, row_stat, scores_out, counts, bitmask,
                                            (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "select launch");
  return ok();
}

size_t bsgm_fused_workspace_bytes(const bsgm_layout* layout) {
  bsgm::Dims d;
  if (check_layout(layout, &d) != BSGM_OK) return 0;
  ok();
  return fused_ws_layout(d).total;
}

int bsgm_select_blocks_fused(const bsgm_layout* layout, const bsgm_select_params* params,
                             const void* q, const void* k, int32_t* row_ptr, int32_t* col_idx,
                             int64_t col_capacity, float* row_stat, float* scores_out, void* ws,
                             size_t ws_bytes, void* stream) {
  bsgm::Dims d;
  int st = check_layout(layout, &d);
  if (st != BSGM_OK) return st;
  bsgm::HeadBudget hb;
  st = check_budget(d, params, &hb);
  if (st != BSGM_OK) return st;
  if (params->mode != BSGM_SEL_TOPK)
    return fail(BSGM_E_UNSUPPORTED, "the one-launch selection takes TOPK only (got mode %d)",
                params->mode);
  if (!q || !k) return fail(BSGM_E_ARG, "q and k must be non-NULL");
  if (!row_ptr || !col_idx) return fail(BSGM_E_ARG, "row_ptr and col_idx must be non-NULL");
  const long long need = (long long)d.B * hb.per_batch;
  if (need > 0x7FFFFFFFLL)
    return fail(BSGM_E_UNSUPPORTED, "worst-case nnz %lld does not fit int32 CSR", need);
  if (col_capacity < need)
    return fail(BSGM_E_CAPACITY, "col_capacity %lld below worst-case nnz %lld",
                (long long)col_capacity, need);
  if (d.nb > bsgm::kSelectMaxBlocks)
    return fail(BSGM_E_UNSUPPORTED, "pooled selection supports at most %d blocks per row",
                bsgm::kSelectMaxBlocks);
  if (!ws) return fail(BSGM_E_ARG, "ws must be non-NULL");
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0)
    return fail(BSGM_E_ARG, "ws must be 256-byte aligned");
  const FusedWs w = fused_ws_layout(d);
  if (ws_bytes < w.total)
    return fail(BSGM_E_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, w.total);
  char* base = static_cast<char*>(ws);
  hipError_t e = bsgm::launch_select_fused(
      d, hb, layout->dtype, params->force_frame_first_block ? 1 : 0, q, k,
      reinterpret_cast<float*>(base + w.qbar), reinterpret_cast<float*>(base + w.kbar),
      reinterpret_cast<int32_t*>(base + w.sync), row_ptr, col_idx, row_stat, scores_out,
      (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "fused select launch");
  return ok();
}

int bsgm_vasc_select_blocks(const bsgm_layout* layout, const bsgm_select_params* params,
                            const void* q, const void* k, const void* v, float* memory,
                            int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                            float* row_stat, float* demand_out, void* ws, size_t ws_bytes,
                            void* stream) {
  bsgm::Dims d;
  int st = check_layout(layout, &d);
  if (st != BSGM_OK) return st;
  bsgm::HeadBudget hb;
  st = check_budget(d, params, &hb);
  if (st != BSGM_OK) return st;
  if (params->mode != BSGM_SEL_VASC)
    return fail(BSGM_E_ARG, "params->mode must be BSGM_SEL_VASC (got %d)", params->mode);
  if (!q || !k || !v || !memory || !row_ptr || !col_idx || !ws)
    return fail(BSGM_E_ARG, "q, k, v, memory, row_ptr, col_idx and ws must be non-NULL");
  const long long need = (long long)d.B * hb.per_batch;
  if (need > 0x7FFFFFFFLL)
    return fail(BSGM_E_UNSUPPORTED, "worst-case nnz %lld does not fit int32 CSR", need);
  if (col_capacity < need)
    return fail(BSGM_E_CAPACITY, "col_capacity %lld below worst-case nnz %lld",
                (long long)col_capacity, need);
  if (d.nb > bsgm::kSelectMaxBlocks)
    return fail(BSGM_E_UNSUPPORTED, "pooled selection supports at most %d blocks per row",
                bsgm::kSelectMaxBlocks);
  const WsLayout w = ws_layout(d, BSGM_SEL_VASC);
  if (ws_bytes < w.total)
    return fail(BSGM_E_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, w.total);
  char* base = static_cast<char*>(ws);
  float* qbar = reinterpret_cast<float*>(base + w.qbar);
  float* kbar = reinterpret_cast<float*>(base + w.kbar);
  float* vbar = reinterpret_cast<float*>(base + w.vbar);
  const int np = vasc_pairs(d);
  float* fac = reinterpret_cast<float*>(base + w.fac);
  float* mhat = reinterpret_cast<float*>(base + w.mhat);
  float* pdem = reinterpret_cast<float*>(base + w.pdem);
  float* pexe = reinterpret_cast<float*>(base + w.pexe);
  const bsgm::VascSel vs{np, fac, mhat, pdem, pexe, demand_out};
  hipStream_t s = (hipStream_t)stream;
  const void* xs[3] = {q, k, v};
  float* means[3] = {qbar, kbar, vbar};
  hipError_t e = bsgm::launch_pool_n(d, layout->dtype, 3, xs, means, s);
  if (e != hipSuccess) return hip_fail(e, "pool launch");
  e = bsgm::launch_vasc_prep(d, np, vbar, memory, fac, mhat, s);
  if (e != hipSuccess) return hip_fail(e, "vasc prep launch");
  e = bsgm::launch_select_pooled(d, hb, BSGM_SEL_VASC, 0.f, params->force_frame_first_block ? 1 : 0,
                                 qbar, kbar, row_ptr, col_idx, row_stat, nullptr, nullptr, nullptr,
                                 s, &vs);
  if (e != hipSuccess) return hip_fail(e, "vasc select launch");
  e = bsgm::launch_vasc_update(d, np, pdem, pexe, memory, s);
  if (e != hipSuccess) return hip_fail(e, "vasc memory launch");
  return ok();
}

size_t bsgm_attn_workspace_bytes(const bsgm_layout* layout) {
  bsgm::Dims d;
  if (check_layout(layout, &d) != BSGM_OK) return 0;
  ok();
  return layout->dtype == BSGM_BF16 ? bsgm::attn_workspace_bytes(d) : 0;
}

}  // extern "C"

namespace {

// Checks of an attention workspace (bf16 layouts): size and alignment, and
// presence when `required`.
int check_attn_ws(const bsgm::Dims& d, const void* ws, size_t ws_bytes, bool required) {
  if (!ws) return required ? fail(BSGM_E_ARG, "ws must be non-NULL") : BSGM_OK;
  if (ws_bytes < bsgm::attn_workspace_bytes(d))
    return fail(BSGM_E_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes,
                bsgm::attn_workspace_bytes(d));
  if (reinterpret_cast<uintptr_t>(ws) % 256)
    return fail(BSGM_E_ARG, "workspace must be 256-byte aligned");
  return BSGM_OK;
}

int attn_fwd(const bsgm_layout* layout, const void* q, const void* k, const void* v,
             const int32_t* row_ptr, const int32_t* col_idx, void* o, float* lse, void* ws,
             size_t ws_bytes, void* stream, bool k_ready) {
  bsgm::Dims d;
  int st = check_layout(layout, &d);
  if (st != BSGM_OK) return st;
  if (!q || !k || !v || !row_ptr || !col_idx || !o)
    return fail(BSGM_E_ARG, "q, k, v, row_ptr, col_idx and o must be non-NULL");
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (layout->dtype == BSGM_BF16) {
    st = check_attn_ws(d, ws, ws_bytes, k_ready);
    if (st != BSGM_OK) return st;
    e = bsgm::launch_attn_bf16(d, q, k, v, row_ptr, col_idx, o, lse, ws, s, k_ready);
  } else {
    e = bsgm::launch_attn_f32(d, q, k, v, row_ptr, col_idx, o, lse, s);
  }
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return ok();
}

}  // namespace

extern "C" {

int bsgm_sparse_attn_fwd(const bsgm_layout* layout, const void* q, const void* k, const void* v,
                         const int32_t* row_ptr, const int32_t* col_idx, void* o, float* lse,
                         void* ws, size_t ws_bytes, void* stream) {
  return attn_fwd(layout, q, k, v, row_ptr, col_idx, o, lse, ws, ws_bytes, stream, false);
}

int bsgm_attn_prepare(const bsgm_layout* layout, const void* k, void* ws, size_t ws_bytes,
                      void* stream) {
  bsgm::Dims d;
  int st = check_layout(layout, &d);
  if (st != BSGM_OK) return st;
  if (!k) return fail(BSGM_E_ARG, "k must be non-NULL");
  if (layout->dtype != BSGM_BF16) return ok();   // fp32 attention takes no workspace
  st = check_attn_ws(d, ws, ws_bytes, true);
  if (st != BSGM_OK) return st;
  const hipError_t e = bsgm::launch_attn_prepare(d, k, ws, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attention prepare launch");
  return ok();
}

int bsgm_sparse_attn_fwd_prepared(const bsgm_layout* layout, const void* q, const void* k,
                                  const void* v, const int32_t* row_ptr, const int32_t* col_idx,
                                  void* o, float* lse, void* ws, size_t ws_bytes, void* stream) {
  return attn_fwd(layout, q, k, v, row_ptr, col_idx, o, lse, ws, ws_bytes, stream, true);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Selection with a library-held scratch array (bsgm_select_blocks_noalloc).
//
// The pooled means (and the CDF counts and bitmask) live in `scratch`, one
// array per GPU that stays allocated until the process ends. Host code never
// passes `scratch` itself to a kernel or copy: in host code the name is a
// host-side stand-in, not the device array. Its device address is looked up
// once per device with hipGetSymbolAddress, with that device current, and
// kept in g_scratch_addr. Every call on a GPU shares that GPU's array, so calls
// that overlap in time on one GPU race; the selection writes every word it
// later reads, so nothing needs clearing between calls.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[BSGM_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kNoAllocScratchBytes = BSGM_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];

// Device address of this GPU's `scratch` (the current device's).
int scratch_addr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(BSGM_E_UNSUPPORTED, "device %d: the scratch table holds %d devices", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(BSGM_E_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return BSGM_OK;
}

}  // namespace

extern "C" {

int bsgm_select_blocks_noalloc(const bsgm_layout* layout, const bsgm_select_params* params,
                               const void* q, const void* k, int32_t* row_ptr, int32_t* col_idx,
                               int64_t col_capacity, float* row_stat, float* scores_out,
                               void* stream) {
  bsgm::Dims d;
  int st = check_layout(layout, &d);
  if (st != BSGM_OK) return st;
  bsgm::HeadBudget hb;
  st = check_budget(d, params, &hb);
  if (st != BSGM_OK) return st;
  const int mode = params->mode;
  if (mode != BSGM_SEL_TOPK && mode != BSGM_SEL_CDF)
    return fail(BSGM_E_UNSUPPORTED, "the scratch-array selection takes TOPK or CDF (got mode %d)",
                mode);
  if (!row_ptr || !col_idx) return fail(BSGM_E_ARG, "row_ptr and col_idx must be non-NULL");
  const long long need = (long long)d.B * hb.per_batch;
  if (need > 0x7FFFFFFFLL)
    return fail(BSGM_E_UNSUPPORTED, "worst-case nnz %lld does not fit int32 CSR", need);
  if (col_capacity < need)
    return fail(BSGM_E_CAPACITY, "col_capacity %lld below worst-case nnz %lld",
                (long long)col_capacity, need);
  st = check_pooled_select(d, params, q, k);
  if (st != BSGM_OK) return st;
  const WsLayout w = ws_layout(d, mode);
  if (w.total > kNoAllocScratchBytes)
    return fail(BSGM_E_WORKSPACE, "layout needs %zu bytes of scratch; the library's array holds %zu",
                w.total, kNoAllocScratchBytes);
  void* ws = nullptr;
  st = scratch_addr(&ws);
  if (st != BSGM_OK) return st;
  return run_pooled_select(d, hb, layout->dtype, params, q, k, row_ptr, col_idx, row_stat,
                           scores_out, ws, w, (hipStream_t)stream);
}

}  // extern "C"
