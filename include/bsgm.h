/*
 * bsgm.h - C ABI of the block-sparse global attention library for MI355X (gfx950).
 *
 * The library computes one global-attention layer of a multi-view geometry
 * transformer with block sparsity, in two stages joined by a block list:
 *
 *   1. selection: for every (batch, head, query block) pick the key blocks to
 *      execute, by pooled top-k, by a cumulative pooled-mass threshold under a
 *      per-head cap, or by residual-drift score with swap restoration;
 *   2. block-sparse attention forward over the selected blocks only.
 *
 * Sources (pages, by title):
 *   [ReSS] "ReSS: Residual-Restoring Sparse Attention for 3D Vision
 *          Transformers" (thelatestinai.com 2609.35593).
 *   [VASC] "VASC: Value-Aware Sparse Attention with Cross-Layer Memory for
 *          Efficient 3D Reconstruction" (paperlayer.ai 2610.01013v1 summary).
 *
 * Conventions shared by every entry point
 *   - Q, K, V, O are device tensors [batch, heads, N, head_dim], row-major,
 *     head_dim contiguous, N = frames * frame_len. Token f*frame_len + p is a
 *     real token iff p < frame_valid; the others are padding and are ignored
 *     by every pool, softmax and drift sum. Their contents must be finite
 *     (any finite values give the same results; a padding NaN or infinity in
 *     V reaches the outputs through a zero weight).
 *   - Blocks: block j covers tokens [j*block, (j+1)*block); Nb = N / block.
 *     Query and key blocks share the grid.
 *   - Block lists are CSR: row r = (b*heads + h)*Nb + i, row_ptr int32
 *     [batch*heads*Nb + 1], col_idx int32 key-block indices, strictly
 *     ascending within a row.
 *   - Ownership: the caller allocates every buffer (device memory for all
 *     tensors and the workspace, host memory only where stated). The library
 *     allocates nothing, keeps no state besides the per-thread error text,
 *     and never synchronises: all work is enqueued on `stream` (a
 *     hipStream_t; NULL means the default stream).
 *   - Errors: arguments are checked on the host before any launch; on error
 *     nothing is enqueued and a negative bsgm_status is returned, with text in
 *     bsgm_last_error(). A launch failure reported by HIP returns
 *     BSGM_E_HIP. Device-side contents (e.g. CSR indices passed to
 *     bsgm_sparse_attn_fwd) are not validated.
 *   - Supported: head_dim 64; block 64 or 128 dividing frame_len; at most one
 *     partially padded block per frame (frame_len - frame_valid < block);
 *     heads <= 128; dtype BSGM_BF16 (bf16 MFMA attention) or BSGM_F32.
 */
#ifndef BSGM_H
#define BSGM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BSGM_OK = 0,
  BSGM_E_ARG = -1,          /* null pointer or out-of-range argument            */
  BSGM_E_UNSUPPORTED = -2,  /* valid but not implemented (head_dim, block, ...) */
  BSGM_E_CAPACITY = -3,     /* col_capacity below the worst-case nnz            */
  BSGM_E_WORKSPACE = -4,    /* ws_bytes below bsgm_workspace_bytes()            */
  BSGM_E_HIP = -5           /* HIP reported an error at launch                  */
} bsgm_status;

typedef enum { BSGM_F32 = 0, BSGM_BF16 = 1 } bsgm_dtype;

typedef enum {
  BSGM_SEL_TOPK = 0,   /* fixed budget by pooled score                        */
  BSGM_SEL_CDF = 1,    /* cumulative pooled mass >= tau, capped per head      */
  BSGM_SEL_DRIFT = 2,  /* drift score + swap restoration at a fixed budget    */
  BSGM_SEL_VASC = 3    /* value-aware demand + pair memory (bsgm_vasc_select_blocks) */
} bsgm_sel_mode;

typedef struct {
  int32_t batch, heads, head_dim;
  int32_t frames, frame_len, frame_valid;
  int32_t block;
  int32_t dtype;   /* bsgm_dtype of Q, K, V and O */
  float scale;     /* softmax scale, normally 1/sqrt(head_dim) */
} bsgm_layout;

typedef enum {
  BSGM_DRIFT_DROPPED_SUM = 0,     /* J = || sum_{dropped} contrib ||                  */
  BSGM_DRIFT_RENORMALISED = 1     /* J = || sum_{kept} contrib / sum_{kept} zmass
                                         - sum_{all} contrib || (output shift)        */
} bsgm_drift_objective;

typedef enum {
  BSGM_RESTORE_BEST_SWAP = 0,         /* one best-improvement swap per round          */
  BSGM_RESTORE_RERANK = 1,            /* re-rank every block per round, keep the last */
  BSGM_RESTORE_RERANK_TRACK_BEST = 2  /* re-rank every block per round, keep the set
                                         of least J seen                            */
} bsgm_restoration;

typedef struct {
  int32_t mode;                   /* bsgm_sel_mode                                    */
  const int32_t* keep_per_head;   /* HOST array [heads]: kept blocks per query block
                                     (TOPK, DRIFT) or the cap (CDF); 1..Nb            */
  float cdf_tau;                  /* CDF only: threshold in (0, 1]                    */
  int32_t force_frame_first_block;/* keep the block holding token f*frame_len of every
                                     frame in every row; forced blocks count toward
                                     the budget                                       */
  int32_t swap_rounds;            /* DRIFT only: restoration rounds, >= 0             */
  int32_t drift_objective;        /* DRIFT only: bsgm_drift_objective                 */
  int32_t restoration;            /* DRIFT only: bsgm_restoration                     */
} bsgm_select_params;

/* Version of this ABI (major*10000 + minor*100 + patch). */
int32_t bsgm_version(void);

/* Text of the last error on the calling thread ("" if none). Valid until the
 * next call of this library on the same thread. */
const char* bsgm_last_error(void);

/* Device workspace that bsgm_select_blocks (TOPK, CDF), bsgm_drift_scores
 * (mode = BSGM_SEL_DRIFT) or bsgm_vasc_select_blocks (mode = BSGM_SEL_VASC)
 * needs for this layout; 0 if the layout is invalid (see bsgm_last_error).
 * bsgm_select_blocks in DRIFT mode needs none. */
size_t bsgm_workspace_bytes(const bsgm_layout* layout, int32_t mode);

/* Worst-case number of CSR entries: batch * Nb * sum_h keep_per_head[h];
 * -1 on invalid arguments. */
int64_t bsgm_col_capacity(const bsgm_layout* layout, const bsgm_select_params* params);

/* Block mean pool ([ReSS] Table S5, SpargeAttn row: selection on pooled
 * query/key inner products; [VASC] A.1: pooled query blocks index key/value
 * child blocks).
 *   x    device [B,H,N,D] of layout->dtype
 *   mean device float [B,H,Nb,D]: mean of x over the real tokens of each block.
 */
int bsgm_pool_blocks(const bsgm_layout* layout, const void* x, float* mean, void* stream);

/* Block mean pool of two tensors of one layout in a single launch, typically
 * the Q and K of a layer before selection from pooled means (same sources as
 * bsgm_pool_blocks). mean0 and mean1 receive exactly what two
 * bsgm_pool_blocks calls would write.
 *   x0, x1       device [B,H,N,D] of layout->dtype
 *   mean0, mean1 device float [B,H,Nb,D]; must not overlap each other or x0, x1
 * Returns BSGM_E_ARG if any pointer is NULL.
 */
int bsgm_pool_blocks2(const bsgm_layout* layout, const void* x0, float* mean0, const void* x1,
                      float* mean1, void* stream);

/* Drift contributions ([ReSS] abstract, Figs. 1-3: the shift that dropping a
 * key block leaves in what attention writes into the residual stream).
 * For pooled query block i (mean of Q over its real tokens) and every real key
 * token u: l = scale*<qbar_i, k_u>, e_u = exp(l - max_u l);
 *   contrib[b,h,i,j,:] = sum_{u in block j} e_u v_u / sum_u e_u   (float)
 *   score[b,h,i,j]     = || contrib[b,h,i,j,:] ||_2                (float)
 *   zmass[b,h,i,j]     = sum_{u in block j} e_u / sum_u e_u         (float)
 *   q, k, v  device [B,H,N,D] of layout->dtype
 *   contrib  device float [B,H,Nb,Nb,D], required
 *   score    device float [B,H,Nb,Nb], required
 *   zmass    device float [B,H,Nb,Nb] or NULL (needed by the renormalised
 *            drift objective of bsgm_select_blocks)
 *   ws       device, >= bsgm_workspace_bytes(layout, BSGM_SEL_DRIFT) bytes
 */
int bsgm_drift_scores(const bsgm_layout* layout, const void* q, const void* k, const void* v,
                      float* contrib, float* score, float* zmass, void* ws, size_t ws_bytes,
                      void* stream);

/* Block selection ([VASC] A.2: exact binary capacity per query; [ReSS]
 * Fig. 3(b): per-head budget; [ReSS] Table 2: the cumulative-threshold rule;
 * [VASC] 4.2: special-token key blocks always kept; selected lists go to the
 * sparse kernel as they are).
 * Priority order of a row: forced blocks (ascending), then the rest by score
 * descending, ties to the lower block index.
 *   TOPK : score = scale*<qbar_i, kbar_j>; keep the first keep_per_head[h].
 *   CDF  : P = softmax_j(score); keep the shortest prefix whose mass reaches
 *          cdf_tau (all blocks if it never does), at most keep_per_head[h],
 *          at least one and at least the forced blocks.
 *   DRIFT: score = ||contrib_ij||; start from the first keep_per_head[h]; then
 *          swap_rounds rounds of restoration ([ReSS] abstract and Fig. 3(c): the
 *          drop set is refined as a whole at a fixed budget), by `restoration`:
 *          BEST_SWAP: each round makes the single swap (restore a dropped block
 *          a, drop a kept non-forced block b) that minimises the drift J of the
 *          resulting set (ties: lower a, then lower b) if it lowers J, stopping
 *          otherwise. J is chosen by drift_objective:
 *          DROPPED_SUM  J = ||sum_{dropped} contrib||;
 *          RENORMALISED J = ||sum_{kept} contrib / sum_{kept} zmass - sum_{all} contrib||,
 *          the shift of the pooled query's attention output once the dropped
 *          blocks are removed and the kept weights renormalised ([ReSS] Fig. 3(a)).
 *          RERANK, RERANK_TRACK_BEST (DROPPED_SUM only, else BSGM_E_UNSUPPORTED):
 *          each round scores every block j against the residual r of the current
 *          drop set D, g_j = ||r_j + contrib_j||^2 - ||r_j||^2 with r_j = r minus
 *          contrib_j for j in D (else r), and keeps the forced blocks plus the
 *          highest g (ties: lower block), all blocks at once, for every one of the
 *          swap_rounds rounds. A round may raise J; TRACK_BEST returns the set of
 *          least J among the initial set and every round's set (ties: the
 *          earlier; [ReSS] Table S3), RERANK the last one. Rows of up to 19856
 *          blocks (the row's scores and kept flags sit in LDS; BEST_SWAP: at
 *          most 4096; above 512 the row is read from global memory in every
 *          pass instead of held on chip).
 *   q, k       device [B,H,N,D] (TOPK, CDF; may be NULL for DRIFT)
 *   contrib    device float [B,H,Nb,Nb,D] from bsgm_drift_scores (DRIFT only)
 *   zmass      device float [B,H,Nb,Nb] from bsgm_drift_scores (RENORMALISED only)
 *   row_ptr    device int32 [B*H*Nb + 1], written
 *   col_idx    device int32 [col_capacity], first row_ptr[last] entries written
 *   col_capacity >= bsgm_col_capacity(layout, params)
 *   row_stat   device float [B*H*Nb] or NULL: kept pooled mass sum_{kept} P
 *              (TOPK, CDF) or the final drift J under the objective (DRIFT)
 *   scores_out device float [B,H,Nb,Nb] or NULL: the pooled logits (TOPK, CDF)
 *   swap_log   device int32 or NULL (DRIFT). BEST_SWAP: [B*H*Nb, swap_rounds, 2],
 *              the (a, b) of each round, (-1, -1) once restoration has stopped.
 *              RERANK modes: [B*H*Nb, swap_rounds + 1, ceil(Nb / 32)], the kept
 *              set of the initial selection and of each round as bitmask words
 *              (bit j % 32 of word j / 32 set iff block j is kept)
 *   ws         device, >= bsgm_workspace_bytes(layout, mode) bytes
 */
int bsgm_select_blocks(const bsgm_layout* layout, const bsgm_select_params* params,
                       const void* q, const void* k, const float* contrib, const float* zmass,
                       int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                       float* row_stat, float* scores_out, int32_t* swap_log,
                       void* ws, size_t ws_bytes, void* stream);

/* Drift selection by re-rank rounds without the contributions ([ReSS]
 * Table 1: drift scoring with and without expansion, and its scoring memory).
 * The same selection as bsgm_select_blocks with mode DRIFT, objective
 * DROPPED_SUM and restoration RERANK or RERANK_TRACK_BEST, computed from Q,
 * K and V directly. A round's score expands as
 *   g_j = 2 <r, contrib_j> + ||contrib_j||^2   (j kept; minus for j dropped),
 *   <r, contrib_ij> = sum_{u in block j} e_u <v_u, r> / sum_u e_u,
 * so each round recomputes the residual r of its drop set (a weighted value
 * sum over the dropped blocks or, when every head keeps fewer blocks than it
 * drops, the total sum_j contrib_ij minus that over the kept blocks) and then
 * one scalar per (row, block) from the keys and values; the row statistics
 * (max and sum of exp) and the total are computed once.
 * Scoring memory is per (row, block) scalars, not [B,H,Nb,Nb,D] floats; the
 * cost is two passes over K and V per round.
 *   params     mode BSGM_SEL_DRIFT, keep_per_head, force_frame_first_block,
 *              swap_rounds (>= 0), drift_objective DROPPED_SUM, restoration
 *              RERANK or RERANK_TRACK_BEST
 *   q, k, v    device [B,H,N,D] of layout->dtype (bf16: the passes run on the
 *              matrix cores with fp32-accurate split operands; fp32: vector ALU)
 *   row_ptr, col_idx, col_capacity  as bsgm_select_blocks
 *   row_stat   device float [B*H*Nb] or NULL: the drift J of the returned set
 *   set_log    device int32 [B*H*Nb, swap_rounds + 1, ceil(Nb / 32)] or NULL:
 *              the kept set of the initial selection and of each round, as
 *              bsgm_select_blocks' swap_log in the re-rank modes
 *   ws         device, >= bsgm_drift_streamed_workspace_bytes(layout) bytes
 * Errors: BSGM_E_ARG for a NULL q, k, v, row_ptr, col_idx or ws, another mode,
 * or negative swap_rounds; BSGM_E_UNSUPPORTED for the best-swap rule or the
 * renormalised objective; BSGM_E_CAPACITY, BSGM_E_WORKSPACE as
 * bsgm_select_blocks, and BSGM_E_UNSUPPORTED for rows of more than 39716
 * blocks (the row's scores and kept flags sit in LDS).
 */
int bsgm_select_drift_streamed(const bsgm_layout* layout, const bsgm_select_params* params,
                               const void* q, const void* k, const void* v, int32_t* row_ptr,
                               int32_t* col_idx, int64_t col_capacity, float* row_stat,
                               int32_t* set_log, void* ws, size_t ws_bytes, void* stream);

/* Device workspace of bsgm_select_drift_streamed: about
 * B*H*Nb * (8*Nb + 1296 + 12*ceil(Nb/32)) bytes, plus min(16, Nb) x 64 floats
 * per row of partial residual sums; 0 if the layout is invalid. */
size_t bsgm_drift_streamed_workspace_bytes(const bsgm_layout* layout);

/* TOPK or CDF selection from pooled means the caller already holds (from
 * bsgm_pool_blocks of Q and of K): the second half of bsgm_select_blocks, with
 * the same results bit for bit when given the same means. A caller can thus
 * order other work between the pooling and the selection, for instance the
 * fp16 copy of K for the attention (bsgm_attn_prepare), which then overlaps
 * the selection instead of the pooling.
 *   params     mode BSGM_SEL_TOPK or BSGM_SEL_CDF (BSGM_E_UNSUPPORTED
 *              otherwise); the other fields as bsgm_select_blocks
 *   qbar, kbar device float [B,H,Nb,D], the block means of Q and K
 *   row_ptr, col_idx, col_capacity, row_stat, scores_out
 *              as bsgm_select_blocks
 *   ws         CDF: device, >= bsgm_workspace_bytes(layout, BSGM_SEL_CDF)
 *              bytes (its pooled-mean part is not used); TOPK: not used, may
 *              be NULL
 * Errors: BSGM_E_ARG for a NULL qbar, kbar, row_ptr or col_idx (or ws in CDF
 * mode) or a bad budget or cdf_tau; BSGM_E_CAPACITY, BSGM_E_WORKSPACE,
 * BSGM_E_UNSUPPORTED as bsgm_select_blocks; BSGM_E_HIP on a launch error.
 */
int bsgm_select_blocks_pooled(const bsgm_layout* layout, const bsgm_select_params* params,
                              const float* qbar, const float* kbar, int32_t* row_ptr,
                              int32_t* col_idx, int64_t col_capacity, float* row_stat,
                              float* scores_out, void* ws, size_t ws_bytes, void* stream);

/* TOPK selection with the pooling and the selection in one kernel launch
 * ([ReSS] Table 1: selection overhead with and without a fused kernel). The
 * result is bitwise that of bsgm_select_blocks in TOPK mode (same pooling and
 * selection arithmetic); the pooled means stay in the workspace. Inside the
 * launch each (batch, head) is pooled and then selected on one XCD of the GPU,
 * its selection starting once that head's pooling is done, while other heads
 * still pool.
 *   params     mode must be BSGM_SEL_TOPK (BSGM_E_UNSUPPORTED otherwise);
 *              keep_per_head and force_frame_first_block as bsgm_select_blocks
 *   q, k, row_ptr, col_idx, col_capacity, row_stat, scores_out
 *              as bsgm_select_blocks (TOPK)
 *   ws         device, >= bsgm_fused_workspace_bytes(layout) bytes, 256-byte
 *              aligned. Its first part holds synchronisation words that must
 *              be zero before the first call on this workspace (allocate it
 *              zeroed, or clear it once); every call leaves them zero again, so
 *              later calls need no clearing. Calls that share a workspace must
 *              not overlap in time (same stream, or ordered by events).
 * Errors: BSGM_E_ARG for a NULL q, k, row_ptr, col_idx or ws, or a misaligned
 * ws; BSGM_E_CAPACITY, BSGM_E_WORKSPACE and BSGM_E_UNSUPPORTED as above;
 * BSGM_E_HIP on a launch error. The kernel's waits are bounded: a wait that
 * has polled 2^22 times (on the order of a second) gives up and sets the
 * word at int32 index 64 of ws to 1; it stays set and the
 * results are then undefined. By construction every wait ends long before.
 */
int bsgm_select_blocks_fused(const bsgm_layout* layout, const bsgm_select_params* params,
                             const void* q, const void* k, int32_t* row_ptr, int32_t* col_idx,
                             int64_t col_capacity, float* row_stat, float* scores_out, void* ws,
                             size_t ws_bytes, void* stream);

/* Device workspace bytes of bsgm_select_blocks_fused: 128 * (19 + batch * heads)
 * bytes of synchronisation words and the pooled Q and K (4 * B * H * Nb * D
 * bytes each), each part rounded up to 256 bytes; 0 for an invalid layout (see
 * bsgm_last_error). */
size_t bsgm_fused_workspace_bytes(const bsgm_layout* layout);

/* Block-sparse attention forward ([VASC] section 3: retained weights are
 * renormalised after dropping connections; [ReSS] Table S6: every selection
 * rule drives the same block grid and sparse kernel). For each real query
 * token t of query block i, over the real key tokens u of the listed blocks:
 *   o_t = sum_u exp(scale <q_t,k_u> - m_t) v_u / sum_u exp(scale <q_t,k_u> - m_t),
 *   lse_t = m_t + log(sum_u exp(scale <q_t,k_u> - m_t)),  m_t = max_u scale <q_t,k_u>.
 * Padding query rows get o = 0 and lse = -inf; a row with no listed block
 * gets the same.
 *   q, k, v   device [B,H,N,D] of layout->dtype
 *   row_ptr, col_idx  device CSR as above (strictly ascending indices < Nb)
 *   o         device [B,H,N,D] of layout->dtype (bf16: rounded to nearest even)
 *   lse       device float [B,H,N] or NULL
 *   ws        device, >= bsgm_attn_workspace_bytes(layout) bytes, or NULL. bf16
 *             layouts: with ws, K is first copied to fp16 and the logits come
 *             from fp16 products of K and q * scale * log2(e) (c below), which
 *             takes no per-score arithmetic. That copy of K is exact for
 *             |k| >= 2^-17 and within 2^-25 below; the scaled query keeps 11
 *             significant bits above 2^-14 and is within 2^-25 below. The fp16
 *             products are used for a query block only when every |q c| of the
 *             block and every |k| of its listed key blocks is below 128; its
 *             base-2 logits are then within 2^-12 * sum_d |q_d c k_d| + 2^-11 of
 *             exact, plus fp32 accumulation. Every other query block takes bf16
 *             products (exact products, fp32 accumulation), as every block does
 *             with ws = NULL. The workspace holds only scratch; its contents on
 *             entry do not matter. fp32 layouts ignore ws.
 *   ws_bytes  size of ws (ignored when ws is NULL)
 * Errors: BSGM_E_ARG for a NULL q, k, v, row_ptr, col_idx or o, or a ws not
 * 256-byte aligned; BSGM_E_WORKSPACE when ws is given with fewer bytes than
 * needed; BSGM_E_HIP on a launch error.
 */
int bsgm_sparse_attn_fwd(const bsgm_layout* layout, const void* q, const void* k, const void* v,
                         const int32_t* row_ptr, const int32_t* col_idx, void* o, float* lse,
                         void* ws, size_t ws_bytes, void* stream);

/* The fp16 copy of K and its range flags alone, into ws (the first step of
 * bsgm_sparse_attn_fwd with a workspace). It depends on k only, so a caller can
 * run it on another stream while the blocks are being selected, then call
 * bsgm_sparse_attn_fwd_prepared, which skips the copy. fp32 layouts: nothing to
 * do, returns BSGM_OK.
 *   k         device [B,H,N,D] bf16
 *   ws        device, >= bsgm_attn_workspace_bytes(layout) bytes, 256-byte
 *             aligned (BSGM_E_ARG if NULL or misaligned, BSGM_E_WORKSPACE if
 *             smaller)
 */
int bsgm_attn_prepare(const bsgm_layout* layout, const void* k, void* ws, size_t ws_bytes,
                      void* stream);

/* bsgm_sparse_attn_fwd for a workspace that already holds the fp16 copy of this
 * k, made by bsgm_attn_prepare on the same layout (bf16 layouts; fp32 layouts
 * behave as bsgm_sparse_attn_fwd). ws is required. The caller orders the two
 * calls (an event, or the same stream) and keeps k and ws unchanged between
 * them; nothing checks that.
 */
int bsgm_sparse_attn_fwd_prepared(const bsgm_layout* layout, const void* q, const void* k,
                                  const void* v, const int32_t* row_ptr, const int32_t* col_idx,
                                  void* o, float* lse, void* ws, size_t ws_bytes, void* stream);

/* Scratch bytes for bsgm_sparse_attn_fwd's fp16 logits: the fp16 copy of K
 * (2 * B * H * N * D bytes) and two int32 flags per (b, h, block), each part
 * rounded up to 256 bytes, for bf16 layouts; 0 for fp32 or an invalid layout
 * (see bsgm_last_error). */
size_t bsgm_attn_workspace_bytes(const bsgm_layout* layout);

/* Bytes of the scratch array that bsgm_select_blocks_noalloc keeps on every
 * GPU it runs on (16 MiB). */
#define BSGM_NOALLOC_SCRATCH_BYTES (16u << 20)

/* TOPK or CDF selection as bsgm_select_blocks, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): it takes no workspace. Its pooled means
 * (and the CDF counts and flags) go to a scratch array of
 * BSGM_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it is called
 * on, from its first call there until the process ends; the call itself
 * allocates and frees nothing. The results are those of bsgm_select_blocks
 * with the same arguments, bit for bit (same kernels).
 * The array is that of the current device, which must be the device of
 * `stream`. Every call on one GPU shares its array: calls that overlap in time
 * on one GPU (other streams, other threads) race and give undefined results;
 * order them (one stream, or events). Nothing in the array needs clearing: each
 * call writes every word it later reads.
 *   params     mode BSGM_SEL_TOPK or BSGM_SEL_CDF (BSGM_E_UNSUPPORTED otherwise);
 *              the other fields as bsgm_select_blocks
 *   q, k, row_ptr, col_idx, col_capacity, row_stat, scores_out
 *              as bsgm_select_blocks
 * Errors: those of bsgm_select_blocks; BSGM_E_WORKSPACE when the layout needs
 * more scratch than the array holds (bsgm_workspace_bytes(layout, mode) >
 * BSGM_NOALLOC_SCRATCH_BYTES; for example a 100-frame layer of 16 heads and
 * blocks of 128 needs about 12 MiB in CDF mode), checked before anything is
 * enqueued; BSGM_E_HIP if the array's device address cannot be looked up.
 */
int bsgm_select_blocks_noalloc(const bsgm_layout* layout, const bsgm_select_params* params,
                               const void* q, const void* k, int32_t* row_ptr, int32_t* col_idx,
                               int64_t col_capacity, float* row_stat, float* scores_out,
                               void* stream);

/* Value-aware block selection with cross-layer pair memory ([VASC] 4.1-4.3,
 * A.1-A.5), one layer: selection from the memory, then the memory update.
 * Key blocks 2p and 2p+1 form pair p (an odd last block is a singleton).
 * Per (b, h): contrast c_p = sqrt(mean_d (vbar_2p - vbar_2p+1)^2) of the pooled
 * values (0 for the singleton), cbar = mean_p c_p. Per query block i, with P
 * the row softmax of the pooled scores (as in bsgm_select_blocks) and
 * k = keep_per_head[h]:
 *   a_ij   = P_ij * (1 + c_p(j) / cbar)      (factor 1 when cbar = 0)
 *   d_ij   = min(1, k * a_ij / sum_j a_ij)  (proportional clipping)
 *   rho_ij = d_ij + max(0, R_p(j)) / max_p max(0, R_p)   (0 if no deficit)
 * keeps the forced blocks (force_frame_first_block) and then the highest rho
 * (ties: lower block), exactly k per row, emitted as CSR like TOPK. Then for
 * every pair, with x the executed flags and the means over all query blocks
 * and the pair's children:  R_p += mean(d) - mean(x).
 *   params->mode must be BSGM_SEL_VASC; keep_per_head and
 *   force_frame_first_block are used
 *   q, k, v      device [B,H,N,D] of layout->dtype
 *   memory       device float [B, H, (Nb+1)/2], in/out: the raw pair balance
 *                R; zero it for a new inference or a new layout. The caller
 *                owns it and carries it from layer to layer.
 *   row_ptr, col_idx, col_capacity   as bsgm_select_blocks
 *   row_stat     device float [B*H*Nb] or NULL: kept pooled mass sum_kept P
 *   demand_out   device float [B,H,Nb,Nb] or NULL: d
 *   ws           device, >= bsgm_workspace_bytes(layout, BSGM_SEL_VASC) bytes
 */
int bsgm_vasc_select_blocks(const bsgm_layout* layout, const bsgm_select_params* params,
                            const void* q, const void* k, const void* v, float* memory,
                            int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                            float* row_stat, float* demand_out, void* ws, size_t ws_bytes,
                            void* stream);

/* Dense attention of the camera and register query rows ([VASC] 4.2 and A.5:
 * camera and register queries keep dense attention while patch queries use the
 * selected blocks). In every frame the first n_special tokens (the special
 * tokens, which open each frame) attend over all real keys of their (b, h):
 *   o_t = sum_u exp(scale <q_t,k_u> - m_t) v_u / sum_u exp(scale <q_t,k_u> - m_t),
 *   lse_t = m_t + log(sum_u exp(scale <q_t,k_u> - m_t)), over every real key u.
 * Only those rows of o and lse are written; run it after bsgm_sparse_attn_fwd
 * to replace their sparse result. bf16 only (BSGM_E_UNSUPPORTED otherwise).
 *   n_special  1..frame_valid special tokens per frame (VGGT: camera + 4 registers = 5)
 *   q, k, v    device [B,H,N,D] of layout->dtype (bf16: the passes run on the
 *              matrix cores with fp32-accurate split operands; fp32: vector ALU)
 *   o          device [B,H,N,D] bf16, rows f*frame_len + p (p < n_special) written
 *   lse        device float [B,H,N] or NULL, the same rows written
 *   ws         device, >= bsgm_special_rows_workspace_bytes(layout, n_special) bytes
 *              (per-chunk partial results of the split over key blocks)
 */
size_t bsgm_special_rows_workspace_bytes(const bsgm_layout* layout, int32_t n_special);
int bsgm_special_rows_dense_fwd(const bsgm_layout* layout, const void* q, const void* k,
                                const void* v, int32_t n_special, void* o, float* lse,
                                void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BSGM_H */
