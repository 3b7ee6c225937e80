// Internal interface between the C-ABI host layer (api.hip) and the kernel
// launchers. Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bsgm {

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Layout as the kernels see it (validated on the host).
struct Dims {
  int B, H, D;         // batch, heads, head_dim (64)
  int F, L, Lv;        // frames, padded frame length, real tokens per frame
  int blk;             // block size (64 or 128)
  int N;               // tokens per (b, h) = F * L
  int nb;              // blocks per (b, h) = N / blk
  int rows;            // B * H * nb
  float scale;         // softmax scale
};

constexpr int kMaxHeads = 128;

// Per-head budget and the CSR offset of each head's first row inside one
// batch entry (closed form when every row of head h keeps exactly keep[h]).
struct HeadBudget {
  int keep[kMaxHeads];
  long long head_off[kMaxHeads];   // sum_{h' < h} nb * keep[h']
  long long per_batch;             // sum_h nb * keep[h]
};

// Pooling: mean over real tokens of each block. dtype: 0 f32, 1 bf16.
hipError_t launch_pool(const Dims& d, int dtype, const void* x, float* mean, hipStream_t s);
// The same for n <= 3 tensors in one launch.
hipError_t launch_pool_n(const Dims& d, int dtype, int n, const void* const* xs,
                        float* const* means, hipStream_t s);

// Value-aware selection state for one layer (mode 3): per (b, h) and pair of
// key blocks the contrast factor and the memory's ranking copy (inputs), per
// row and pair the summed clipped demand and executed children (outputs).
struct VascSel {
  int npairs;
  const float* pair_fac;
  const float* mhat;
  float* pair_dem;
  float* pair_exe;
  float* demand_out;   // [rows, nb] or null
};

// Pooled selection (TOPK = 0, CDF = 1, VASC = 3 with vasc set) from pooled Q and K.
hipError_t launch_select_pooled(const Dims& d, const HeadBudget& hb, int mode, float tau,
                                int force, const float* qbar, const float* kbar,
                                int32_t* row_ptr, int32_t* col_idx, float* row_stat,
                                float* scores_out, int32_t* counts, uint32_t* bitmask,
                                hipStream_t s, const VascSel* vasc = nullptr);

// VASC, before selection: pair contrast factors and the memory's ranking copy
// from the pooled values and the raw memory [B*H, npairs].
hipError_t launch_vasc_prep(const Dims& d, int npairs, const float* vbar, const float* memory,
                            float* pair_fac, float* mhat, hipStream_t s);
// VASC, after selection: memory += mean demand - mean execution per pair.
hipError_t launch_vasc_update(const Dims& d, int npairs, const float* pair_dem,
                              const float* pair_exe, float* memory, hipStream_t s);

// Drift contributions and scores from pooled Q and K, V.
hipError_t launch_drift_contrib(const Dims& d, int dtype, const float* qbar, const void* k,
                                const void* v, float* contrib, float* score, float* zmass,
                                hipStream_t s);

// The same on the matrix cores for bf16 K and V (fp32-accurate via split
// operands). stats: [rows, nb] float2 scratch; mz: [rows] float2 scratch.
hipError_t launch_drift_contrib_bf16(const Dims& d, const float* qbar, void* qsplit, const void* k,
                                     const void* v, float2* stats, float2* mz, float* contrib,
                                     float* score, float* zmass, hipStream_t s);

// Drift selection with swap restoration.
hipError_t launch_select_drift(const Dims& d, const HeadBudget& hb, int force, int rounds,
                               int objective, const float* contrib, const float* zmass,
                               int32_t* row_ptr, int32_t* col_idx, float* row_stat,
                               int32_t* swap_log, hipStream_t s);

// Dynamic LDS of the per-row re-rank kernels (materialised and streamed); a
// row is supported while it fits kMaxRowLds.
constexpr size_t kMaxRowLds = 160 * 1024;
size_t drift_rerank_lds(int nb);
size_t drift_stream_step_lds(int nb);

// Drift selection by re-rank rounds (dropped-sum objective), optionally
// returning the least-J set seen (track_best). set_log: [rows, rounds + 1,
// ceil(nb / 32)] kept bitmasks or null.
hipError_t launch_select_drift_rerank(const Dims& d, const HeadBudget& hb, int force, int rounds,
                                      int track_best, const float* contrib, int32_t* row_ptr,
                                      int32_t* col_idx, float* row_stat, int32_t* set_log,
                                      hipStream_t s);

// Re-rank rounds in the expanded form, without the contributions (bf16 K and
// V). sqnorm: the squared drift scores ||c_ij||^2 [rows, nb], after qbar's
// split terms, the statistics and (M_i, Z_i) as launch_drift_contrib_bf16.
hipError_t launch_drift_sqnorms_bf16(const Dims& d, const float* qbar, void* qsplit, const void* k,
                                     const void* v, float2* stats, float2* mz, float* sqnorm,
                                     hipStream_t s);
// Most groups of key blocks of the residual pass (part holds [rows, groups, 64]).
int drift_round_groups_max(const Dims& d);
// The residual r_i of the drop set of `kept` ([rows, ceil(nb / 32)] bitmasks),
// as three bf16 terms in rsplit [rows, 3, 64], and J^2 = ||r_i||^2 in jsq; with
// best non-null, best/jbest keep the set of least J (round 0 starts them).
// via_kept: r_i = obar_i minus the sum over the kept blocks. kept null: obar_i =
// sum_j contrib_ij into obar [rows, 64] (nothing else written).
hipError_t launch_drift_residual_bf16(const Dims& d, const void* qsplit, const void* k,
                                      const void* v, const float2* mz, const uint32_t* kept,
                                      int via_kept, float* obar, float* part, void* rsplit,
                                      float* jsq, uint32_t* best, float* jbest, int round,
                                      hipStream_t s);
// The per-row step after the residual partials: part [rows, ngroups, 64] summed
// in group order into r (or into obar when kept is null), as above.
hipError_t launch_drift_resid(const Dims& d, const uint32_t* kept, int via_kept, float* obar,
                              float* part, int ngroups, void* rsplit, float* jsq, uint32_t* best,
                              float* jbest, int round, hipStream_t s);
// The same three passes for fp32 K and V on the vector ALU (part: one group).
hipError_t launch_drift_sqnorms_f32(const Dims& d, const float* qbar, const void* k, const void* v,
                                    float* sqnorm, hipStream_t s);
hipError_t launch_drift_residual_f32(const Dims& d, const float* qbar, const void* k,
                                     const void* v, const uint32_t* kept, int via_kept,
                                     float* obar, float* part, void* rsplit, float* jsq,
                                     uint32_t* best, float* jbest, int round, hipStream_t s);
hipError_t launch_drift_dot_f32(const Dims& d, const float* qbar, const void* rsplit,
                                const void* k, const void* v, float* dot, hipStream_t s);
// dot[i, j] = <r_i, c_ij> for every block, recomputed from qbar, K and V.
hipError_t launch_drift_dot_bf16(const Dims& d, const void* qsplit, const void* rsplit,
                                 const void* k, const void* v, const float2* mz, float* dot,
                                 hipStream_t s);
// One round's selection from sqnorm and dot (round 0: sqnorm alone), into next.
hipError_t launch_drift_stream_step(const Dims& d, const HeadBudget& hb, int force, int rounds,
                                    int round, const float* sqnorm, const float* dot,
                                    const uint32_t* prev, uint32_t* next, int32_t* set_log,
                                    hipStream_t s);
// The CSR of the kept sets, and row_stat = sqrt(jsq) when row_stat is non-null.
hipError_t launch_drift_stream_emit(const Dims& d, const HeadBudget& hb, const uint32_t* kept,
                                    const float* jsq, int32_t* row_ptr, int32_t* col_idx,
                                    float* row_stat, hipStream_t s);

// Block-sparse attention forward. ws: attn_workspace_bytes(d) bytes of device
// scratch (enables the fp16 logits: an fp16 copy of K, a range flag per
// (b, h, key block) and a fallback flag per row), or null (bf16 logits only).
// k_ready: ws already holds the fp16 copy of this k (launch_attn_prepare).
hipError_t launch_attn_bf16(const Dims& d, const void* q, const void* k, const void* v,
                            const int32_t* row_ptr, const int32_t* col_idx, void* o,
                            float* lse, void* ws, hipStream_t s, bool k_ready = false);
// The fp16 copy of K and its range flags into ws, on its own.
hipError_t launch_attn_prepare(const Dims& d, const void* k, void* ws, hipStream_t s);
inline size_t attn_workspace_bytes(const Dims& d) {
  return align256((size_t)d.B * d.H * d.N * 64 * 2) + 2 * align256((size_t)d.rows * 4);
}
hipError_t launch_attn_f32(const Dims& d, const void* q, const void* k, const void* v,
                           const int32_t* row_ptr, const int32_t* col_idx, void* o,
                           float* lse, hipStream_t s);

// Dense attention of the camera/register rows: work split and scratch sizes.
struct DenseRowsPlan {
  int nrows, ngroups, cpc, nchunks;
  size_t po_bytes, pml_bytes;
};
DenseRowsPlan dense_rows_plan(const Dims& d, int ns);
hipError_t launch_dense_rows(const Dims& d, int ns, const void* q, const void* k, const void* v,
                             void* o, float* lse, void* ws, hipStream_t s);

// Largest key-block count whose drift selection row the best-swap kernel keeps
// in LDS; wider rows (up to kDriftMaxBlocks) leave the row in L2.
constexpr int kDriftLdsRowBlocks = 512;
constexpr int kDriftMaxBlocks = 4096;
// Largest block count a pooled selection row handles (16 per thread x 256).
constexpr int kSelectMaxBlocks = 4096;

}  // namespace bsgm
