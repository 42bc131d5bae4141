// Internal launchers of libmla: the C ABI in api.cpp validates arguments, then calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "mla.h"

namespace mla {

// Split-K plan of the append projection (shared by the workspace query and the launch).
struct AppendPlan {
  int n_ksplit, k_chunk, col_blocks, tok_tiles;
};
AppendPlan append_plan(const mla_dims& d, int n_tok);

// Workspace of an append of n_tok tokens: the split-K partial sums.
size_t append_ws_bytes(const mla_dims& d, int n_tok);
hipError_t launch_append(const mla_dims& d, int n_tok, const void* x, const int32_t* seq_idx,
                         const int32_t* pos, const void* w_dkv, const void* gamma,
                         const void* w_kr, const int32_t* table, int batch, int max_blocks,
                         int num_blocks, void* cache, float* cache_scale, void* ws,
                         hipStream_t s);
// The append, then the absorption of q_batch x s_q queries (none when q_batch * s_q == 0). On
// the matrix cores the absorption shares a launch with the append's projection. cache_scale
// non-null: bf16 dims, and the rows go out as e4m3 bytes with one scale per slot.
hipError_t launch_append_absorb(const mla_dims& d, int n_tok, const void* x,
                                const int32_t* seq_idx, const int32_t* pos, const void* w_dkv,
                                const void* gamma, const void* w_kr, const int32_t* table,
                                int batch, int max_blocks, int num_blocks, void* cache,
                                float* cache_scale, void* ws, int q_batch, int s_q, const void* q_nope, const void* q_pe,
                                const int32_t* q_pos, const void* w_uk, void* q_abs,
                                hipStream_t s);

// bf16 rows of ncols (a multiple of 4, at most 1024) values to e4m3 bytes and one scale per row.
hipError_t launch_quantize_e4m3(int64_t n_rows, int ncols, const void* rows, void* out,
                               float* scale, hipStream_t s);

// Split-K partial sums of y = x · [W_a | W_b] for n_tok tokens (K-wide rows of x):
// y_part[k][n][c] over C range [256 k, 256 k + 256), k < projection_ksplit(K). The matrix-core
// kernel needs bf16, K, n_a and n_b multiples of 8 and 16-byte aligned operands.
int projection_ksplit(int K);
hipError_t launch_projection_partials(int dt, bool mfma, int n_tok, int K, const void* x,
                                      const void* w_a, int n_a, const void* w_b, int n_b,
                                      float* y_part, hipStream_t s);
// Decode-layer projections around the path (project.hip); ws as sized by the matching
// *_workspace_bytes call of the C ABI.
size_t query_project_ws_bytes(const mla_dims& d, int n_tok, int d_q);
hipError_t launch_query_project(const mla_dims& d, int n_tok, int d_q, const void* x,
                                const void* w_dq, const void* gamma_q, const void* w_uq,
                                const void* w_qr, void* q_nope, void* q_pe, void* ws,
                                hipStream_t s);
size_t output_project_ws_bytes(const mla_dims& d, int n_tok);
hipError_t launch_output_project(const mla_dims& d, int n_tok, const void* o, const void* w_o,
                                 const void* b_o, void* y, void* ws, hipStream_t s);

hipError_t launch_absorb(const mla_dims& d, int batch, int s_q, const void* q_nope,
                         const void* q_pe, const int32_t* q_pos, const void* w_uk, void* q_abs,
                         hipStream_t s);

// Workspace of one split-K decode, each part 256-byte aligned: partial o [B, s_q, H, n_split,
// width] fp32, partial lse2 [B, s_q, H, n_split] fp32 (log2 domain of scale*score), recompute
// flags [B, s_q, n_split] int32, and the merged rows [B, s_q, H, width] fp32.
size_t partials_bytes(int batch, int s_q, int heads, int n_split, int width, int elt);

// Split-K core: every (split, query, sequence) writes its partials (and recompute flag).
// scales != NULL: the cache rows are e4m3 bytes, row r worth bytes x scales[r] (bf16 dims
// otherwise, on the matrix-core kernel: mfma_decode_fp8_fits).
hipError_t launch_decode_splitk(const mla_dims& d, int batch, int s_q, const void* q_abs,
                                const void* cache, const float* scales, int num_blocks,
                                const int32_t* table, int max_blocks, const int32_t* seq_lens,
                                int n_split, void* ws, hipStream_t s);

// A decode step's new rows, formed inside the split-K core: the s_q new tokens of every
// sequence are its positions L - s_q .. L - 1 (token n = b s_q + i), projected but not yet
// written (y_part: the append's split-K partial sums, [n_ksplit][B s_q][d_c + d_r]).
struct StepRows {
  const float* y_part;
  const void* gamma;  // RMSNorm gain [d_c]
  void* cache;        // the latent cache, written at the new rows' slots
  float* scale;       // e4m3 rows: the per-slot scales, written with them (NULL for bf16 rows)
  int n_ksplit;
  float eps, base;
};
// Whether the core can form the new rows itself (bf16, d_c 512, d_r 64, H = 128), and the
// split-K core of such a step (the merge is launch_decode_merge's).
bool mfma_step_fits(const mla_dims& d);
hipError_t launch_decode_step_splitk(const mla_dims& d, int batch, int s_q, const void* q_abs,
                                     void* cache, int num_blocks, const int32_t* table,
                                     int max_blocks, const int32_t* seq_lens, int n_split,
                                     void* ws, const StepRows& rows, hipStream_t s);
// The step's projection of the B s_q new tokens into y_part together with the absorption of
// their queries (positions implied by the lengths) in one launch; needs
// step_project_fits(d, B s_q). The rows themselves are formed by the core.
bool step_project_fits(const mla_dims& d, int n_tok);
hipError_t launch_step_project(const mla_dims& d, int batch, int s_q, const void* x,
                               const void* w_dkv, const void* w_kr, float* y_part,
                               const void* q_nope, const void* q_pe, const int32_t* seq_lens,
                               const void* w_uk, void* q_abs, hipStream_t s);
// Positions of a step's new tokens for the separate calls: seq_idx[n] = n / s_q,
// pos[n] = seq_lens[n / s_q] - s_q + n % s_q (pos doubles as the queries' positions).
hipError_t launch_step_positions(int batch, int s_q, const int32_t* seq_lens, int32_t* seq_idx,
                                 int32_t* pos, hipStream_t s);
// Merge: flagged splits recomputed, log-sum-exp merge over splits, W_UV per group.
hipError_t launch_decode_merge(const mla_dims& d, int batch, int s_q, const void* q_abs,
                               const void* cache, const float* scales, int num_blocks,
                               const int32_t* table, int max_blocks, const int32_t* seq_lens,
                               const void* w_uv, int n_split, void* ws, void* out, float* lse,
                               hipStream_t s);

hipError_t launch_expand(const mla_dims& d, int batch, const void* cache, int num_blocks,
                         const int32_t* table, int max_blocks, const int32_t* seq_lens,
                         const int32_t* start_pos, const void* w_uk, const void* w_uv,
                         void* gqa, hipStream_t s);

hipError_t launch_gqa_decode(const mla_dims& d, int batch, int s_q, const void* q_nope,
                             const void* q_pe, const int32_t* q_pos, const void* gqa,
                             int num_blocks, const int32_t* table, int max_blocks,
                             const int32_t* seq_lens, int n_split, void* ws, void* out,
                             float* lse, hipStream_t s);

// Whether the MFMA decode kernel handles these dims (bf16, d_c 512, d_r 64, H % 32 == 0), and
// with e4m3 rows (H = 128 as well).
bool mfma_decode_fits(const mla_dims& d);
bool mfma_decode_fp8_fits(const mla_dims& d);
struct StepRows;
// With plan != NULL the splits follow the length-balanced plan (plan.hpp), which the kernel
// computes and stores at *plan; else n_split uniform splits per (sequence, query).
struct SplitPlan;
hipError_t launch_decode_mfma(const mla_dims& d, int batch, int s_q, const void* q_abs,
                              const void* cache, const float* scales, int num_blocks,
                              const int32_t* table, int max_blocks, const int32_t* seq_lens,
                              int n_split, void* part_o, float* part_lse, int* redo,
                              SplitPlan* plan, const StepRows* app, hipStream_t s);
// Whether n_split = 0 takes the length-balanced plan for these dims and rows, and the
// workspace of a planned decode (the plan, then partials for every slot).
bool plan_applies(const mla_dims& d, int batch, int s_q);
size_t planned_workspace_bytes(const mla_dims& d);

// Whether the MFMA GQA decode kernel handles these dims and query count (bf16, D = D_v = 128,
// d_r = 64, block size a multiple of 32), and its launch: every (sequence, split, group,
// 32 query rows) writes the partials of its rows, or with direct (n_split = 1) the final
// output and natural-log lse (lse may then be null).
bool gqa_mfma_fits(const mla_dims& d, int s_q);
// The shared-tile kernel (at least 64 query rows per group, same shape limits as the GQA
// kernel): with direct (n_split = 1) out and natural-log lse (nullable) written directly,
// otherwise every split's partials as the GQA kernel writes them.
bool prefill_mfma_fits(const mla_dims& d, int s_q);
hipError_t launch_prefill_mfma(const mla_dims& d, int batch, int s_q, const void* q_nope,
                               const void* q_pe, const int32_t* q_pos, const void* gqa,
                               int num_blocks, const int32_t* table, int max_blocks,
                               const int32_t* seq_lens, int n_split, void* out, float* lse,
                               bool direct, hipStream_t s);
hipError_t launch_gqa_mfma(const mla_dims& d, int batch, int s_q, const void* q_nope,
                           const void* q_pe, const int32_t* q_pos, const void* gqa,
                           int num_blocks, const int32_t* table, int max_blocks,
                           const int32_t* seq_lens, int n_split, void* part_o, float* part_lse,
                           bool direct, hipStream_t s);

inline float softmax_scale_of(const mla_dims& d) {
  return d.softmax_scale > 0.f ? d.softmax_scale
                               : 1.0f / sqrtf(static_cast<float>(d.d_nope + d.d_r));
}

constexpr int kSplitAlign = 64;  // split boundaries fall on multiples of this many positions

}  // namespace mla
