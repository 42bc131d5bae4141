// C ABI of libmla (declared and documented in include/mla.h): host-side validation, workspace
// sizing and dispatch to the kernel launchers. Nothing here allocates, synchronises or prints.
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "launch.hpp"
#include "mla.h"

namespace {

inline int cdiv(int a, int b) { return (a + b - 1) / b; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Bytes per element of every float tensor, and of the split partial rows.
int elt_of(const mla_dims& d) { return d.dtype == MLA_BF16 ? 2 : 4; }

mla_status check_dims(const mla_dims* d) {
  if (d == nullptr) return MLA_ERR_NULL;
  if (d->dtype != MLA_F32 && d->dtype != MLA_BF16) return MLA_ERR_DTYPE;
  if (d->d_model < 1 || d->n_heads < 1 || d->d_nope < 1 || d->d_v < 1 || d->d_c < 1 ||
      d->d_r < 0 || (d->d_r & 1) || d->n_groups < 1 || d->block_size < 1)
    return MLA_ERR_SHAPE;
  if (d->n_heads % d->n_groups != 0) return MLA_ERR_SHAPE;
  if (d->d_c % 8 != 0) return MLA_ERR_SHAPE;  // 16-byte weight loads never straddle c and k_r
  if (d->d_v % 8 != 0) return MLA_ERR_SHAPE;  // the merge reads partial rows 16 bytes at a time
  // LDS budgets of the portable kernels: query row + value row + 2 KiB of per-pass state,
  // and 16 merged latent rows in the combine.
  if (d->d_c + d->d_r > 4096 || d->d_nope + d->d_r > 4096 || d->d_v > 1024 || d->d_c > 1024 ||
      d->d_nope > 1024)
    return MLA_ERR_SHAPE;
  if (!(d->rope_base > 0.f) || !(d->rms_eps >= 0.f) || !(d->softmax_scale >= 0.f) ||
      !isfinite(d->rope_base) || !isfinite(d->softmax_scale))
    return MLA_ERR_SHAPE;
  return MLA_OK;
}

int resolve_split(const mla_dims& d, int batch, int s_q, int max_blocks) {
  // Aim at one workgroup per CU (256 CUs), with at least kSplitAlign positions per split.
  const int rows = batch * s_q;
  int n = cdiv(256, rows > 0 ? rows : 1);
  const int max_by_len = cdiv(max_blocks * d.block_size, mla::kSplitAlign);
  if (n > max_by_len) n = max_by_len;
  if (n > 64) n = 64;
  return n < 1 ? 1 : n;
}

mla_status hip_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

// the expanded rows of a prefill: [K_0 .. K_{G-1} || V_0 .. V_{G-1} || k_r] per cached slot
size_t prefill_kv_bytes(const mla_dims& d, int num_blocks) {
  const size_t row = static_cast<size_t>(d.n_groups) * (d.d_nope + d.d_v) + d.d_r;
  const size_t b = static_cast<size_t>(num_blocks) * d.block_size * row * elt_of(d);
  return (b + 255) / 256 * 256;
}

}  // namespace

extern "C" {

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL: return "a required pointer is NULL";
    case MLA_ERR_SHAPE: return "a dimension is out of range or inconsistent";
    case MLA_ERR_DTYPE: return "unknown dtype";
    case MLA_ERR_RANGE: return "a count is out of range";
    case MLA_ERR_WORKSPACE: return "workspace missing or too small";
    case MLA_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case MLA_ERR_HIP: return "a kernel launch failed";
    case MLA_ERR_BLOCK_TABLE: return "block table holds a bad or shared block id";
    case MLA_STATUS_INT32_: break;
  }
  return "unknown status";
}

int32_t mla_auto_split(const mla_dims* dims, int32_t batch, int32_t s_q, int32_t max_blocks) {
  if (check_dims(dims) != MLA_OK || batch < 1 || s_q < 1 || max_blocks < 1) return 0;
  return resolve_split(*dims, batch, s_q, max_blocks);
}

int32_t mla_select_path(const mla_dims* dims, int32_t s_q, int64_t context,
                        double hbm_bytes_per_s, double flops_per_s, double* t_absorbed,
                        double* t_gqa) {
  const mla_status st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (s_q < 1 || context < 1) return MLA_ERR_RANGE;
  if (hbm_bytes_per_s == 0.0 && flops_per_s == 0.0) {
    hbm_bytes_per_s = MLA_MI355X_HBM_BYTES_PER_S;
    flops_per_s = MLA_MI355X_BF16_FLOPS;
  }
  if (!(hbm_bytes_per_s > 0.0) || !(flops_per_s > 0.0)) return MLA_ERR_RANGE;
  const mla_dims& d = *dims;
  const double elt = d.dtype == MLA_BF16 ? 2.0 : 4.0;
  const double H = d.n_heads, G = d.n_groups, L = static_cast<double>(context), q = s_q;
  const double abs_bytes = L * (d.d_c + d.d_r) * elt;
  const double abs_flops = L * q * (2.0 * H * (d.d_c + d.d_r) + 2.0 * H * d.d_c);
  const double gqa_bytes = L * (G * (d.d_nope + d.d_v) + d.d_r) * elt;
  const double gqa_flops = L * q * (2.0 * H * (d.d_nope + d.d_r) + 2.0 * H * d.d_v);
  const double ta = std::max(abs_bytes / hbm_bytes_per_s, abs_flops / flops_per_s);
  const double tg = std::max(gqa_bytes / hbm_bytes_per_s, gqa_flops / flops_per_s);
  if (t_absorbed) *t_absorbed = ta;
  if (t_gqa) *t_gqa = tg;
  return tg < ta ? MLA_PATH_GQA : MLA_PATH_ABSORBED;
}

size_t mla_cache_append_workspace_bytes(const mla_dims* dims, int32_t n_tok) {
  if (check_dims(dims) != MLA_OK || n_tok < 0) return 0;
  return mla::append_ws_bytes(*dims, n_tok);
}

}  // extern "C"

namespace {

// Host checks of mla_cache_append (dims already checked); MLA_OK with n_tok == 0 means
// nothing to do.
// e4m3 rows: quantised from bf16 values, 16-byte rows of at most 1024 values.
bool fp8_rows_ok(const mla_dims& d) {
  const int n = d.d_c + d.d_r;
  return d.dtype == MLA_BF16 && n % 16 == 0 && n <= 1024;
}

mla_status check_append(const mla_dims* dims, int32_t n_tok, const void* x,
                        const int32_t* seq_idx, const int32_t* pos, const void* w_dkv,
                        const void* rms_gamma, const void* w_kr, const int32_t* block_table,
                        int32_t batch, int32_t max_blocks, int32_t num_blocks,
                        const void* latent_cache, const void* workspace, size_t ws_bytes) {
  if (n_tok < 0 || batch < 0 || max_blocks < 1 || num_blocks < 1) return MLA_ERR_RANGE;
  if (n_tok == 0) return MLA_OK;
  if (!x || !seq_idx || !pos || !w_dkv || !rms_gamma || !block_table || !latent_cache ||
      (dims->d_r > 0 && !w_kr))
    return MLA_ERR_NULL;
  if (batch < 1) return MLA_ERR_RANGE;
  if (static_cast<int64_t>(max_blocks) * dims->block_size > INT32_MAX) return MLA_ERR_RANGE;
  if (!aligned16(x) || !aligned16(w_dkv) || !aligned16(rms_gamma) ||
      (w_kr && !aligned16(w_kr)) || !aligned16(latent_cache) || !aligned16(block_table))
    return MLA_ERR_ALIGN;
  const size_t need = mla_cache_append_workspace_bytes(dims, n_tok);
  if (workspace == nullptr || ws_bytes < need) return MLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MLA_ERR_ALIGN;
  return MLA_OK;
}

// Host checks of mla_absorb_q (dims already checked); MLA_OK with batch == 0 means nothing
// to do.
mla_status check_absorb(const mla_dims* dims, int32_t batch, int32_t s_q, const void* q_nope,
                        const void* q_pe, const int32_t* q_pos, const void* w_uk,
                        const void* q_abs) {
  if (batch < 0 || s_q < 1) return MLA_ERR_RANGE;
  if (batch == 0) return MLA_OK;
  if (!q_nope || !q_pos || !w_uk || !q_abs || (dims->d_r > 0 && !q_pe)) return MLA_ERR_NULL;
  if (static_cast<int64_t>(batch) * s_q > 65535 * 16) return MLA_ERR_RANGE;
  if (!aligned16(q_nope) || (q_pe && !aligned16(q_pe)) || !aligned16(w_uk) || !aligned16(q_abs))
    return MLA_ERR_ALIGN;
  return MLA_OK;
}

}  // namespace

extern "C" {

mla_status mla_cache_append(const mla_dims* dims, int32_t n_tok, const void* x,
                            const int32_t* seq_idx, const int32_t* pos, const void* w_dkv,
                            const void* rms_gamma, const void* w_kr, const int32_t* block_table,
                            int32_t batch, int32_t max_blocks, int32_t num_blocks,
                            void* latent_cache, void* workspace, size_t ws_bytes,
                            hipStream_t stream) {
  mla_status st = check_dims(dims);
  if (st != MLA_OK) return st;
  st = check_append(dims, n_tok, x, seq_idx, pos, w_dkv, rms_gamma, w_kr, block_table, batch,
                    max_blocks, num_blocks, latent_cache, workspace, ws_bytes);
  if (st != MLA_OK || n_tok == 0) return st;
  return hip_status(mla::launch_append(*dims, n_tok, x, seq_idx, pos, w_dkv, rms_gamma, w_kr,
                                       block_table, batch, max_blocks, num_blocks, latent_cache,
                                       nullptr, workspace, stream));
}

mla_status mla_absorb_q(const mla_dims* dims, int32_t batch, int32_t s_q, const void* q_nope,
                        const void* q_pe, const int32_t* q_pos, const void* w_uk, void* q_abs,
                        hipStream_t stream) {
  mla_status st = check_dims(dims);
  if (st != MLA_OK) return st;
  st = check_absorb(dims, batch, s_q, q_nope, q_pe, q_pos, w_uk, q_abs);
  if (st != MLA_OK || batch == 0) return st;
  return hip_status(mla::launch_absorb(*dims, batch, s_q, q_nope, q_pe, q_pos, w_uk, q_abs, stream));
}

mla_status mla_cache_append_absorb_q(const mla_dims* dims, int32_t n_tok, const void* x,
                                     const int32_t* seq_idx, const int32_t* pos,
                                     const void* w_dkv, const void* rms_gamma, const void* w_kr,
                                     const int32_t* block_table, int32_t batch,
                                     int32_t max_blocks, int32_t num_blocks, void* latent_cache,
                                     void* workspace, size_t ws_bytes, int32_t s_q,
                                     const void* q_nope, const void* q_pe, const int32_t* q_pos,
                                     const void* w_uk, void* q_abs, hipStream_t stream) {
  mla_status st = check_dims(dims);
  if (st != MLA_OK) return st;
  st = check_append(dims, n_tok, x, seq_idx, pos, w_dkv, rms_gamma, w_kr, block_table, batch,
                    max_blocks, num_blocks, latent_cache, workspace, ws_bytes);
  if (st != MLA_OK) return st;
  st = check_absorb(dims, batch, s_q, q_nope, q_pe, q_pos, w_uk, q_abs);
  if (st != MLA_OK) return st;
  if (n_tok == 0 && batch == 0) return MLA_OK;
  if (n_tok == 0)
    return hip_status(mla::launch_absorb(*dims, batch, s_q, q_nope, q_pe, q_pos, w_uk, q_abs,
                                         stream));
  return hip_status(mla::launch_append_absorb(*dims, n_tok, x, seq_idx, pos, w_dkv, rms_gamma,
                                              w_kr, block_table, batch, max_blocks, num_blocks,
                                              latent_cache, nullptr, workspace, batch, s_q, q_nope,
                                              q_pe, q_pos, w_uk, q_abs, stream));
}

mla_status mla_cache_quantize_fp8(const mla_dims* dims, int64_t n_rows, const void* rows,
                                  void* rows_fp8, float* row_scale, hipStream_t stream) {
  mla_status st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (!fp8_rows_ok(*dims)) return MLA_ERR_SHAPE;
  if (n_rows < 0) return MLA_ERR_RANGE;
  if (n_rows == 0) return MLA_OK;
  if (!rows || !rows_fp8 || !row_scale) return MLA_ERR_NULL;
  if (!aligned16(rows) || !aligned16(rows_fp8) || !aligned16(row_scale)) return MLA_ERR_ALIGN;
  return hip_status(mla::launch_quantize_e4m3(n_rows, dims->d_c + dims->d_r, rows, rows_fp8,
                                              row_scale, stream));
}

mla_status mla_cache_append_fp8(const mla_dims* dims, int32_t n_tok, const void* x,
                                const int32_t* seq_idx, const int32_t* pos, const void* w_dkv,
                                const void* rms_gamma, const void* w_kr,
                                const int32_t* block_table, int32_t batch, int32_t max_blocks,
                                int32_t num_blocks, void* cache_fp8, float* cache_scale,
                                void* workspace, size_t ws_bytes, hipStream_t stream) {
  return mla_cache_append_absorb_q_fp8(dims, n_tok, x, seq_idx, pos, w_dkv, rms_gamma, w_kr,
                                       block_table, batch, max_blocks, num_blocks, cache_fp8,
                                       cache_scale, workspace, ws_bytes, 0, nullptr, nullptr,
                                       nullptr, nullptr, nullptr, stream);
}

mla_status mla_cache_append_absorb_q_fp8(const mla_dims* dims, int32_t n_tok, const void* x,
                                         const int32_t* seq_idx, const int32_t* pos,
                                         const void* w_dkv, const void* rms_gamma,
                                         const void* w_kr, const int32_t* block_table,
                                         int32_t batch, int32_t max_blocks, int32_t num_blocks,
                                         void* cache_fp8, float* cache_scale, void* workspace,
                                         size_t ws_bytes, int32_t s_q, const void* q_nope,
                                         const void* q_pe, const int32_t* q_pos,
                                         const void* w_uk, void* q_abs, hipStream_t stream) {
  // s_q == 0: the append alone (mla_cache_append_fp8)
  mla_status st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (!fp8_rows_ok(*dims)) return MLA_ERR_SHAPE;
  st = check_append(dims, n_tok, x, seq_idx, pos, w_dkv, rms_gamma, w_kr, block_table, batch,
                    max_blocks, num_blocks, cache_fp8, workspace, ws_bytes);
  if (st != MLA_OK) return st;
  if (n_tok > 0) {
    if (!cache_scale) return MLA_ERR_NULL;
    if (!aligned16(cache_scale)) return MLA_ERR_ALIGN;
  }
  const int q_batch = s_q == 0 ? 0 : batch;
  if (s_q != 0) {
    st = check_absorb(dims, batch, s_q, q_nope, q_pe, q_pos, w_uk, q_abs);
    if (st != MLA_OK) return st;
  }
  if (n_tok == 0 && q_batch == 0) return MLA_OK;
  if (n_tok == 0)
    return hip_status(mla::launch_absorb(*dims, q_batch, s_q, q_nope, q_pe, q_pos, w_uk, q_abs,
                                         stream));
  return hip_status(mla::launch_append_absorb(*dims, n_tok, x, seq_idx, pos, w_dkv, rms_gamma,
                                              w_kr, block_table, batch, max_blocks, num_blocks,
                                              cache_fp8, cache_scale, workspace, q_batch, s_q,
                                              q_nope, q_pe, q_pos, w_uk, q_abs, stream));
}

size_t mla_query_project_workspace_bytes(const mla_dims* dims, int32_t n_tok, int32_t d_q) {
  if (check_dims(dims) != MLA_OK || n_tok < 1 || d_q < 1) return 0;
  return mla::query_project_ws_bytes(*dims, n_tok, d_q);
}

mla_status mla_query_project(const mla_dims* dims, int32_t n_tok, int32_t d_q, const void* x,
                             const void* w_dq, const void* gamma_q, const void* w_uq,
                             const void* w_qr, void* q_nope, void* q_pe, void* workspace,
                             size_t ws_bytes, hipStream_t stream) {
  mla_status st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (n_tok < 0 || d_q < 1) return MLA_ERR_RANGE;
  if (n_tok == 0) return MLA_OK;
  const bool rope = dims->d_r > 0;
  if (!x || !w_dq || !gamma_q || !w_uq || !q_nope || (rope && (!w_qr || !q_pe)))
    return MLA_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_dq) || !aligned16(gamma_q) || !aligned16(w_uq) ||
      !aligned16(q_nope) || (rope && (!aligned16(w_qr) || !aligned16(q_pe))))
    return MLA_ERR_ALIGN;
  if (workspace == nullptr || ws_bytes < mla_query_project_workspace_bytes(dims, n_tok, d_q))
    return MLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MLA_ERR_ALIGN;
  return hip_status(mla::launch_query_project(*dims, n_tok, d_q, x, w_dq, gamma_q, w_uq,
                                              rope ? w_qr : nullptr, q_nope,
                                              rope ? q_pe : nullptr, workspace, stream));
}

size_t mla_output_project_workspace_bytes(const mla_dims* dims, int32_t n_tok) {
  if (check_dims(dims) != MLA_OK || n_tok < 1) return 0;
  return mla::output_project_ws_bytes(*dims, n_tok);
}

mla_status mla_output_project(const mla_dims* dims, int32_t n_tok, const void* o,
                              const void* w_o, const void* b_o, void* y, void* workspace,
                              size_t ws_bytes, hipStream_t stream) {
  mla_status st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (n_tok < 0) return MLA_ERR_RANGE;
  if (n_tok == 0) return MLA_OK;
  if (!o || !w_o || !y) return MLA_ERR_NULL;
  if (!aligned16(o) || !aligned16(w_o) || (b_o && !aligned16(b_o)) || !aligned16(y))
    return MLA_ERR_ALIGN;
  if (workspace == nullptr || ws_bytes < mla_output_project_workspace_bytes(dims, n_tok))
    return MLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MLA_ERR_ALIGN;
  return hip_status(mla::launch_output_project(*dims, n_tok, o, w_o, b_o, y, workspace, stream));
}

size_t mla_decode_workspace_bytes(const mla_dims* dims, int32_t batch, int32_t s_q,
                                  int32_t n_split, int32_t max_blocks) {
  if (check_dims(dims) != MLA_OK || batch < 1 || s_q < 1 || max_blocks < 1 || n_split < 0 ||
      n_split > MLA_MAX_SPLIT)
    return 0;
  if (n_split == 0 && mla::plan_applies(*dims, batch, s_q)) return mla::planned_workspace_bytes(*dims);
  const int ns = n_split == 0 ? resolve_split(*dims, batch, s_q, max_blocks) : n_split;
  return mla::partials_bytes(batch, s_q, dims->n_heads, ns, dims->d_c, elt_of(*dims));
}

}  // extern "C"

namespace {

// Shared validation of the decode calls; on success *ns holds the resolved split count.
mla_status check_decode(const mla_dims* dims, int32_t batch, int32_t s_q, const void* q_abs,
                        const void* latent_cache, int32_t num_blocks, const int32_t* block_table,
                        int32_t max_blocks, const int32_t* seq_lens, int32_t n_split,
                        const void* workspace, size_t ws_bytes, int* ns) {
  mla_status st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (batch < 0 || s_q < 1 || max_blocks < 1 || num_blocks < 1 || n_split < 0 ||
      n_split > MLA_MAX_SPLIT)
    return MLA_ERR_RANGE;
  if (batch > 65535 || s_q > 65535 || static_cast<int64_t>(batch) * s_q > 65535)
    return MLA_ERR_RANGE;
  if (static_cast<int64_t>(max_blocks) * dims->block_size > INT32_MAX) return MLA_ERR_RANGE;
  if (batch == 0) return MLA_OK;
  if (!q_abs || !latent_cache || !block_table || !seq_lens) return MLA_ERR_NULL;
  if (!aligned16(q_abs) || !aligned16(latent_cache)) return MLA_ERR_ALIGN;
  // n_split = 0: the length-balanced plan where it applies (*ns = 0 tells the launchers),
  // else the uniform count the library picks
  const bool planned = n_split == 0 && mla::plan_applies(*dims, batch, s_q);
  *ns = planned ? 0 : n_split == 0 ? resolve_split(*dims, batch, s_q, max_blocks) : n_split;
  const size_t need = planned ? mla::planned_workspace_bytes(*dims)
                              : mla::partials_bytes(batch, s_q, dims->n_heads, *ns, dims->d_c,
                                                    elt_of(*dims));
  if (workspace == nullptr || ws_bytes < need) return MLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MLA_ERR_ALIGN;
  return MLA_OK;
}

// The decode calls: the split-K core, the merge, or both, over bf16/fp32 rows (scales NULL) or
// e4m3 rows with per-slot scales.
enum DecodePart { kSplit = 1, kMerge = 2 };
mla_status decode_call(int parts, const mla_dims* dims, int32_t batch, int32_t s_q,
                       const void* q_abs, const void* latent_cache, const float* scales,
                       bool fp8, int32_t num_blocks, const int32_t* block_table,
                       int32_t max_blocks, const int32_t* seq_lens, const void* w_uv,
                       int32_t n_split, void* workspace, size_t ws_bytes, void* out, float* lse,
                       hipStream_t stream) {
  int ns = 0;
  mla_status st = check_decode(dims, batch, s_q, q_abs, latent_cache, num_blocks, block_table,
                               max_blocks, seq_lens, n_split, workspace, ws_bytes, &ns);
  if (st != MLA_OK || batch == 0) return st;
  if (fp8) {
    if (!mla::mfma_decode_fp8_fits(*dims) || (dims->flags & MLA_FLAG_GENERIC_KERNELS))
      return MLA_ERR_SHAPE;
    if (!scales) return MLA_ERR_NULL;
    if (!aligned16(scales)) return MLA_ERR_ALIGN;
  }
  if (parts & kMerge) {
    if (!w_uv || !out) return MLA_ERR_NULL;
    if (!aligned16(w_uv) || !aligned16(out)) return MLA_ERR_ALIGN;
  }
  if (parts & kSplit) {
    st = hip_status(mla::launch_decode_splitk(*dims, batch, s_q, q_abs, latent_cache, scales,
                                              num_blocks, block_table, max_blocks, seq_lens, ns,
                                              workspace, stream));
    if (st != MLA_OK) return st;
  }
  if (parts & kMerge)
    st = hip_status(mla::launch_decode_merge(*dims, batch, s_q, q_abs, latent_cache, scales,
                                             num_blocks, block_table, max_blocks, seq_lens, w_uv,
                                             ns, workspace, out, lse, stream));
  return st;
}

}  // namespace

extern "C" {

mla_status mla_decode_splitk(const mla_dims* dims, int32_t batch, int32_t s_q, const void* q_abs,
                             const void* latent_cache, int32_t num_blocks,
                             const int32_t* block_table, int32_t max_blocks,
                             const int32_t* seq_lens, int32_t n_split, void* workspace,
                             size_t ws_bytes, hipStream_t stream) {
  return decode_call(kSplit, dims, batch, s_q, q_abs, latent_cache, nullptr, false, num_blocks,
                     block_table, max_blocks, seq_lens, nullptr, n_split, workspace, ws_bytes,
                     nullptr, nullptr, stream);
}

mla_status mla_decode_merge(const mla_dims* dims, int32_t batch, int32_t s_q, const void* q_abs,
                            const void* latent_cache, int32_t num_blocks,
                            const int32_t* block_table, int32_t max_blocks,
                            const int32_t* seq_lens, const void* w_uv, int32_t n_split,
                            void* workspace, size_t ws_bytes, void* out, float* lse,
                            hipStream_t stream) {
  return decode_call(kMerge, dims, batch, s_q, q_abs, latent_cache, nullptr, false, num_blocks,
                     block_table, max_blocks, seq_lens, w_uv, n_split, workspace, ws_bytes, out,
                     lse, stream);
}

mla_status mla_decode(const mla_dims* dims, int32_t batch, int32_t s_q, const void* q_abs,
                      const void* latent_cache, int32_t num_blocks, const int32_t* block_table,
                      int32_t max_blocks, const int32_t* seq_lens, const void* w_uv,
                      int32_t n_split, void* workspace, size_t ws_bytes, void* out, float* lse,
                      hipStream_t stream) {
  return decode_call(kSplit | kMerge, dims, batch, s_q, q_abs, latent_cache, nullptr, false,
                     num_blocks, block_table, max_blocks, seq_lens, w_uv, n_split, workspace,
                     ws_bytes, out, lse, stream);
}

mla_status mla_decode_fp8(const mla_dims* dims, int32_t batch, int32_t s_q, const void* q_abs,
                          const void* cache_fp8, const float* cache_scale, int32_t num_blocks,
                          const int32_t* block_table, int32_t max_blocks,
                          const int32_t* seq_lens, const void* w_uv, int32_t n_split,
                          void* workspace, size_t ws_bytes, void* out, float* lse,
                          hipStream_t stream) {
  return decode_call(kSplit | kMerge, dims, batch, s_q, q_abs, cache_fp8, cache_scale, true,
                     num_blocks, block_table, max_blocks, seq_lens, w_uv, n_split, workspace,
                     ws_bytes, out, lse, stream);
}

mla_status mla_decode_fp8_splitk(const mla_dims* dims, int32_t batch, int32_t s_q,
                                 const void* q_abs, const void* cache_fp8,
                                 const float* cache_scale, int32_t num_blocks,
                                 const int32_t* block_table, int32_t max_blocks,
                                 const int32_t* seq_lens, int32_t n_split, void* workspace,
                                 size_t ws_bytes, hipStream_t stream) {
  return decode_call(kSplit, dims, batch, s_q, q_abs, cache_fp8, cache_scale, true, num_blocks,
                     block_table, max_blocks, seq_lens, nullptr, n_split, workspace, ws_bytes,
                     nullptr, nullptr, stream);
}

mla_status mla_decode_fp8_merge(const mla_dims* dims, int32_t batch, int32_t s_q,
                                const void* q_abs, const void* cache_fp8,
                                const float* cache_scale, int32_t num_blocks,
                                const int32_t* block_table, int32_t max_blocks,
                                const int32_t* seq_lens, const void* w_uv, int32_t n_split,
                                void* workspace, size_t ws_bytes, void* out, float* lse,
                                hipStream_t stream) {
  return decode_call(kMerge, dims, batch, s_q, q_abs, cache_fp8, cache_scale, true, num_blocks,
                     block_table, max_blocks, seq_lens, w_uv, n_split, workspace, ws_bytes, out,
                     lse, stream);
}

}  // extern "C"

// ---- a whole decode step: the workspace holds, each part 256-byte aligned, the append's
// partial sums, the absorbed queries, the new tokens' sequence and position indices, then the
// decode's own workspace.
namespace {
struct StepLayout {
  size_t y_part, q_abs, idx, dec, total;
};
size_t al256(size_t x) { return (x + 255) / 256 * 256; }
StepLayout step_layout(const mla_dims& d, int32_t batch, int32_t s_q, size_t dec_bytes) {
  StepLayout l;
  const size_t n_tok = static_cast<size_t>(batch) * s_q;
  l.y_part = 0;
  l.q_abs = al256(mla::append_ws_bytes(d, static_cast<int>(n_tok)));
  l.idx = l.q_abs + al256(n_tok * d.n_heads * (d.d_c + d.d_r) * elt_of(d));
  l.dec = l.idx + al256(2 * n_tok * sizeof(int32_t));
  l.total = l.dec + dec_bytes;
  return l;
}
}  // namespace

extern "C" {

size_t mla_decode_step_workspace_bytes(const mla_dims* dims, int32_t batch, int32_t s_q,
                                       int32_t n_split, int32_t max_blocks) {
  const size_t dec = mla_decode_workspace_bytes(dims, batch, s_q, n_split, max_blocks);
  if (dec == 0 || static_cast<int64_t>(batch) * s_q > 65535 * 16) return 0;
  return step_layout(*dims, batch, s_q, dec).total;
}

}  // extern "C"

namespace {

// The decode step over bf16 rows (scales NULL) or e4m3 rows with per-slot scales.
mla_status decode_step(const mla_dims* dims, int32_t batch, int32_t s_q, const void* x,
                       const void* w_dkv, const void* rms_gamma, const void* w_kr,
                       const void* q_nope, const void* q_pe, const void* w_uk, const void* w_uv,
                       void* latent_cache, float* scales, bool fp8, int32_t num_blocks,
                       const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens,
                       int32_t n_split, void* workspace, size_t ws_bytes, void* out, float* lse,
                       hipStream_t stream) {
  mla_status st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (fp8 && (!fp8_rows_ok(*dims) || !mla::mfma_decode_fp8_fits(*dims) ||
              (dims->flags & MLA_FLAG_GENERIC_KERNELS)))
    return MLA_ERR_SHAPE;
  if (batch < 0 || s_q < 1 || max_blocks < 1 || num_blocks < 1 || n_split < 0 ||
      n_split > MLA_MAX_SPLIT)
    return MLA_ERR_RANGE;
  if (batch == 0) return MLA_OK;
  if (static_cast<int64_t>(batch) * s_q > 65535 * 16) return MLA_ERR_RANGE;
  if (!workspace || !seq_lens || !w_uv || !out || (fp8 && !scales)) return MLA_ERR_NULL;
  const size_t need = mla_decode_step_workspace_bytes(dims, batch, s_q, n_split, max_blocks);
  if (need == 0) return MLA_ERR_RANGE;
  if (ws_bytes < need) return MLA_ERR_WORKSPACE;
  if (!aligned16(workspace) || !aligned16(w_uv) || !aligned16(out) ||
      (fp8 && !aligned16(scales)))
    return MLA_ERR_ALIGN;
  const mla_dims& d = *dims;
  const StepLayout l = step_layout(d, batch, s_q, 0);
  char* ws = static_cast<char*>(workspace);
  float* y_part = reinterpret_cast<float*>(ws + l.y_part);
  void* q_abs = ws + l.q_abs;
  int32_t* seq_idx = reinterpret_cast<int32_t*>(ws + l.idx);
  const int n_tok = batch * s_q;
  int32_t* pos = seq_idx + n_tok;
  void* dws = ws + l.dec;
  const size_t dws_bytes = ws_bytes - l.dec;
  // the checks of the calls the step stands for
  st = check_append(dims, n_tok, x, seq_idx, pos, w_dkv, rms_gamma, w_kr, block_table, batch,
                    max_blocks, num_blocks, latent_cache, y_part, l.q_abs - l.y_part);
  if (st != MLA_OK) return st;
  st = check_absorb(dims, batch, s_q, q_nope, q_pe, pos, w_uk, q_abs);
  if (st != MLA_OK) return st;
  int ns = 0;
  st = check_decode(dims, batch, s_q, q_abs, latent_cache, num_blocks, block_table, max_blocks,
                    seq_lens, n_split, dws, dws_bytes, &ns);
  if (st != MLA_OK) return st;
  const bool core_rows = fp8 ? mla::mfma_decode_fp8_fits(d) : mla::mfma_step_fits(d);
  if (core_rows && mla::step_project_fits(d, n_tok)) {
    // three launches: projection with the absorption, the core forming the new rows, merge
    st = hip_status(mla::launch_step_project(d, batch, s_q, x, w_dkv, w_kr, y_part, q_nope, q_pe,
                                             seq_lens, w_uk, q_abs, stream));
    if (st != MLA_OK) return st;
    const mla::StepRows rows{y_part, rms_gamma, latent_cache, fp8 ? scales : nullptr,
                             mla::projection_ksplit(d.d_model), d.rms_eps, d.rope_base};
    st = hip_status(mla::launch_decode_step_splitk(d, batch, s_q, q_abs, latent_cache,
                                                   num_blocks, block_table, max_blocks,
                                                   seq_lens, ns, dws, rows, stream));
  } else {
    // the separate calls, the new tokens' indices written by the device from the lengths
    st = hip_status(mla::launch_step_positions(batch, s_q, seq_lens, seq_idx, pos, stream));
    if (st != MLA_OK) return st;
    st = hip_status(mla::launch_append_absorb(d, n_tok, x, seq_idx, pos, w_dkv, rms_gamma,
                                              w_kr, block_table, batch, max_blocks, num_blocks,
                                              latent_cache, fp8 ? scales : nullptr, y_part,
                                              batch, s_q, q_nope, q_pe, pos, w_uk, q_abs,
                                              stream));
    if (st != MLA_OK) return st;
    st = hip_status(mla::launch_decode_splitk(d, batch, s_q, q_abs, latent_cache,
                                              fp8 ? scales : nullptr, num_blocks, block_table,
                                              max_blocks, seq_lens, ns, dws, stream));
  }
  if (st != MLA_OK) return st;
  return hip_status(mla::launch_decode_merge(d, batch, s_q, q_abs, latent_cache,
                                             fp8 ? scales : nullptr, num_blocks, block_table,
                                             max_blocks, seq_lens, w_uv, ns, dws, out, lse,
                                             stream));
}

}  // namespace

extern "C" {

mla_status mla_decode_step(const mla_dims* dims, int32_t batch, int32_t s_q, const void* x,
                           const void* w_dkv, const void* rms_gamma, const void* w_kr,
                           const void* q_nope, const void* q_pe, const void* w_uk,
                           const void* w_uv, void* latent_cache, int32_t num_blocks,
                           const int32_t* block_table, int32_t max_blocks,
                           const int32_t* seq_lens, int32_t n_split, void* workspace,
                           size_t ws_bytes, void* out, float* lse, hipStream_t stream) {
  return decode_step(dims, batch, s_q, x, w_dkv, rms_gamma, w_kr, q_nope, q_pe, w_uk, w_uv,
                     latent_cache, nullptr, false, num_blocks, block_table, max_blocks, seq_lens,
                     n_split, workspace, ws_bytes, out, lse, stream);
}

mla_status mla_decode_step_fp8(const mla_dims* dims, int32_t batch, int32_t s_q, const void* x,
                               const void* w_dkv, const void* rms_gamma, const void* w_kr,
                               const void* q_nope, const void* q_pe, const void* w_uk,
                               const void* w_uv, void* cache_fp8, float* cache_scale,
                               int32_t num_blocks, const int32_t* block_table,
                               int32_t max_blocks, const int32_t* seq_lens, int32_t n_split,
                               void* workspace, size_t ws_bytes, void* out, float* lse,
                               hipStream_t stream) {
  return decode_step(dims, batch, s_q, x, w_dkv, rms_gamma, w_kr, q_nope, q_pe, w_uk, w_uv,
                     cache_fp8, cache_scale, true, num_blocks, block_table, max_blocks, seq_lens,
                     n_split, workspace, ws_bytes, out, lse, stream);
}

mla_status gqla_expand(const mla_dims* dims, int32_t batch, const void* latent_cache,
                       int32_t num_blocks, const int32_t* block_table, int32_t max_blocks,
                       const int32_t* seq_lens, const int32_t* start_pos, const void* w_uk,
                       const void* w_uv, void* gqa_cache, hipStream_t stream) {
  mla_status st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (batch < 0 || max_blocks < 1 || num_blocks < 1) return MLA_ERR_RANGE;
  if (batch == 0) return MLA_OK;
  if (batch > 65535) return MLA_ERR_RANGE;
  if (static_cast<int64_t>(max_blocks) * dims->block_size > INT32_MAX) return MLA_ERR_RANGE;
  if (!latent_cache || !block_table || !seq_lens || !w_uk || !w_uv || !gqa_cache)
    return MLA_ERR_NULL;
  if (!aligned16(latent_cache) || !aligned16(w_uk) || !aligned16(w_uv) || !aligned16(gqa_cache))
    return MLA_ERR_ALIGN;
  return hip_status(mla::launch_expand(*dims, batch, latent_cache, num_blocks, block_table,
                                       max_blocks, seq_lens, start_pos, w_uk, w_uv, gqa_cache,
                                       stream));
}

size_t gqla_decode_workspace_bytes(const mla_dims* dims, int32_t batch, int32_t s_q,
                                   int32_t n_split, int32_t max_blocks) {
  if (check_dims(dims) != MLA_OK || batch < 1 || s_q < 1 || max_blocks < 1 || n_split < 0 ||
      n_split > MLA_MAX_SPLIT)
    return 0;
  const int ns = n_split == 0 ? resolve_split(*dims, batch, s_q, max_blocks) : n_split;
  return mla::partials_bytes(batch, s_q, dims->n_heads, ns, dims->d_v, elt_of(*dims));
}

mla_status gqla_decode(const mla_dims* dims, int32_t batch, int32_t s_q, const void* q_nope,
                       const void* q_pe, const int32_t* q_pos, const void* gqa_cache,
                       int32_t num_blocks, const int32_t* block_table, int32_t max_blocks,
                       const int32_t* seq_lens, int32_t n_split, void* workspace,
                       size_t ws_bytes, void* out, float* lse, hipStream_t stream) {
  mla_status st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (batch < 0 || s_q < 1 || max_blocks < 1 || num_blocks < 1 || n_split < 0 ||
      n_split > MLA_MAX_SPLIT)
    return MLA_ERR_RANGE;
  if (batch == 0) return MLA_OK;
  if (batch > 65535 || s_q > 65535 || static_cast<int64_t>(batch) * s_q > 65535)
    return MLA_ERR_RANGE;
  if (static_cast<int64_t>(max_blocks) * dims->block_size > INT32_MAX) return MLA_ERR_RANGE;
  if (!q_nope || !q_pos || !gqa_cache || !block_table || !seq_lens || !out ||
      (dims->d_r > 0 && !q_pe))
    return MLA_ERR_NULL;
  if (!aligned16(q_nope) || (q_pe && !aligned16(q_pe)) || !aligned16(gqa_cache) || !aligned16(out))
    return MLA_ERR_ALIGN;
  const int ns = n_split == 0 ? resolve_split(*dims, batch, s_q, max_blocks) : n_split;
  const size_t need = mla::partials_bytes(batch, s_q, dims->n_heads, ns, dims->d_v, elt_of(*dims));
  if (workspace == nullptr || ws_bytes < need) return MLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MLA_ERR_ALIGN;
  return hip_status(mla::launch_gqa_decode(*dims, batch, s_q, q_nope, q_pe, q_pos, gqa_cache,
                                           num_blocks, block_table, max_blocks, seq_lens, ns,
                                           workspace, out, lse, stream));
}

size_t mla_prefill_workspace_bytes(const mla_dims* dims, int32_t batch, int32_t s_q,
                                   int32_t num_blocks, int32_t max_blocks) {
  if (check_dims(dims) != MLA_OK || batch < 1 || s_q < 1 || num_blocks < 1 || max_blocks < 1)
    return 0;
  const size_t dec = gqla_decode_workspace_bytes(dims, batch, s_q, 0, max_blocks);
  return dec == 0 ? 0 : prefill_kv_bytes(*dims, num_blocks) + dec;
}

mla_status mla_prefill(const mla_dims* dims, int32_t batch, int32_t s_q, const void* q_nope,
                       const void* q_pe, const int32_t* q_pos, const void* latent_cache,
                       int32_t num_blocks, const int32_t* block_table, int32_t max_blocks,
                       const int32_t* seq_lens, const void* w_uk, const void* w_uv,
                       void* workspace, size_t ws_bytes, void* out, float* lse,
                       hipStream_t stream) {
  mla_status st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (batch < 0 || s_q < 1 || max_blocks < 1 || num_blocks < 1) return MLA_ERR_RANGE;
  if (batch == 0) return MLA_OK;
  const size_t need = mla_prefill_workspace_bytes(dims, batch, s_q, num_blocks, max_blocks);
  if (need == 0) return MLA_ERR_RANGE;
  if (workspace == nullptr || ws_bytes < need) return MLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MLA_ERR_ALIGN;
  // the checks of both calls below, made before either enqueues anything
  if (batch > 65535 || s_q > 65535 || static_cast<int64_t>(batch) * s_q > 65535 ||
      static_cast<int64_t>(max_blocks) * dims->block_size > INT32_MAX)
    return MLA_ERR_RANGE;
  if (!q_nope || !q_pos || !out || (dims->d_r > 0 && !q_pe) || !latent_cache || !block_table ||
      !seq_lens || !w_uk || !w_uv)
    return MLA_ERR_NULL;
  if (!aligned16(q_nope) || (q_pe && !aligned16(q_pe)) || !aligned16(out) ||
      !aligned16(latent_cache) || !aligned16(w_uk) || !aligned16(w_uv))
    return MLA_ERR_ALIGN;
  // every head's (or group's) keys and values of the sequences' positions, then attention
  // over them
  const size_t kv = prefill_kv_bytes(*dims, num_blocks);
  char* dec_ws = static_cast<char*>(workspace) + kv;
  st = gqla_expand(dims, batch, latent_cache, num_blocks, block_table, max_blocks, seq_lens,
                   nullptr, w_uk, w_uv, workspace, stream);
  if (st != MLA_OK) return st;
  return gqla_decode(dims, batch, s_q, q_nope, q_pe, q_pos, workspace, num_blocks, block_table,
                     max_blocks, seq_lens, 0, dec_ws, ws_bytes - kv, out, lse, stream);
}

mla_status mla_validate_block_table(const mla_dims* dims, const int32_t* host_table,
                                    int32_t batch, int32_t max_blocks,
                                    const int32_t* host_seq_lens, int32_t num_blocks) {
  if (dims == nullptr || host_table == nullptr || host_seq_lens == nullptr) return MLA_ERR_NULL;
  if (dims->block_size < 1) return MLA_ERR_SHAPE;
  if (batch < 0 || max_blocks < 1 || num_blocks < 1) return MLA_ERR_RANGE;
  const int64_t cap = static_cast<int64_t>(max_blocks) * dims->block_size;
  for (int b = 0; b < batch; ++b) {
    if (host_seq_lens[b] < 0 || host_seq_lens[b] > cap) return MLA_ERR_RANGE;
  }
  for (int b = 0; b < batch; ++b) {
    const int nb = cdiv(host_seq_lens[b], dims->block_size);
    for (int j = 0; j < nb; ++j) {
      const int id = host_table[static_cast<int64_t>(b) * max_blocks + j];
      if (id < 0 || id >= num_blocks) return MLA_ERR_BLOCK_TABLE;
    }
  }
  // A block used twice: sweep the id space in 64Ki-id windows with a bitmap on the stack
  // (the library allocates nothing).
  constexpr int kWin = 1 << 16;
  uint64_t seen[kWin / 64];
  for (int64_t lo = 0; lo < num_blocks; lo += kWin) {
    for (int i = 0; i < kWin / 64; ++i) seen[i] = 0;
    for (int b = 0; b < batch; ++b) {
      const int nb = cdiv(host_seq_lens[b], dims->block_size);
      for (int j = 0; j < nb; ++j) {
        const int64_t id = host_table[static_cast<int64_t>(b) * max_blocks + j];
        if (id < lo || id >= lo + kWin) continue;
        const int64_t r = id - lo;
        const uint64_t bit = 1ull << (r & 63);
        if (seen[r >> 6] & bit) return MLA_ERR_BLOCK_TABLE;
        seen[r >> 6] |= bit;
      }
    }
  }
  return MLA_OK;
}

}  // extern "C"
