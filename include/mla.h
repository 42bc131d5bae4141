/*
 * mla.h -- C ABI of libmla.so: multi-head latent attention (MLA) decode over a compressed,
 * paged latent KV cache, and the grouped GQLA variant, on AMD MI355X (gfx950).
 *
 * The operations follow these pages:
 *  [Smallem]  smallbard.com, Smallem article 13, "L'attention latente : compresser le cache"
 *  [KV-cache] mkdocs.reaper.mx, DeepSeek-V4.1-Flash, "Le cache clé-valeur"
 *  [Slides]   cours.spawnkit.ai, session 18 slides, "Cache KV, mémoire récurrente, MLA et bas rang"
 *  [GQLA]     gist.science summary of arXiv 2605.15250, "GQLA – Attention Latente par Groupes
 *             de Requêtes pour le Décodage Adaptatif au Matériel"
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Notation: C = d_model, H = n_heads (h_q), D = d_nope (d_h), D_v = d_v, d_c = latent width
 *    (r_kv), d_r = shared rotary key width (d^R_h), G = n_groups, bs = block_size.
 *  - Weights are row-major [in, out]: a row vector multiplies them from the left, as the pages
 *    write x · W. Group g of W_UK / W_UV is columns [g*D, (g+1)*D) / [g*D_v, (g+1)*D_v);
 *    head h belongs to group h / (H / G) ([GQLA] section 2, "Architecture"). G == H is MLA.
 *  - Latent cache: [num_blocks, bs, d_c + d_r]; row = [c || k_r] with k_r already rotated.
 *    Position p of sequence b lives in slot block_table[b*max_blocks + p/bs]*bs + p%bs.
 *  - Expanded GQA cache: [num_blocks, bs, G*D + G*D_v + d_r]; row =
 *    [K_0 .. K_{G-1} || V_0 .. V_{G-1} || k_r], same block table as the latent cache.
 *  - RoPE: pair (2j, 2j+1) of a d_r-wide vector turns by pos * rope_base^(-2j/d_r), the
 *    angle formed in double precision; positions are 0-based.
 *  - A step appends s_q positions per sequence first; seq_lens[b] = L_b counts them, and query
 *    i (0-based) of sequence b sits at position L_b - s_q + i and sees positions 0 .. itself.
 *  - Every float tensor (activations, weights, caches, q_abs, out) has type dims->dtype; all
 *    arithmetic accumulates in fp32; bf16 results round to nearest, ties to even. lse is fp32.
 *  - Ownership: the caller owns every buffer (device memory unless noted) and the stream.
 *    The library allocates nothing, frees nothing, never synchronises and keeps no state, so
 *    calls are reentrant (the one exception, mla_decode_noalloc, keeps its partials in a
 *    device array of its own). Work is enqueued on `stream` (NULL = the default stream) and the
 *    call returns at once. Device pointers must be 16-byte aligned.
 *  - Errors: the status is decided on the host before anything is enqueued, except
 *    MLA_ERR_HIP, which reports a failed launch. Nothing is printed and nothing aborts.
 *    Integer arrays that live on the device (block tables, positions, lengths) are not read on
 *    the host: kernels clamp what they use to the buffers they were given (a block id outside
 *    [0, num_blocks), or a position past max_blocks*bs, leaves that position out), so a bad
 *    table cannot make them touch memory out of bounds. mla_validate_block_table() checks a
 *    host copy for callers who want the error instead.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MLA_F32 = 0, MLA_BF16 = 1 } mla_dtype;

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = -1,        /* a required pointer is NULL */
  MLA_ERR_SHAPE = -2,       /* a dimension is out of range or inconsistent */
  MLA_ERR_DTYPE = -3,       /* dims->dtype is not an mla_dtype */
  MLA_ERR_RANGE = -4,       /* a count (batch, s_q, n_tok, n_split, ...) is out of range */
  MLA_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than the *_workspace_bytes() size */
  MLA_ERR_ALIGN = -6,       /* a device pointer is not 16-byte aligned */
  MLA_ERR_HIP = -7,         /* a kernel launch failed */
  MLA_ERR_BLOCK_TABLE = -8, /* mla_validate_block_table(): bad or shared block id */
  MLA_STATUS_INT32_ = 0x7fffffff /* not a status: gives the type the range of an int32, so
                                    that any int a caller passes (mla_status_string) is a
                                    valid value of it */
} mla_status;

/* dims->flags bits */
#define MLA_FLAG_GENERIC_KERNELS 1 /* use the portable kernels even where an MFMA kernel fits */

/* Largest split count mla_decode / gqla_decode accept. */
#define MLA_MAX_SPLIT 256

typedef struct mla_dims {
  int32_t d_model;     /* C: width of the hidden states appended to the cache */
  int32_t n_heads;     /* H: query heads */
  int32_t d_nope;      /* D: per-head content (non-rotary) query/key width */
  int32_t d_v;         /* D_v: per-head value width (a multiple of 8) */
  int32_t d_c;         /* d_c: latent width (a multiple of 8) */
  int32_t d_r;         /* d_r: shared rotary key width (even, may be 0) */
  int32_t n_groups;    /* G: groups indexing W_UK / W_UV; divides H; G == H is plain MLA */
  int32_t block_size;  /* bs: positions per cache block */
  int32_t dtype;       /* mla_dtype of every float tensor */
  int32_t flags;       /* MLA_FLAG_* */
  float rope_base;     /* RoPE base, e.g. 10000 */
  float rms_eps;       /* epsilon of the latent RMSNorm */
  float softmax_scale; /* 0 selects 1/sqrt(D + d_r) */
} mla_dims;

/*
 * mla_cache_append -- write the cache row of n_tok new positions ([Smallem] "L'idée : garder
 * un résumé", "L'obstacle : RoPE" and the cache extension in "Le code"; [Slides] "Carte du
 * mécanisme"):
 *     c   = RMSNorm(x · W_DKV) * gamma,  RMSNorm(y) = y / sqrt(mean_j y_j^2 + rms_eps)
 *     k_r = RoPE(x · W_KR, pos)
 *     latent_cache[slot(seq_idx[n], pos[n])] = [c || k_r]
 *  x [n_tok, C]; seq_idx, pos int32 [n_tok] (device); w_dkv [C, d_c]; rms_gamma [d_c];
 *  w_kr [C, d_r]; block_table int32 [batch, max_blocks] (device); latent_cache as above.
 *  Every new position must have its own slot (two tokens writing one slot race).
 *  workspace: at least mla_cache_append_workspace_bytes(dims, n_tok) bytes of device memory.
 *  n_tok == 0 enqueues nothing and returns MLA_OK. Tokens whose slot falls outside the cache
 *  (negative id, id >= num_blocks, position >= max_blocks*bs, seq_idx outside [0, batch)) are
 *  not written.
 */
size_t mla_cache_append_workspace_bytes(const mla_dims* dims, int32_t n_tok);
mla_status mla_cache_append(const mla_dims* dims, int32_t n_tok, const void* x,
                            const int32_t* seq_idx, const int32_t* pos, const void* w_dkv,
                            const void* rms_gamma, const void* w_kr, const int32_t* block_table,
                            int32_t batch, int32_t max_blocks, int32_t num_blocks,
                            void* latent_cache, void* workspace, size_t ws_bytes,
                            hipStream_t stream);

/*
 * mla_absorb_q -- carry the queries into latent space once ([Smallem] "Ce que DeepSeek fait de
 * plus": q · (c · W) = (q · W^T) · c; [GQLA] "Chemin MQA-Absorbé" with group-indexed W_UK):
 *     q_abs[b,i,h] = [ q_nope[b,i,h] · W_UK[:, g(h)]^T  ||  RoPE(q_pe[b,i,h], q_pos[b,i]) ]
 *  q_nope [batch, s_q, H, D]; q_pe [batch, s_q, H, d_r]; q_pos int32 [batch, s_q] (device);
 *  w_uk [d_c, G*D]; q_abs [batch, s_q, H, d_c + d_r] (output).
 */
mla_status mla_absorb_q(const mla_dims* dims, int32_t batch, int32_t s_q, const void* q_nope,
                        const void* q_pe, const int32_t* q_pos, const void* w_uk, void* q_abs,
                        hipStream_t stream);

/*
 * mla_cache_append_absorb_q -- mla_cache_append(dims, n_tok, x, ..., workspace, ws_bytes)
 *  followed by mla_absorb_q(dims, batch, s_q, q_nope, q_pe, q_pos, w_uk, q_abs), the two
 *  independent calls that open a decode step. On the matrix-core path (bf16) the absorption
 *  runs in the same launch as the append's projection (two launches for both instead of
 *  three); otherwise the two calls run in order. batch is both the block table's row count and
 *  the number of query sequences. Arguments, results, errors and the workspace are those of
 *  the two calls.
 */
mla_status mla_cache_append_absorb_q(const mla_dims* dims, int32_t n_tok, const void* x,
                                     const int32_t* seq_idx, const int32_t* pos,
                                     const void* w_dkv, const void* rms_gamma, const void* w_kr,
                                     const int32_t* block_table, int32_t batch,
                                     int32_t max_blocks, int32_t num_blocks, void* latent_cache,
                                     void* workspace, size_t ws_bytes, int32_t s_q,
                                     const void* q_nope, const void* q_pe, const int32_t* q_pos,
                                     const void* w_uk, void* q_abs, hipStream_t stream);

/*
 * mla_decode -- absorbed decode over the latent cache ([Smallem] "Ce que DeepSeek fait de plus";
 * [GQLA] "Chemin MQA-Absorbé"): for every sequence b, query i and head h,
 *     z_t = scale * (q_abs[b,i,h] . row_t)          for visible positions t
 *     o   = sum_t softmax(z)_t * c_t                (the latent part of the rows)
 *     out[b,i,h] = o · W_UV[:, g(h)],   lse[b,i,h] = log sum_t exp(z_t)
 *  The history is split into n_split chunks per (sequence, query) that are reduced
 *  independently and merged by their log-sum-exp; the result does not depend on n_split
 *  beyond rounding.
 *  q_abs [batch, s_q, H, d_c + d_r]; block_table int32 [batch, max_blocks], seq_lens int32
 *  [batch] (device; s_q <= L_b <= max_blocks*bs expected: a query with no visible position
 *  gets out = 0 and lse = -inf); w_uv [d_c, G*D_v]; out [batch, s_q, H, D_v];
 *  lse fp32 [batch, s_q, H] or NULL.
 *  n_split: 1 .. MLA_MAX_SPLIT uniform chunks per (sequence, query), or 0 to let the library
 *  choose. With 0, bf16 caches on the matrix-core path (d_c 512, d_r 64, D_v 128, block size
 *  a multiple of 32) with batch * s_q <= 128 take a length-balanced plan made on the device
 *  from seq_lens: every row is cut into chunks of one common size, the smallest multiple of 64
 *  for which all rows need at most 256 chunks (at most 64 per row), so rows of mixed lengths
 *  keep every CU busy; other cases take mla_auto_split(...) uniform chunks.
 *  workspace: mla_decode_workspace_bytes(dims, batch, s_q, n_split, max_blocks) bytes (for
 *  n_split = 0 the size of whichever scheme applies).
 */
size_t mla_decode_workspace_bytes(const mla_dims* dims, int32_t batch, int32_t s_q,
                                  int32_t n_split, int32_t max_blocks);
mla_status mla_decode(const mla_dims* dims, int32_t batch, int32_t s_q, const void* q_abs,
                      const void* latent_cache, int32_t num_blocks, const int32_t* block_table,
                      int32_t max_blocks, const int32_t* seq_lens, const void* w_uv,
                      int32_t n_split, void* workspace, size_t ws_bytes, void* out, float* lse,
                      hipStream_t stream);

/*
 * The two halves of mla_decode, for callers that time or schedule them separately; calling
 * mla_decode_splitk then mla_decode_merge on one stream with the same arguments and workspace
 * is exactly mla_decode.
 *  mla_decode_splitk -- every (split, query, sequence) reduces its positions and writes its
 *    partial (o / l, log2-domain lse) into the workspace.
 *  mla_decode_merge -- merges the partials of each (sequence, query, head) by their
 *    log-sum-exp and applies the head's group of W_UV; q_abs, cache, table and lengths are
 *    read again only for splits the matrix-core kernel flagged for exact recomputation
 *    (scores that outgrew its fixed per-head reference by 2^64).
 */
mla_status mla_decode_splitk(const mla_dims* dims, int32_t batch, int32_t s_q, const void* q_abs,
                             const void* latent_cache, int32_t num_blocks,
                             const int32_t* block_table, int32_t max_blocks,
                             const int32_t* seq_lens, int32_t n_split, void* workspace,
                             size_t ws_bytes, hipStream_t stream);
mla_status mla_decode_merge(const mla_dims* dims, int32_t batch, int32_t s_q, const void* q_abs,
                            const void* latent_cache, int32_t num_blocks,
                            const int32_t* block_table, int32_t max_blocks,
                            const int32_t* seq_lens, const void* w_uv, int32_t n_split,
                            void* workspace, size_t ws_bytes, void* out, float* lse,
                            hipStream_t stream);

/*
 * mla_decode_step -- one decode step of one layer over the latent cache ([Smallem] "Le code":
 * the cache is extended by the new tokens, then attended over its whole length; "Ce que
 * DeepSeek fait de plus" for the absorbed form): the s_q new tokens of every sequence b are
 * its positions L_b - s_q .. L_b - 1 (L_b = seq_lens[b], already counting them), token
 * n = b * s_q + i of x and of the queries. Results are those of
 *     mla_cache_append_absorb_q(dims, B * s_q, x, seq_idx, pos, w_dkv, rms_gamma, w_kr, ...,
 *                               s_q, q_nope, q_pe, q_pos = pos, w_uk, q_abs)
 *     mla_decode(dims, B, s_q, q_abs, latent_cache, ..., w_uv, n_split, ..., out, lse)
 *  with seq_idx[n] = n / s_q and pos[n] = L_b - s_q + n % s_q, bit for bit; the new rows are
 *  left in the cache. On the matrix-core path (bf16, d_c 512, d_r 64, H = 128, block size a
 *  multiple of 32, B * s_q <= 2048) the step takes three launches instead of four: the split-K
 *  core forms the new rows itself, each split workgroup those inside its range, from the
 *  projection's partial sums.
 *  x [B * s_q, C]; q_nope [B, s_q, H, D]; q_pe [B, s_q, H, d_r]; other arguments as in the
 *  calls above. workspace: mla_decode_step_workspace_bytes(dims, B, s_q, n_split, max_blocks)
 *  bytes (the append's partial sums, the absorbed queries, the new tokens' indices, then the
 *  decode's workspace). Errors: those of the calls above; nothing is enqueued when a check fails.
 */
size_t mla_decode_step_workspace_bytes(const mla_dims* dims, int32_t batch, int32_t s_q,
                                       int32_t n_split, int32_t max_blocks);
mla_status mla_decode_step(const mla_dims* dims, int32_t batch, int32_t s_q, const void* x,
                           const void* w_dkv, const void* rms_gamma, const void* w_kr,
                           const void* q_nope, const void* q_pe, const void* w_uk,
                           const void* w_uv, void* latent_cache, int32_t num_blocks,
                           const int32_t* block_table, int32_t max_blocks,
                           const int32_t* seq_lens, int32_t n_split, void* workspace,
                           size_t ws_bytes, void* out, float* lse, hipStream_t stream);

/*
 * mla_decode_noalloc -- mla_decode for callers that cannot allocate device memory: code under
 *  HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. Arguments, results
 *  and errors are mla_decode's, without workspace and ws_bytes: the split-K partials live in a
 *  file-scope device array of MLA_NOALLOC_SCRATCH_BYTES inside the library. Each GPU the call
 *  runs on holds its own copy until the process ends (its device address is looked up on the
 *  first call made with that device current); the call itself allocates and frees nothing.
 *  Limits: a batch whose mla_decode_workspace_bytes(dims, batch, s_q, n_split, max_blocks)
 *  exceeds MLA_NOALLOC_SCRATCH_BYTES is rejected with MLA_ERR_WORKSPACE (36 MiB holds the
 *  length-balanced plan of any batch, and uniform splits of up to 32,768 query rows x heads x
 *  splits with d_c = 512 in bf16). All calls on one GPU share its array, which keeps the last
 *  call's contents: calls that overlap on one GPU (two streams or two threads) race and must
 *  be ordered by the caller. Nothing in the array needs clearing between calls. MLA_ERR_HIP
 *  also reports a failed lookup of the array.
 */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)36 << 20)
mla_status mla_decode_noalloc(const mla_dims* dims, int32_t batch, int32_t s_q,
                              const void* q_abs, const void* latent_cache, int32_t num_blocks,
                              const int32_t* block_table, int32_t max_blocks,
                              const int32_t* seq_lens, const void* w_uv, int32_t n_split,
                              void* out, float* lse, hipStream_t stream);

/*
 * FP8 latent cache. The pages count the bytes of one cache entry among the costs to cut and
 * list quantisation among the ways to cut them, down to FP4 for the "CSA2" design's latent
 * ([KV-cache] "Les trois dimensions de compression": the entry-size row of its table and
 * CSA2's 512-channel FP4 latent; [Slides] trainer notes on the INT8 check: one byte per value
 * halves the cache). They fix no format; this library stores a row as OCP FP8 E4M3 bytes (sign, 4
 * exponent bits of bias 7, 3 mantissa bits; largest finite value 448, smallest subnormal
 * 2^-9, no infinities) and one fp32 scale per position:
 *     scale = the smallest power of two s with max_j |row_j| <= 448 s   (1 for a zero row)
 *     byte_j = e4m3(row_j / s), rounded to nearest, ties to the even code
 *     row_j ~ value(byte_j) * s   (exact in bf16)
 *  A row costs d_c + d_r bytes plus 4 (580 instead of 1,152 for d_c 512, d_r 64). The rows
 *  quantised are bf16 values: those the bf16 call (mla_cache_append) would have written.
 *  Layout: cache_fp8 uint8 [num_blocks, bs, d_c + d_r] and cache_scale fp32 [num_blocks, bs],
 *  both indexed by slot = block_table[b][p / bs] * bs + p % bs; owned by the caller.
 *  Shapes: dims->dtype MLA_BF16 (every float tensor other than the cache), d_c + d_r a
 *  multiple of 16 and at most 1024 (MLA_ERR_SHAPE otherwise).
 *
 * mla_cache_quantize_fp8 -- n_rows contiguous bf16 rows [n_rows, d_c + d_r] (a whole bf16
 *  cache: n_rows = num_blocks * bs) to rows_fp8 uint8 [n_rows, d_c + d_r] and row_scale fp32
 *  [n_rows]. n_rows == 0 enqueues nothing.
 * mla_cache_append_fp8 -- mla_cache_append writing e4m3 rows and their scales (arguments,
 *  workspace and errors otherwise mla_cache_append's).
 * mla_cache_append_absorb_q_fp8 -- mla_cache_append_absorb_q writing e4m3 rows; s_q == 0
 *  leaves out the absorption (q_nope, q_pe, q_pos, w_uk, q_abs are then not read).
 */
mla_status mla_cache_quantize_fp8(const mla_dims* dims, int64_t n_rows, const void* rows,
                                  void* rows_fp8, float* row_scale, hipStream_t stream);
mla_status mla_cache_append_fp8(const mla_dims* dims, int32_t n_tok, const void* x,
                                const int32_t* seq_idx, const int32_t* pos, const void* w_dkv,
                                const void* rms_gamma, const void* w_kr,
                                const int32_t* block_table, int32_t batch, int32_t max_blocks,
                                int32_t num_blocks, void* cache_fp8, float* cache_scale,
                                void* workspace, size_t ws_bytes, hipStream_t stream);
mla_status mla_cache_append_absorb_q_fp8(const mla_dims* dims, int32_t n_tok, const void* x,
                                         const int32_t* seq_idx, const int32_t* pos,
                                         const void* w_dkv, const void* rms_gamma,
                                         const void* w_kr, const int32_t* block_table,
                                         int32_t batch, int32_t max_blocks, int32_t num_blocks,
                                         void* cache_fp8, float* cache_scale, void* workspace,
                                         size_t ws_bytes, int32_t s_q, const void* q_nope,
                                         const void* q_pe, const int32_t* q_pos,
                                         const void* w_uk, void* q_abs, hipStream_t stream);

/*
 * mla_decode_fp8, mla_decode_fp8_splitk, mla_decode_fp8_merge -- mla_decode, mla_decode_splitk
 *  and mla_decode_merge over an e4m3 cache (cache_fp8, cache_scale as above): every row is
 *  read as value(byte) * scale, which is exact in bf16, so the result is that of the bf16
 *  calls on the dequantised cache, bit for bit, from half the cache bytes. Shapes: H = 128,
 *  d_c 512, d_r 64, D_v 128, block size a multiple of 32, dims->dtype MLA_BF16, no
 *  MLA_FLAG_GENERIC_KERNELS (MLA_ERR_SHAPE otherwise). Workspace sizes, n_split, errors and
 *  the exact recomputation of flagged splits are those of the bf16 calls.
 */
mla_status mla_decode_fp8(const mla_dims* dims, int32_t batch, int32_t s_q, const void* q_abs,
                          const void* cache_fp8, const float* cache_scale, int32_t num_blocks,
                          const int32_t* block_table, int32_t max_blocks,
                          const int32_t* seq_lens, const void* w_uv, int32_t n_split,
                          void* workspace, size_t ws_bytes, void* out, float* lse,
                          hipStream_t stream);
mla_status mla_decode_fp8_splitk(const mla_dims* dims, int32_t batch, int32_t s_q,
                                 const void* q_abs, const void* cache_fp8,
                                 const float* cache_scale, int32_t num_blocks,
                                 const int32_t* block_table, int32_t max_blocks,
                                 const int32_t* seq_lens, int32_t n_split, void* workspace,
                                 size_t ws_bytes, hipStream_t stream);
mla_status mla_decode_fp8_merge(const mla_dims* dims, int32_t batch, int32_t s_q,
                                const void* q_abs, const void* cache_fp8,
                                const float* cache_scale, int32_t num_blocks,
                                const int32_t* block_table, int32_t max_blocks,
                                const int32_t* seq_lens, const void* w_uv, int32_t n_split,
                                void* workspace, size_t ws_bytes, void* out, float* lse,
                                hipStream_t stream);

/*
 * mla_decode_step_fp8 -- mla_decode_step over an e4m3 cache (cache_fp8, cache_scale as in
 *  mla_cache_append_fp8): results are those of
 *     mla_cache_append_absorb_q_fp8(dims, B * s_q, x, seq_idx, pos, ..., cache_fp8,
 *                                   cache_scale, ..., s_q, q_nope, q_pe, q_pos = pos, w_uk, q_abs)
 *     mla_decode_fp8(dims, B, s_q, q_abs, cache_fp8, cache_scale, ..., w_uv, n_split, ...)
 *  bit for bit (the new rows' bytes and scales left in the cache). The split-K core quantises
 *  the new rows itself, by the append's rule, when B * s_q <= 2048 and C % 8 == 0; otherwise
 *  the step runs the separate calls. Shapes, workspace (mla_decode_step_workspace_bytes) and
 *  errors as for mla_decode_step and mla_decode_fp8.
 */
mla_status mla_decode_step_fp8(const mla_dims* dims, int32_t batch, int32_t s_q, const void* x,
                               const void* w_dkv, const void* rms_gamma, const void* w_kr,
                               const void* q_nope, const void* q_pe, const void* w_uk,
                               const void* w_uv, void* cache_fp8, float* cache_scale,
                               int32_t num_blocks, const int32_t* block_table,
                               int32_t max_blocks, const int32_t* seq_lens, int32_t n_split,
                               void* workspace, size_t ws_bytes, void* out, float* lse,
                               hipStream_t stream);

/*
 * gqla_expand -- expand latent rows into the GQA cache once ([GQLA] "Chemin GQA"):
 *     gqa_row = [c · W_UK[:, 0] .. c · W_UK[:, G-1] || c · W_UV[:, 0] .. c · W_UV[:, G-1] || k_r]
 *  for positions start_pos[b] .. seq_lens[b]-1 of every sequence (start_pos NULL: from 0).
 *  The GQA cache shares the latent cache's block table and block size.
 */
mla_status gqla_expand(const mla_dims* dims, int32_t batch, const void* latent_cache,
                       int32_t num_blocks, const int32_t* block_table, int32_t max_blocks,
                       const int32_t* seq_lens, const int32_t* start_pos, const void* w_uk,
                       const void* w_uv, void* gqa_cache, hipStream_t stream);

/*
 * gqla_decode -- standard grouped-query decode over the expanded cache ([GQLA] "Chemin GQA"):
 * head h of group g compares [q_nope ; RoPE(q_pe, q_pos)] with [K_g ; k_r] and averages V_g.
 *  q_nope [batch, s_q, H, D]; q_pe [batch, s_q, H, d_r]; q_pos int32 [batch, s_q] (device);
 *  out [batch, s_q, H, D_v]; lse as in mla_decode; seq_lens and n_split as in mla_decode.
 *  workspace: gqla_decode_workspace_bytes(dims, batch, s_q, n_split, max_blocks) bytes.
 */
size_t gqla_decode_workspace_bytes(const mla_dims* dims, int32_t batch, int32_t s_q,
                                   int32_t n_split, int32_t max_blocks);
mla_status gqla_decode(const mla_dims* dims, int32_t batch, int32_t s_q, const void* q_nope,
                       const void* q_pe, const int32_t* q_pos, const void* gqa_cache,
                       int32_t num_blocks, const int32_t* block_table, int32_t max_blocks,
                       const int32_t* seq_lens, int32_t n_split, void* workspace,
                       size_t ws_bytes, void* out, float* lse, hipStream_t stream);

/*
 * mla_prefill -- attention of many new tokens per sequence over the latent cache, in the
 * expanded form that the no-cache (training) pass uses ([Smallem] "Le code": keys and values
 * of every head are key_up and value_up of the latent; "Deux produits ou une concaténation ?":
 * one score product over the concatenation [k_nope ; k_r] and [q_nope ; q_r]):
 *     K_h(p) = c_p · W_UK[:, g(h)],  V_h(p) = c_p · W_UV[:, g(h)]   for every visible p
 *     out_h(i) = softmax_p(([q_nope,h ; RoPE(q_pe,h, q_pos)] · [K_h(p) ; k_r(p)]) * scale) · V_h
 *  with the causal visibility of mla_decode (query i of a sequence of length L sees positions
 *  0 .. L - s_q + i). G = H is MLA (one key and value per head); G < H is the GQLA grouping.
 *  Arguments as in mla_decode (q_nope [batch, s_q, H, D], q_pe [batch, s_q, H, d_r], q_pos,
 *  latent_cache [num_blocks, bs, d_c + d_r], block_table, seq_lens) and gqla_expand (w_uk,
 *  w_uv [d_c, G * D] and [d_c, G * D_v]); out [batch, s_q, H, D_v]; lse as in mla_decode
 *  (nullable). The rows of the new tokens must already be in the cache (mla_cache_append).
 *  The call expands positions 0 .. seq_lens[b] - 1 of every sequence into the workspace
 *  (laid out as a GQA cache of num_blocks blocks under the same block table), then runs the
 *  grouped-query attention over it; a chunked prefill that keeps its expanded cache between
 *  chunks calls gqla_expand (start_pos = the chunk) and gqla_decode itself instead.
 *  workspace: at least mla_prefill_workspace_bytes(dims, batch, s_q, num_blocks, max_blocks)
 *  bytes (num_blocks * block_size * (G * (D + D_v) + d_r) elements, then gqla_decode's).
 *  Errors: as gqla_expand and gqla_decode; nothing is enqueued when a check fails.
 */
size_t mla_prefill_workspace_bytes(const mla_dims* dims, int32_t batch, int32_t s_q,
                                   int32_t num_blocks, int32_t max_blocks);
mla_status mla_prefill(const mla_dims* dims, int32_t batch, int32_t s_q, const void* q_nope,
                       const void* q_pe, const int32_t* q_pos, const void* latent_cache,
                       int32_t num_blocks, const int32_t* block_table, int32_t max_blocks,
                       const int32_t* seq_lens, const void* w_uk, const void* w_uv,
                       void* workspace, size_t ws_bytes, void* out, float* lse,
                       hipStream_t stream);

/* Uniform split count n_split = 0 resolves to for these sizes where the length-balanced plan
 * of mla_decode does not apply (and the count gqla_decode uses for n_split = 0). */
int32_t mla_auto_split(const mla_dims* dims, int32_t batch, int32_t s_q, int32_t max_blocks);

/*
 * mla_query_project -- the query side of the layer, before mla_absorb_q ([Smallem] "Le code":
 * query_down, query_norm, query_up and query_rope; "L'obstacle : RoPE": the queries' rotary
 * part comes from their own latent c_q):
 *     c_q    = RMSNorm(x · W_DQ) * gamma_q        [d_q]   (rounded once to the dtype)
 *     q_nope = c_q · W_UQ                         [H, D]
 *     q_pe   = c_q · W_QR                         [H, d_r] (not rotated: mla_absorb_q rotates)
 *  x [n_tok, C]; w_dq [C, d_q]; gamma_q [d_q]; w_uq [d_q, H*D]; w_qr [d_q, H*d_r] (NULL when
 *  d_r = 0); q_nope [n_tok, H, D] and q_pe [n_tok, H, d_r] (outputs, q_pe NULL when d_r = 0).
 *  RMSNorm as in mla_cache_append (dims->rms_eps). n_tok == 0 enqueues nothing.
 *  workspace: at least mla_query_project_workspace_bytes(dims, n_tok, d_q) bytes.
 */
size_t mla_query_project_workspace_bytes(const mla_dims* dims, int32_t n_tok, int32_t d_q);
mla_status mla_query_project(const mla_dims* dims, int32_t n_tok, int32_t d_q, const void* x,
                             const void* w_dq, const void* gamma_q, const void* w_uq,
                             const void* w_qr, void* q_nope, void* q_pe, void* workspace,
                             size_t ws_bytes, hipStream_t stream);

/*
 * mla_output_project -- the layer's output projection, after mla_decode ([Smallem] "Le code",
 * proj, a linear layer with bias):
 *     y = o · W_O + b_O
 *  o [n_tok, H*D_v] (mla_decode's out, heads in order); w_o [H*D_v, C]; b_o [C] (NULL: no
 *  bias); y [n_tok, C] (output). n_tok == 0 enqueues nothing.
 *  workspace: at least mla_output_project_workspace_bytes(dims, n_tok) bytes.
 */
size_t mla_output_project_workspace_bytes(const mla_dims* dims, int32_t n_tok);
mla_status mla_output_project(const mla_dims* dims, int32_t n_tok, const void* o,
                              const void* w_o, const void* b_o, void* y, void* workspace,
                              size_t ws_bytes, hipStream_t stream);

/*
 * mla_select_path -- choose the decode path of a GQLA layer for a target device from the
 * roofline of each path ([GQLA] section 2, "Sélection du chemin": the absorbed MQA path on
 * hardware whose compute/bandwidth ridge sits above its intensity, the GQA path where the
 * ridge is low; section 1 gives the ridges, section 4 the projected throughputs this model
 * reproduces). Per query step of one sequence with `context` cached positions:
 *     absorbed: bytes = context * (d_c + d_r) * elt
 *               FLOPs = context * s_q * (2 H (d_c + d_r) + 2 H d_c)
 *     GQA:      bytes = context * (G (D + D_v) + d_r) * elt
 *               FLOPs = context * s_q * (2 H (D + d_r) + 2 H D_v)
 *     time = max(bytes / hbm_bytes_per_s, FLOPs / flops_per_s)
 *  The path with the smaller time is returned (the absorbed path on a tie). The query,
 *  output and up-projection work around the attention, and the one-off expansion of the GQA
 *  cache, are not counted.
 *  hbm_bytes_per_s, flops_per_s: the target's rates; both 0 selects the rates this library's
 *  kernels sustain on MI355X (MLA_MI355X_HBM_BYTES_PER_S, MLA_MI355X_BF16_FLOPS), so that the
 *  choice is the faster of the two measured paths. t_absorbed, t_gqa: nullable outputs,
 *  the two times in seconds. Returns MLA_PATH_ABSORBED or MLA_PATH_GQA; otherwise a negative
 *  mla_status: the dims checks of the other calls, MLA_ERR_RANGE for s_q < 1, context < 1 or
 *  rates that are not both positive (or both 0). Host only: launches nothing.
 */
typedef enum { MLA_PATH_ABSORBED = 0, MLA_PATH_GQA = 1 } mla_path;
/* MI355X rates used by default, as measured: the GQA decode streams its expanded cache at
 * 6.8e12 B/s (4.43 GB in 0.65 ms at G = 8, 32 x 32,768 positions); the absorbed split-K
 * decode sustains 0.87e15 bf16 FLOP/s at s_q = 2 on the same workload (584 GFLOP in
 * 0.67 ms; 0.86-0.96e15 over s_q = 1..8). The chip's dense bf16 peak is 2.5e15, but under a
 * sustained matrix-core load it holds about 1.3-1.4e15 (the clock falls below 2 GHz), and
 * the decode's matrix cores are busy about half of its launch. */
#define MLA_MI355X_HBM_BYTES_PER_S 6.8e12
#define MLA_MI355X_BF16_FLOPS 0.87e15
int32_t mla_select_path(const mla_dims* dims, int32_t s_q, int64_t context,
                        double hbm_bytes_per_s, double flops_per_s, double* t_absorbed,
                        double* t_gqa);

/* Static, NUL-terminated description of a status. */
const char* mla_status_string(mla_status status);

/*
 * mla_validate_block_table -- host-side check of a block table (host memory): every position
 * 0 .. host_seq_lens[b]-1 of every sequence maps to a block id in [0, num_blocks), no block is
 * used by two (sequence, block index) pairs, and host_seq_lens[b] <= max_blocks*bs.
 * Returns MLA_OK, MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_RANGE or MLA_ERR_BLOCK_TABLE.
 */
mla_status mla_validate_block_table(const mla_dims* dims, const int32_t* host_table,
                                    int32_t batch, int32_t max_blocks,
                                    const int32_t* host_seq_lens, int32_t num_blocks);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
