/*
 * mla.h -- C ABI of the MI355X (gfx950) Multi-head Latent Attention decode
 * library (libmla.so), with a prefill entry point.
 *
 * What it computes.  DeepSeek-V3's MLA, as the DeepSeek-V3 reading lesson
 * "Читаем техотчёт DeepSeek-V3 вместе" (ai.flicky.cc), section 2.1.1 "MLA: что
 * попадает в кэш", and the paper summary "Báo cáo Kỹ thuật DeepSeek-V3"
 * (xyznot.com), "Phương pháp" item 1, state it:
 *
 *     c_t^KV = W^DKV h_t,  k_t^R = RoPE(W^KR h_t),  k^C = W^UK c^KV,
 *     v^C = W^UV c^KV,  key of head i = [k^C_{t,i}; k^R_t],
 *     c^Q = W^DQ h,  W^UQ c^Q = per head [q^C_i ; q^R_i],  q^R rotated.
 *
 * Only c^KV and k^R are cached (§2.1.1 and the summary's closing sentence of
 * item 1).  At decode W^UK is folded into the query (§2.1.1 Question 2) and
 * W^UV is applied after the attention-weighted sum of latents (linearity of
 * v^C = W^UV c^KV).  The attention itself is a scaled softmax over the
 * visible cached tokens.
 *
 * Conventions (the pages leave these open):
 *   - Weights are row-major [out, in], so y = W x as the formulas write it:
 *     W_DKV [d_c, d_model], W_KR [d_rope, d_model], W_DQ [d_cq, d_model],
 *     W_UQ [n_heads*(d_head+d_rope), d_cq] with rows head-major and, within a
 *     head, d_head content rows then d_rope RoPE rows; W_UK and W_UV
 *     [n_heads*d_head, d_c] (rows of head i are i*d_head .. i*d_head+d_head-1).
 *   - RoPE rotates channel pairs (2m, 2m+1) by pos * theta^(-2m/d_rope).
 *   - Positions are 0-based; token t of a sequence sits at position t.  At
 *     decode, seqlens[b] already counts the s_q new tokens, query j sits at
 *     p_j = seqlens[b] - s_q + j and sees tokens 0..p_j (causal).
 *   - Every pointer argument except `dims`, `cache` (the descriptor itself)
 *     and the returned strings is DEVICE memory, contiguous, row-major, owned
 *     by the caller.  The library never allocates or frees.  Its only global
 *     state is a mutex-guarded record of which kernels have had their LDS
 *     limit raised on which device, so calls from several threads and on
 *     different streams do not interfere.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is only
 *     enqueued; nothing synchronises.  Arguments are validated on the host
 *     before anything is enqueued: on error a negative mla_status is returned
 *     and nothing is launched.  Device-side metadata (block tables, seqlens,
 *     positions) is trusted: out-of-range page ids or positions are undefined
 *     behaviour.
 *
 * Cache layout.  Token t of sequence b lives in page block_table[b*max_pages
 * + t/page_size], slot t%page_size.  Its row is c^KV (d_c channels) then k^R
 * (d_rope channels, already rotated at the token's position).
 *   F32 pages:  row-major float [page_size][d_c + d_rope].
 *   BF16 pages: the rows cut into 16-byte chunks of 8 channels and stored
 *     chunk-major: channel ch of slot t is the bf16 at byte
 *         16 * ((ch/8) * page_size + (t ^ x(ch/8))) + 2 * (ch%8),
 *     x(C) = 4 * ((4 - C%4) % 4)  (0, 12, 8, 4).  (d_c + d_rope) % 8 == 0.
 *   FP8_E4M3 pages, in this order:
 *     codes  u8, 16-channel chunks, chunk-major: latent channel ch of slot t
 *            at byte 16 * ((ch/16) * page_size + (t ^ x(ch/16))) + ch%16;
 *     scales f32 [page_size][d_c/128] at byte page_size * d_c;
 *     rope   bf16 k^R at byte page_size * (d_c + 4 * d_c/128), laid out
 *            like a BF16 page of d_rope channels.
 *   FP8 follows the lesson's §3.3 "Обучение в FP8": E4M3 for all tensors,
 *   one scale per 1x128 activation tile.  Scale s = amax/448 (1 for an
 *   all-zero tile), code = round-to-nearest-even(x/s) saturated to +-448,
 *   value = code*s.  Requires d_c % 128 == 0 and d_rope % 8 == 0.
 *   FP8_E4M3_E8 pages: the FP8_E4M3 layout and codes, with power-of-two
 *   (UE8M0) scales, the format the lesson's continuation of §3.5 says
 *   DeepSeek V3.1 adopted: s = the smallest power of two >= amax/448 (the
 *   float32 quotient), at least 2^-126, still stored as f32.  No code
 *   saturates, and every value code*s is exact in bf16.
 * The chunk-major pages are what the gfx950 kernels copy to LDS verbatim;
 * mla_page_bytes() gives a page's size.
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define MLA_API __attribute__((visibility("default")))
#else
#define MLA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = -1,        /* a required pointer is NULL                        */
  MLA_ERR_DIMS = -2,        /* a size is out of range or inconsistent             */
  MLA_ERR_DTYPE = -3,       /* unknown dtype or unsupported dtype combination     */
  MLA_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned                   */
  MLA_ERR_WORKSPACE = -5,   /* workspace missing or smaller than required         */
  MLA_ERR_UNSUPPORTED = -6, /* valid but not implemented for these dims           */
  MLA_ERR_HIP = -7          /* a HIP runtime call failed while enqueueing         */
} mla_status;

typedef enum {
  MLA_F32 = 0,
  MLA_BF16 = 1,
  MLA_FP8_E4M3 = 2,   /* cache only: E4M3 codes, f32 tile scales amax/448 */
  MLA_FP8_E4M3_E8 = 3 /* cache only: E4M3 codes, power-of-two tile scales  */
} mla_dtype;

/* Model dimensions (lesson's V3 shape dictionary: d_model 7168, 128 heads of
 * d_head 128, d_rope 64, d_c 512, d_cq 1536).  page_size is the number of
 * tokens per cache page.  Limits: all > 0; d_head, d_rope, d_c even;
 * d_rope <= 128; d_c <= 1024; d_cq <= 4096; d_model <= 16384; n_heads <= 256;
 * page_size <= 256 and a multiple of 16; for an FP8 cache d_c % 128 == 0.   */
typedef struct {
  int32_t d_model, n_heads, d_head, d_rope, d_c, d_cq, page_size;
  float rope_theta;
} mla_dims;

/* A caller-owned paged latent cache: `pages` (device) holds `num_pages`
 * pages of mla_page_bytes(dims, dtype) bytes each.                          */
typedef struct {
  void* pages;
  int32_t dtype;     /* mla_dtype: MLA_F32, MLA_BF16, MLA_FP8_E4M3 or MLA_FP8_E4M3_E8 */
  int32_t num_pages;
} mla_cache;

/* Bytes of one cache page of `cache_dtype` (0 for invalid arguments).       */
MLA_API size_t mla_page_bytes(const mla_dims* dims, int32_t cache_dtype);

/* Latent-cache append (lesson §2.1.1 KV equations; summary item 1):
 * for each of the n_tok rows of h [n_tok, d_model] (dtype act_dtype, F32 or
 * BF16), computes c^KV = W_DKV h and k^R = RoPE(W_KR h, pos[r]) with fp32
 * accumulation and stores the row into sequence seq_id[r] at position pos[r]
 * of the paged cache (converted, or quantised per 1x128 tile for FP8).
 * seq_id, pos: int32 [n_tok] device.  block_table: int32 [*, max_pages]
 * device.  W_DKV/W_KR have dtype act_dtype.  n_tok == 0 is a no-op.
 * BF16 caches require BF16 activations or F32 activations; F32 caches
 * require F32 activations.                                                  */
MLA_API int mla_cache_append(const mla_dims* dims, int32_t act_dtype, const void* h,
                     int32_t n_tok, const int32_t* seq_id, const int32_t* pos,
                     const void* W_DKV, const void* W_KR, const mla_cache* cache,
                     const int32_t* block_table, int32_t max_pages,
                     void* stream);

/* The append of a decode step with a workspace: the same tokens, the same
 * rows and the same error behaviour as mla_cache_append (same citation), the
 * latent rows' matrix product split over d_model into fp32 partial sums in
 * ws, so that a few tokens spread over the whole GPU; the rows then equal
 * mla_cache_append's up to the fp32 summation order.
 *   ws  device workspace of at least mla_append_workspace_bytes(dims,
 *       act_dtype, n_tok) bytes, 16-byte aligned, caller-owned; its contents
 *       are overwritten.  May be NULL when that size is 0: then this is
 *       mla_cache_append.
 * mla_append_workspace_bytes is non-zero for BF16 activations at the
 * DeepSeek-V3 latent shape (d_c 512, d_rope 64, d_model a multiple of 896)
 * and 1..64 tokens with a BF16 or FP8 cache; 0 otherwise (and for invalid
 * dims).  Extra errors: MLA_ERR_NULL / MLA_ERR_ALIGN for ws, and
 * MLA_ERR_WORKSPACE when ws_bytes is below the required size; nothing is
 * enqueued on an error other than MLA_ERR_HIP.                              */
MLA_API size_t mla_append_workspace_bytes(const mla_dims* dims, int32_t act_dtype, int32_t n_tok);
MLA_API int mla_cache_append_ws(const mla_dims* dims, int32_t act_dtype, const void* h,
                        int32_t n_tok, const int32_t* seq_id, const int32_t* pos,
                        const void* W_DKV, const void* W_KR, const mla_cache* cache,
                        const int32_t* block_table, int32_t max_pages, void* ws,
                        size_t ws_bytes, void* stream);

/* Direct cache write: stores given latent rows c_kv [n_tok, d_c] and already
 * rotated k_rope [n_tok, d_rope] (dtype act_dtype, F32 or BF16) at
 * (seq_id[r], pos[r]), converting or quantising exactly as mla_cache_append
 * does with its fp32 results.  For tests that plant cache contents and for
 * callers that produce latents elsewhere.                                   */
MLA_API int mla_cache_write(const mla_dims* dims, int32_t act_dtype, const void* c_kv,
                    const void* k_rope, int32_t n_tok, const int32_t* seq_id,
                    const int32_t* pos, const mla_cache* cache,
                    const int32_t* block_table, int32_t max_pages, void* stream);

/* Number of KV splits mla_decode uses when num_splits == 0: enough
 * (sequence, split) work items to fill the GPU, never more than max_pages.  */
MLA_API int32_t mla_default_splits(const mla_dims* dims, int32_t batch, int32_t s_q,
                           int32_t max_pages);

/* Split count from the sequences' lengths, for callers that know them on the
 * host (a serving loop keeps them): seqlens is a HOST array [batch], the
 * values of the device seqlens that mla_decode will read.  When the longest
 * length is within 1/16 of the mean, the smallest count that gives one
 * (sequence, query block, split) work item per compute unit, without the
 * page cap of mla_default_splits (whose shorter items only pay off when
 * lengths are ragged); otherwise mla_default_splits.  Pass the result as
 * num_splits.  0 for invalid arguments (NULL, a length below 0 or above
 * max_pages * page_size).                                                   */
MLA_API int32_t mla_plan_splits(const mla_dims* dims, int32_t batch, int32_t s_q,
                                int32_t max_pages, const int32_t* seqlens);

/* Output projection of the attention layer: for each of `rows` rows,
 *     y_r = W^O [o_{r,1}; o_{r,2}; ...; o_{r,H}]
 * (the W_O of the attention_params docstring of "Читаем техотчёт
 * DeepSeek-V3 вместе", practice part, heads*d_head x d; its result is the
 * u_t that the MoE layer of §2.1.2 takes as input; no residual or norm).
 *   o   [rows, n_heads*d_head] (act_dtype), heads concatenated in head order
 *       with d_head innermost: exactly the out tensor of mla_combine
 *       [batch, s_q, H, d_head] with rows = batch*s_q.
 *   W_O [d_model, n_heads*d_head] (act_dtype, stored [out, in]).
 *   y   [rows, d_model] (act_dtype), written.
 *   ws  device workspace of mla_output_project_workspace_bytes() bytes
 *       (fp32 partial sums; may be NULL when that is 0), 16-byte aligned.
 * act_dtype MLA_F32 or MLA_BF16; rows in 0..131072 (0 does nothing).  All
 * device pointers 16-byte aligned and caller-owned.  Errors: MLA_ERR_NULL,
 * MLA_ERR_DTYPE, MLA_ERR_DIMS, MLA_ERR_ALIGN, MLA_ERR_WORKSPACE, MLA_ERR_HIP;
 * nothing is enqueued on an error other than MLA_ERR_HIP.                   */
MLA_API size_t mla_output_project_workspace_bytes(const mla_dims* dims, int32_t act_dtype,
                                                  int32_t rows);
MLA_API int mla_output_project(const mla_dims* dims, int32_t act_dtype, int32_t rows,
                               const void* o, const void* W_O, void* y, void* ws,
                               size_t ws_bytes, void* stream);

/* FP8 projection GEMMs with fine-grained scaling ("Читаем техотчёт
 * DeepSeek-V3 вместе", §3.3 "Обучение в FP8", items 2-4; the same scheme in
 * the "Báo cáo Kỹ thuật DeepSeek-V3" summary): E4M3 everywhere, weights in
 * 128 x 128 blocks and activations in 1 x 128 tiles, each group with its
 * own fp32 scale s = amax / 448 (1 for an all-zero group), code =
 * round-to-nearest-even(x / s) saturated at +-448, and every 128-wide
 * partial sum scaled and accumulated in fp32.
 *
 * mla_fp8_quantize_weight: W [N, K] bf16 (stored [out, in], 16-byte
 *   aligned) -> codes [N, K] uint8 (E4M3FN, 16-byte aligned) and scales
 *   [ceil(N/128), K/128] fp32 (4-byte aligned); the last row-block is
 *   shorter when N % 128 != 0.  N % 16 == 0 and K % 128 == 0 (else
 *   MLA_ERR_UNSUPPORTED), N and K at most 65536.
 * mla_fp8_gemm: Y [M, N] (bf16) = Q(X) . Q(W)^T for X [M, K] bf16, the
 *   weight as quantised above; X is quantised in 1 x 128 tiles (64 rows at
 *   a time) into the workspace.  N % 16 == 0 and K % 512 == 0 (else
 *   MLA_ERR_UNSUPPORTED); M in 0..131072 (0 does nothing); ws (16-byte
 *   aligned) holds mla_fp8_gemm_workspace_bytes() bytes: the activation
 *   codes and scales of one 64-row chunk and the fp32 partial sums.  Made
 *   for decode-sized M: every 64 rows stream the weight once.
 * Errors as for the other calls; nothing is enqueued on an error other than
 * MLA_ERR_HIP.  Device pointers, caller-owned, no allocation.               */
MLA_API int mla_fp8_quantize_weight(const void* W, int32_t N, int32_t K, void* codes,
                                    float* scales, void* stream);
/* mla_fp8_quantize_weight of the transposes of `batch` matrices: W [batch,
 * R, C] bf16 -> codes [batch, C, R] (row b*C + c holds column c of W[b])
 * and scales [batch, C/128, R/128]; each 128 x 128 block of W[b]^T is the
 * transpose of a block of W[b] and gets that block's scale.  R and C
 * multiples of 128 (else MLA_ERR_UNSUPPORTED), at most 65536, batch 1..65536.
 * For W^UK [n_heads, d_head, d_c], which mla_decode_fp8w takes transposed
 * per head.                                                                 */
MLA_API int mla_fp8_quantize_weight_t(const void* W, int32_t batch, int32_t R, int32_t C,
                                      void* codes, float* scales, void* stream);
MLA_API size_t mla_fp8_gemm_workspace_bytes(int32_t M, int32_t N, int32_t K);
MLA_API int mla_fp8_gemm(int32_t M, int32_t N, int32_t K, const void* X, const void* W_codes,
                         const float* W_scales, void* Y, void* ws, size_t ws_bytes, void* stream);

/* Speculative verify with multi-token prediction ("Читаем техотчёт
 * DeepSeek-V3 вместе", §2.2 Multi-Token Prediction; the tokens_per_step
 * exercise of its practice part): one decode step with s_q = 1 + depth query
 * rows verifies a chain of `depth` drafted tokens, each drafted token being
 * kept with probability `acceptance` given that its predecessors were kept.
 * Returns the mean number of tokens the step yields,
 * 1 + acceptance + acceptance^2 + ... + acceptance^depth; NaN for an
 * acceptance outside [0, 1] or a depth outside 0..7 (s_q is at most 8).
 * Pure host arithmetic: no device, no stream.                                */
MLA_API double mla_mtp_tokens_per_step(double acceptance, int32_t depth);

/* Workspace bytes needed by mla_decode/mla_combine for these sizes
 * (num_splits >= 1; 0 for invalid arguments).                               */
MLA_API size_t mla_workspace_bytes(const mla_dims* dims, int32_t act_dtype,
                           int32_t batch, int32_t s_q, int32_t num_splits);

/* Decode, first half: query projection, absorption and split-KV attention.
 *   hq [batch*s_q, d_model] (act_dtype): hidden states of the s_q newest
 *     tokens of each sequence, row b*s_q + j; or, when W_DQ is NULL, their
 *     compressed queries c^Q [batch*s_q, d_cq] (summary item 1: c^Q).
 *   W_DQ [d_cq, d_model] or NULL; W_UQ [n_heads*(d_head+d_rope), d_cq];
 *   W_UK [n_heads*d_head, d_c]  (act_dtype).
 *   cache, block_table [batch, max_pages], seqlens int32 [batch] (device;
 *     seqlens[b] >= s_q, or 0 for an empty sequence whose output is 0).
 *   softmax_scale: tau in softmax(tau * q.k).
 *   num_splits: KV splits per sequence (1..max_pages, 0 = default).
 * For each query row, head i and split s it computes, over the split's
 * visible tokens, the softmax-normalised sum of latents c_t (the absorbed
 * form: scores tau*(q^C_i^T W^UK_i c_t + q^R_i . k^R_t)) and its
 * log-sum-exp, and leaves them, with the split plan, in the workspace
 * ws [ws_bytes >= mla_workspace_bytes(...)] for mla_combine.
 * Supported: act F32 with an F32 or FP8 cache; act BF16 with a BF16 or FP8
 * cache.  s_q in 1..8.                                                      */
MLA_API int mla_decode(const mla_dims* dims, int32_t act_dtype, const void* hq,
               int32_t batch, int32_t s_q, const void* W_DQ, const void* W_UQ,
               const void* W_UK, const mla_cache* cache,
               const int32_t* block_table, int32_t max_pages,
               const int32_t* seqlens, float softmax_scale, int32_t num_splits,
               void* ws, size_t ws_bytes, void* stream);

/* The two halves of mla_decode, for callers that want to schedule or time
 * them separately (same arguments and validation as mla_decode):
 * mla_decode_query runs the query projection and absorption into ws;
 * mla_decode_attend then runs the split-KV attention over the cache using
 * the queries in ws and records the split plan there for mla_combine.  The
 * attention reads neither hq nor the weights, so mla_decode_attend accepts
 * NULL for hq, W_DQ, W_UQ and W_UK (it also serves the queries that
 * mla_decode_fp8w_query leaves in ws).  mla_decode == query then attend.    */
MLA_API int mla_decode_query(const mla_dims* dims, int32_t act_dtype, const void* hq,
               int32_t batch, int32_t s_q, const void* W_DQ, const void* W_UQ,
               const void* W_UK, const mla_cache* cache,
               const int32_t* block_table, int32_t max_pages,
               const int32_t* seqlens, float softmax_scale, int32_t num_splits,
               void* ws, size_t ws_bytes, void* stream);
MLA_API int mla_decode_attend(const mla_dims* dims, int32_t act_dtype, const void* hq,
               int32_t batch, int32_t s_q, const void* W_DQ, const void* W_UQ,
               const void* W_UK, const mla_cache* cache,
               const int32_t* block_table, int32_t max_pages,
               const int32_t* seqlens, float softmax_scale, int32_t num_splits,
               void* ws, size_t ws_bytes, void* stream);

/* Split count that mla_decode uses for these arguments (num_splits 0 = the
 * default of mla_default_splits; a request is rounded so that every split
 * spans the same number of pages).  This is the count mla_combine takes.
 * 0 for invalid arguments.                                                  */
MLA_API int32_t mla_decode_splits(const mla_dims* dims, int32_t batch, int32_t s_q,
                                  int32_t max_pages, int32_t num_splits);

/* Decode, second half: merges the splits that the preceding mla_decode on
 * this workspace left (log-sum-exp weighted; empty splits skipped), then
 * applies W^UV per head (the value path is linear in c^KV, so
 * sum_t p_t W^UV_i c_t = W^UV_i sum_t p_t c_t; lesson §2.1.1):
 *   out [batch, s_q, n_heads, d_head] (act_dtype) = W^UV_i * O_lat_i;
 *   lse_out [batch, s_q, n_heads] fp32 natural-log log-sum-exp of the scaled
 *   scores, or NULL.  An empty sequence gives out = 0 and lse = -inf.
 * num_splits: the split count of that mla_decode, i.e.
 *   mla_decode_splits(dims, batch, s_q, max_pages, its num_splits argument);
 *   1..4096.  The merge reads exactly num_splits partials per row.
 * ws, ws_bytes: the decode's workspace; ws_bytes must be at least
 *   mla_workspace_bytes(dims, act_dtype, batch, s_q, num_splits), else
 *   MLA_ERR_WORKSPACE and nothing is enqueued.  The combine writes its own
 *   scratch region of ws (the merged latent rows when it merges before
 *   W^UV), never the queries or partials, so the halves of mla_decode may be
 *   re-run on the same ws afterwards.
 * batch, s_q, act_dtype and ws must be those of the preceding mla_decode on
 * the same stream; a different num_splits gives wrong results but reads only
 * inside the validated workspace.                                           */
MLA_API int mla_combine(const mla_dims* dims, int32_t act_dtype, int32_t batch,
                int32_t s_q, int32_t num_splits, void* ws, size_t ws_bytes,
                const void* W_UV, void* out, float* lse_out, void* stream);

/* Decode step with FP8 block-scaled projection weights: the query phase
 * and the combine of mla_decode / mla_combine with W^DQ, W^UQ, W^UK and
 * W^UV in E4M3 ("Читаем техотчёт DeepSeek-V3 вместе", §3.3 "Обучение в
 * FP8", items 2-4: weights in 128 x 128 blocks, activations in 1 x 128
 * tiles, scale s = amax / 448 per group, every 128-wide partial product
 * promoted into an fp32 sum with its two scales).  Each projection is
 * Y = Q(X) . Q(W)^T with W quantised once by mla_fp8_quantize_weight and X
 * quantised in the step:
 *   c^Q = W^DQ hq;  u = W^UQ c^Q;  qt_i = tau*log2(e) [W^UK_i^T q^C_i ;
 *   RoPE(q^R_i)];  out_i = W^UV_i O_lat_i
 * (bf16 rounding of c^Q, u and O_lat between the GEMMs, as the bf16 step
 * does).  The attention between them is that of the bf16 step, on a BF16 or
 * FP8 cache.
 *   hq [batch*s_q, d_model] BF16 hidden states (W^DQ is required).
 *   W_DQ: codes [d_cq, d_model], scales [d_cq/128, d_model/128].
 *   W_UQ: codes [n_heads*(d_head+d_rope), d_cq], scales [rows/128, d_cq/128]
 *     (the rows of mla_decode's W_UQ).
 *   W_UKT: W^UK transposed per head, codes [n_heads*d_c, d_head] (row
 *     i*d_c + n, column k holds W^UK[i][k][n]), scales [n_heads*d_c/128,
 *     d_head/128]: mla_fp8_quantize_weight_t(W_UK, n_heads, d_head, d_c).
 *   W_UV: codes [n_heads*d_head, d_c], scales [n_heads*d_head/128, d_c/128].
 * Codes 16-byte aligned, scales 4-byte aligned, all device, caller-owned.
 * The other arguments are mla_decode's (act_dtype is BF16).  ws holds
 * mla_decode_fp8w_workspace_bytes(...) bytes: the bf16 step's workspace
 * (so mla_decode_attend and the split plan work on it unchanged) followed
 * by the FP8 GEMMs' activation codes, scales and partial sums.
 * mla_decode_fp8w = mla_decode_fp8w_query, then the attention;
 * mla_combine_fp8w merges the splits as mla_combine does and applies W_UV.
 * Supported: the DeepSeek-V3 head shape of the MFMA path (d_head 128, d_c
 * 512, d_rope 64, 128 heads, 64-token pages), d_cq and d_model multiples of
 * 512, s_q 1..8; anything else returns MLA_ERR_UNSUPPORTED (and the
 * workspace size 0).  Errors as for mla_decode; nothing is enqueued on an
 * error other than MLA_ERR_HIP.                                             */
MLA_API size_t mla_decode_fp8w_workspace_bytes(const mla_dims* dims, int32_t batch, int32_t s_q,
                                               int32_t num_splits);
MLA_API int mla_decode_fp8w(const mla_dims* dims, const void* hq, int32_t batch, int32_t s_q,
               const void* W_DQ_codes, const float* W_DQ_scales, const void* W_UQ_codes,
               const float* W_UQ_scales, const void* W_UKT_codes, const float* W_UKT_scales,
               const mla_cache* cache, const int32_t* block_table, int32_t max_pages,
               const int32_t* seqlens, float softmax_scale, int32_t num_splits,
               void* ws, size_t ws_bytes, void* stream);
MLA_API int mla_decode_fp8w_query(const mla_dims* dims, const void* hq, int32_t batch, int32_t s_q,
               const void* W_DQ_codes, const float* W_DQ_scales, const void* W_UQ_codes,
               const float* W_UQ_scales, const void* W_UKT_codes, const float* W_UKT_scales,
               const mla_cache* cache, const int32_t* block_table, int32_t max_pages,
               const int32_t* seqlens, float softmax_scale, int32_t num_splits,
               void* ws, size_t ws_bytes, void* stream);
MLA_API int mla_combine_fp8w(const mla_dims* dims, int32_t batch, int32_t s_q, int32_t num_splits,
               void* ws, size_t ws_bytes, const void* W_UV_codes, const float* W_UV_scales,
               void* out, float* lse_out, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the decode
 * step, mla_decode followed by mla_combine, with its workspace in a static
 * array of MLA_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it
 * runs on until the process ends, instead of a caller's ws.  Arguments are
 * those of mla_decode without ws/ws_bytes, plus W_UV, out and lse_out of
 * mla_combine, with the same meaning, layout and validation; out and lse_out
 * receive what mla_decode + mla_combine give on the same inputs.
 * The MFMA path only (the DeepSeek-V3 head shape, BF16 activations, BF16 or
 * FP8 cache, s_q 1..8): anything else returns MLA_ERR_UNSUPPORTED.  A split
 * plan whose workspace exceeds the array returns MLA_ERR_WORKSPACE (the
 * 64 x 4096-token batch with 4 splits takes about 58 MB).  Nothing is
 * allocated and nothing is enqueued on an error.  Every call on one GPU uses
 * that GPU's one array, and nothing in it needs to start at zero (a call
 * writes every byte it reads): calls that overlap on one GPU, on different
 * streams or threads, race.                                                */
#define MLA_NOALLOC_SCRATCH_BYTES (64 << 20)
MLA_API int mla_decode_step_noalloc(const mla_dims* dims, int32_t act_dtype, const void* hq,
               int32_t batch, int32_t s_q, const void* W_DQ, const void* W_UQ,
               const void* W_UK, const void* W_UV, const mla_cache* cache,
               const int32_t* block_table, int32_t max_pages,
               const int32_t* seqlens, float softmax_scale, int32_t num_splits,
               void* out, float* lse_out, void* stream);

/* Prefill (the non-absorbed form of the lesson's §2.1.1 for many new tokens
 * at once): n_seq fresh sequences packed back to back in
 *   h [n_tok, d_model] (BF16): sequence b is rows cu_seqlens[b] ..
 *     cu_seqlens[b+1]-1, and its token t sits at position t;
 *   cu_seqlens int32 [n_seq + 1] device, cu_seqlens[0] = 0, non-decreasing,
 *     cu_seqlens[n_seq] = n_tok, no sequence longer than max_seqlen (host);
 *   W_DQ [d_cq, d_model], W_UQ [n_heads*(d_head+d_rope), d_cq],
 *   W_UK, W_UV [n_heads*d_head, d_c], W_DKV [d_c, d_model],
 *   W_KR [d_rope, d_model] (BF16, the layouts of mla_decode/mla_cache_append).
 * For every token j and head i it computes, with explicit per-head keys
 * k_{t,i} = [W^UK_i c^KV_t ; k^R_t] and values v_{t,i} = W^UV_i c^KV_t,
 *   out[j][i] = sum over t <= j of softmax_t(softmax_scale * q_{j,i}.k_{t,i}) v_{t,i}
 * into out [n_tok, n_heads, d_head] (BF16) and the natural-log log-sum-exp
 * into lse_out [n_tok, n_heads] fp32 (or NULL), with fp32 accumulation.  The
 * cache is not written: mla_cache_append stores the same tokens' latents.
 * ws [ws_bytes >= mla_prefill_workspace_bytes(...)] holds the projections.
 * Supported: BF16 activations at the DeepSeek-V3 head shape (128 heads of
 * d_head 128, d_rope 64, d_c 512); anything else returns
 * MLA_ERR_UNSUPPORTED.  n_tok == 0 is a no-op.                              */
MLA_API size_t mla_prefill_workspace_bytes(const mla_dims* dims, int32_t act_dtype, int32_t n_tok);
MLA_API int mla_prefill(const mla_dims* dims, int32_t act_dtype, const void* h, int32_t n_tok,
                int32_t n_seq, const int32_t* cu_seqlens, int32_t max_seqlen,
                const void* W_DQ, const void* W_UQ, const void* W_UK, const void* W_UV,
                const void* W_DKV, const void* W_KR, float softmax_scale, void* out,
                float* lse_out, void* ws, size_t ws_bytes, void* stream);

/* The two halves of mla_prefill (same arguments and validation), for callers
 * that schedule or time them separately: mla_prefill_project computes the
 * token positions, c^KV, k^R, c^Q, q, k^C and v^C into ws; mla_prefill_attend
 * then runs the causal attention from ws into out and lse_out.
 * mla_prefill == project then attend on the same stream.                    */
MLA_API int mla_prefill_project(const mla_dims* dims, int32_t act_dtype, const void* h, int32_t n_tok,
                int32_t n_seq, const int32_t* cu_seqlens, int32_t max_seqlen,
                const void* W_DQ, const void* W_UQ, const void* W_UK, const void* W_UV,
                const void* W_DKV, const void* W_KR, float softmax_scale, void* out,
                float* lse_out, void* ws, size_t ws_bytes, void* stream);
MLA_API int mla_prefill_attend(const mla_dims* dims, int32_t act_dtype, const void* h, int32_t n_tok,
                int32_t n_seq, const int32_t* cu_seqlens, int32_t max_seqlen,
                const void* W_DQ, const void* W_UQ, const void* W_UK, const void* W_UV,
                const void* W_DKV, const void* W_KR, float softmax_scale, void* out,
                float* lse_out, void* ws, size_t ws_bytes, void* stream);

/* Metadata check before a decode step (what the host validation of the
 * other calls cannot see, since it lives in device memory): counts
 *   bad[0]: sequences whose seqlens[b] is negative or exceeds
 *           max_pages * page_size;
 *   bad[1]: block-table entries block_table[b][p] of pages the sequence uses
 *           (p * page_size < seqlens[b]) outside 0 .. cache->num_pages - 1,
 * and writes both to bad (device int32[2], 4-byte aligned) on `stream`; the
 * caller reads them after the stream.  An entry counted in bad[1] would make
 * mla_decode read outside the page pool, which the decode itself does not
 * check.  Arguments as for mla_decode; batch 0 writes zeros (seqlens may
 * then be NULL).  Errors:
 * MLA_ERR_NULL, MLA_ERR_DIMS, MLA_ERR_DTYPE, MLA_ERR_ALIGN; nothing is
 * enqueued on an error other than MLA_ERR_HIP.                              */
MLA_API int mla_check_metadata(const mla_dims* dims, const mla_cache* cache, const int32_t* block_table,
                               int32_t max_pages, const int32_t* seqlens, int32_t batch, int32_t* bad,
                               void* stream);

/* Measurement helper (no part of the decode maths): streams `bytes` (a
 * multiple of 16) of device memory at src with 16-byte loads over the whole
 * GPU and writes nothing (sink: one device int32 that is practically never
 * written).  Timing it gives the achievable HBM read bandwidth that the
 * decode kernels' byte roofline is read against next to the data-sheet
 * figure.  Errors: MLA_ERR_NULL, MLA_ERR_DIMS (bytes % 16), MLA_ERR_ALIGN.  */
MLA_API int mla_hbm_read_probe(const void* src, size_t bytes, int32_t* sink, void* stream);

/* Measurement helper (no part of the decode maths): 4096 waves, each
 * running iters x 32 v_mfma_f32_32x32x16_bf16 in eight independent chains on
 * operands held in registers, loaded once from ops (12 x 64 bf16x8 = 12 KiB
 * of device memory, 16-byte aligned; finite values such as N(0,1) samples).
 * No other memory traffic; sink (one device float) is practically never
 * written.  *flops (host, may be NULL) receives the launch's floating-point
 * operations (2 per multiply-add).  Run back to back, it gives the bf16 MFMA
 * rate that the board's power limit allows, the ceiling that the MFMA-bound
 * kernels are read against next to the data-sheet peak.  iters == 0 only
 * sets *flops.  Errors: MLA_ERR_DIMS (iters < 0), MLA_ERR_NULL,
 * MLA_ERR_ALIGN.                                                             */
MLA_API int mla_mfma_probe(const void* ops, int32_t iters, float* sink, double* flops, void* stream);

/* Static description of a status code.                                      */
MLA_API const char* mla_status_str(int status);

/* Description of the HIP error behind the last MLA_ERR_HIP returned on the
 * calling thread ("none" if there was none); static string.                 */
MLA_API const char* mla_last_hip_error(void);

/* Library build identifier (kernel set and target), static string.         */
MLA_API const char* mla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
