// C-ABI entry points of libmla.so: argument validation, split planning,
// workspace layout and dispatch to the kernel launchers.  Nothing here
// allocates device memory or synchronises.
#include <algorithm>
#include <math.h>
#include <mutex>
#include <set>
#include <stdlib.h>
#include <string.h>
#include <utility>
#include "internal.hpp"

using namespace mla;

namespace mla {

// The MFMA path's shape: DeepSeek-V3's MLA (d_c 512, d_rope 64, 128 heads of
// 128, 64-token pages), bf16 activations.
static bool v3_shape(const mla_dims& d) {
  return d.d_c == 512 && d.d_rope == 64 && d.n_heads == 128 && d.d_head == 128 && d.page_size == 64 &&
         d.d_model % 32 == 0 && d.d_cq % 64 == 0;
}

bool fast_append_supported(const mla_dims& d, int act, int cache_dtype) {
  return fast_append_shape(d) && act == MLA_BF16 && (cache_dtype == MLA_BF16 || is_fp8_cache(cache_dtype));
}

bool fast_decode_supported(const mla_dims& d, int act, int cache_dtype, int s_q) {
  return v3_shape(d) && act == MLA_BF16 && (cache_dtype == MLA_BF16 || is_fp8_cache(cache_dtype)) && s_q >= 1 &&
         s_q <= 8;
}

hipError_t lds_limit(const void* kernel, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::set<std::pair<const void*, int>> done;
  std::lock_guard<std::mutex> lock(mu);
  if (done.count({kernel, dev})) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.insert({kernel, dev});
  return e;
}

}  // namespace mla

namespace {

constexpr int MAX_S_Q = 8;
constexpr int TARGET_ITEMS = 256;  // (sequence, query, split) work items aimed for per decode: one per CU
constexpr int MAX_PAGES_PER_SPLIT = 32;  // caps one item's work (2048 tokens) so that ragged batches balance
constexpr int MAX_OUT_ROWS = 1 << 17;  // rows of one output projection (and of one FP8 GEMM)
constexpr int MAX_FP8_DIM = 1 << 16;   // N and K of one FP8 GEMM
constexpr int MAX_PREFILL_TOKENS = 1 << 17;  // keeps every per-head byte offset of the prefill workspace in 32 bits

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

thread_local hipError_t t_last_hip = hipSuccess;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return MLA_OK;
  t_last_hip = e;
  return MLA_ERR_HIP;
}

int check_dims(const mla_dims* d) {
  if (!d) return MLA_ERR_NULL;
  if (d->d_model <= 0 || d->n_heads <= 0 || d->d_head <= 0 || d->d_rope <= 0 || d->d_c <= 0 || d->d_cq <= 0 ||
      d->page_size <= 0)
    return MLA_ERR_DIMS;
  if ((d->d_head | d->d_rope | d->d_c) & 1) return MLA_ERR_DIMS;
  if (d->d_rope > 128 || d->d_c > 1024 || d->d_cq > 4096 || d->d_model > 16384 || d->n_heads > 256 ||
      d->d_head > 512)
    return MLA_ERR_DIMS;
  if (d->page_size > 256 || d->page_size % 16) return MLA_ERR_DIMS;
  if (!(d->rope_theta > 0.0f)) return MLA_ERR_DIMS;
  return MLA_OK;
}

bool valid_act(int t) { return t == MLA_F32 || t == MLA_BF16; }
bool valid_cache(int t) { return t == MLA_F32 || t == MLA_BF16 || is_fp8_cache(t); }

int check_cache(const mla_dims* d, const mla_cache* c, const int32_t* bt, int32_t max_pages) {
  if (!c || !c->pages || !bt) return MLA_ERR_NULL;
  if (!valid_cache(c->dtype)) return MLA_ERR_DTYPE;
  if (is_fp8_cache(c->dtype) && (d->d_c % 128 || d->d_rope % 8)) return MLA_ERR_UNSUPPORTED;
  if (c->dtype == MLA_BF16 && (d->d_c + d->d_rope) % 8) return MLA_ERR_UNSUPPORTED;
  if (c->num_pages <= 0 || max_pages <= 0) return MLA_ERR_DIMS;
  if (!aligned16(c->pages) || !aligned16(bt)) return MLA_ERR_ALIGN;
  return MLA_OK;
}

bool force_generic() {
  const char* e = getenv("MLA_FORCE_GENERIC");
  return e && e[0] == '1';
}

int resolve_splits(const mla_dims* d, int32_t batch, int32_t s_q, int32_t max_pages, int32_t num_splits,
                   int* S, int* pps) {
  int s = num_splits > 0 ? num_splits : mla_default_splits(d, batch, s_q, max_pages);
  if (s > max_pages) s = max_pages;
  if (s < 1) s = 1;
  int p = (max_pages + s - 1) / s;
  *pps = p;
  *S = (max_pages + p - 1) / p;
  return MLA_OK;
}

// fp32 partial bytes of the workspace append, or 0 where it does not apply
size_t append_ws_bytes(const mla_dims& d, int act, int n_tok) {
  if (force_generic() || act != MLA_BF16 || !fast_append_shape(d) || !skinny_append_supported(d, n_tok)) return 0;
  return (size_t)skinny_append_kgroups(d) * n_tok * (d.d_c + d.d_rope) * 4;
}

int append_common(const mla_dims* dims, int32_t act, const void* a0, const void* a1, int32_t n_tok,
                  const int32_t* seq_id, const int32_t* pos, const void* W_DKV, const void* W_KR,
                  const mla_cache* cache, const int32_t* bt, int32_t max_pages, void* stream, bool write,
                  void* ws = nullptr, size_t ws_bytes = 0, bool with_ws = false) {
  int st = check_dims(dims);
  if (st) return st;
  if (!valid_act(act)) return MLA_ERR_DTYPE;
  if (n_tok < 0) return MLA_ERR_DIMS;
  if ((st = check_cache(dims, cache, bt, max_pages))) return st;
  if (n_tok == 0) return MLA_OK;
  if (!a0 || !seq_id || !pos) return MLA_ERR_NULL;
  if (write ? !a1 : (!W_DKV || !W_KR)) return MLA_ERR_NULL;
  if (!aligned16(a0) || !aligned16(seq_id) || !aligned16(pos)) return MLA_ERR_ALIGN;
  if (write ? !aligned16(a1) : (!aligned16(W_DKV) || !aligned16(W_KR))) return MLA_ERR_ALIGN;
  const bool fast = !write && !force_generic() && fast_append_supported(*dims, act, cache->dtype);
  const size_t need = with_ws && fast ? append_ws_bytes(*dims, act, n_tok) : 0;
  if (need) {
    if (!ws) return MLA_ERR_NULL;
    if (!aligned16(ws)) return MLA_ERR_ALIGN;
    if (ws_bytes < need) return MLA_ERR_WORKSPACE;
  }
  AppendArgs a;
  a.d = *dims; a.act = act; a.h = a0; a.k_rope = a1; a.n_tok = n_tok; a.seq_id = seq_id; a.pos = pos;
  a.W_DKV = W_DKV; a.W_KR = W_KR; a.pages = (uint8_t*)cache->pages; a.g = make_geom(*dims, cache->dtype);
  a.block_table = bt; a.max_pages = max_pages; a.stream = (hipStream_t)stream;
  hipError_t e;
  if (need) {
    e = skinny_append_partials(a, (float*)ws);
    if (e == hipSuccess) e = append_reduce(a, (const float*)ws, skinny_append_kgroups(*dims));
  } else if (write) e = generic_write(a);
  else if (!force_generic() && fast_append_supported(*dims, act, cache->dtype)) e = fast_append(a);
  else e = generic_append(a);
  return hip_status(e);
}

}  // namespace

extern "C" {

size_t mla_page_bytes(const mla_dims* dims, int32_t cache_dtype) {
  if (check_dims(dims) || !valid_cache(cache_dtype)) return 0;
  if (is_fp8_cache(cache_dtype) && (dims->d_c % 128 || dims->d_rope % 8)) return 0;
  if (cache_dtype == MLA_BF16 && (dims->d_c + dims->d_rope) % 8) return 0;
  return page_bytes_of(dims->d_c, dims->d_rope, dims->page_size, cache_dtype);
}

int mla_cache_append(const mla_dims* dims, int32_t act_dtype, const void* h, int32_t n_tok, const int32_t* seq_id,
                     const int32_t* pos, const void* W_DKV, const void* W_KR, const mla_cache* cache,
                     const int32_t* block_table, int32_t max_pages, void* stream) {
  return append_common(dims, act_dtype, h, nullptr, n_tok, seq_id, pos, W_DKV, W_KR, cache, block_table, max_pages,
                       stream, false);
}

size_t mla_append_workspace_bytes(const mla_dims* dims, int32_t act_dtype, int32_t n_tok) {
  if (check_dims(dims) || !valid_act(act_dtype) || n_tok < 0) return 0;
  return append_ws_bytes(*dims, act_dtype, n_tok);
}

int mla_cache_append_ws(const mla_dims* dims, int32_t act_dtype, const void* h, int32_t n_tok, const int32_t* seq_id,
                        const int32_t* pos, const void* W_DKV, const void* W_KR, const mla_cache* cache,
                        const int32_t* block_table, int32_t max_pages, void* ws, size_t ws_bytes, void* stream) {
  return append_common(dims, act_dtype, h, nullptr, n_tok, seq_id, pos, W_DKV, W_KR, cache, block_table, max_pages,
                       stream, false, ws, ws_bytes, true);
}

int mla_cache_write(const mla_dims* dims, int32_t act_dtype, const void* c_kv, const void* k_rope, int32_t n_tok,
                    const int32_t* seq_id, const int32_t* pos, const mla_cache* cache, const int32_t* block_table,
                    int32_t max_pages, void* stream) {
  return append_common(dims, act_dtype, c_kv, k_rope, n_tok, seq_id, pos, nullptr, nullptr, cache, block_table,
                       max_pages, stream, true);
}

int32_t mla_default_splits(const mla_dims* dims, int32_t batch, int32_t s_q, int32_t max_pages) {
  if (check_dims(dims) || batch <= 0 || s_q <= 0 || max_pages <= 0) return 0;
  const int rows = dims->n_heads * s_q;
  const int row_blocks = (rows + 127) / 128;
  long items = (long)batch * row_blocks;
  int s = (int)((TARGET_ITEMS + items - 1) / items);
  const int s_cap = (max_pages + MAX_PAGES_PER_SPLIT - 1) / MAX_PAGES_PER_SPLIT;
  if (s < s_cap) s = s_cap;
  if (s > max_pages) s = max_pages;
  if (s > MAX_SPLITS) s = MAX_SPLITS;
  return s < 1 ? 1 : s;
}

// From the lengths: a batch whose longest sequence is within 1/16 of the mean
// balances with one item per CU, and the page cap above would only add the
// fixed cost of more items (query rows loaded, partial rows written and
// merged); any other batch takes the default.
int32_t mla_plan_splits(const mla_dims* dims, int32_t batch, int32_t s_q, int32_t max_pages,
                        const int32_t* seqlens) {
  if (check_dims(dims) || batch <= 0 || s_q <= 0 || max_pages <= 0 || !seqlens) return 0;
  long sum = 0;
  int lmax = 0;
  for (int b = 0; b < batch; ++b) {
    const int L = seqlens[b];
    if (L < 0 || (long)L > (long)max_pages * dims->page_size) return 0;
    sum += L;
    lmax = L > lmax ? L : lmax;
  }
  const int fallback = mla_default_splits(dims, batch, s_q, max_pages);
  if (lmax == 0 || (long)lmax * batch * 16 > sum * 17) return fallback;
  const long items = (long)batch * ((dims->n_heads * s_q + 127) / 128);
  int s = (int)((TARGET_ITEMS + items - 1) / items);
  const int pages = (lmax + dims->page_size - 1) / dims->page_size;
  if (s > pages) s = pages;
  if (s > max_pages) s = max_pages;
  if (s > MAX_SPLITS) s = MAX_SPLITS;
  return s < 1 ? 1 : s;
}

size_t mla_workspace_bytes(const mla_dims* dims, int32_t act_dtype, int32_t batch, int32_t s_q, int32_t num_splits) {
  if (check_dims(dims) || !valid_act(act_dtype) || batch <= 0 || s_q <= 0 || s_q > MAX_S_Q || num_splits <= 0 ||
      num_splits > MAX_SPLITS)
    return 0;
  return ws_layout(*dims, act_dtype, batch, s_q, num_splits).total;
}

static int decode_impl(const mla_dims* dims, int32_t act_dtype, const void* hq, int32_t batch, int32_t s_q,
                       const void* W_DQ, const void* W_UQ, const void* W_UK, const mla_cache* cache,
                       const int32_t* block_table, int32_t max_pages, const int32_t* seqlens, float softmax_scale,
                       int32_t num_splits, void* ws, size_t ws_bytes, void* stream, int parts) {
  int st = check_dims(dims);
  if (st) return st;
  if (!valid_act(act_dtype)) return MLA_ERR_DTYPE;
  if (batch < 0 || s_q < 1 || s_q > MAX_S_Q || num_splits < 0 || num_splits > MAX_SPLITS) return MLA_ERR_DIMS;
  if ((st = check_cache(dims, cache, block_table, max_pages))) return st;
  if (act_dtype == MLA_BF16 && cache->dtype == MLA_F32) return MLA_ERR_DTYPE;
  if (!(softmax_scale == softmax_scale)) return MLA_ERR_DIMS;
  if (batch == 0) return MLA_OK;
  if (!seqlens || !ws) return MLA_ERR_NULL;
  if (!aligned16(seqlens) || !aligned16(ws)) return MLA_ERR_ALIGN;
  if (parts & 1) {  // the attention alone reads only the workspace's queries, the cache and seqlens
    if (!hq || !W_UQ || !W_UK) return MLA_ERR_NULL;
    if (!aligned16(hq) || !aligned16(W_UQ) || !aligned16(W_UK) || (W_DQ && !aligned16(W_DQ))) return MLA_ERR_ALIGN;
  }
  DecodeArgs a;
  a.d = *dims; a.act = act_dtype; a.cache_dtype = cache->dtype; a.hq = hq; a.batch = batch; a.s_q = s_q;
  a.W_DQ = W_DQ; a.W_UQ = W_UQ; a.W_UK = W_UK; a.pages = (const uint8_t*)cache->pages;
  a.g = make_geom(*dims, cache->dtype); a.block_table = block_table; a.max_pages = max_pages; a.seqlens = seqlens;
  a.scale = softmax_scale;
  resolve_splits(dims, batch, s_q, max_pages, num_splits, &a.S, &a.pages_per_split);
  a.L = ws_layout(*dims, act_dtype, batch, s_q, a.S);
  if (ws_bytes < a.L.total) return MLA_ERR_WORKSPACE;
  a.ws = (uint8_t*)ws; a.stream = (hipStream_t)stream;
  const bool fast = !force_generic() && fast_decode_supported(*dims, act_dtype, cache->dtype, s_q);
  hipError_t e = hipSuccess;
  if (parts & 1) e = fast ? fast_query(a) : generic_query(a);
  if (e == hipSuccess && (parts & 2)) e = fast ? fast_attention(a) : generic_attention(a);
  return hip_status(e);
}

int mla_decode(const mla_dims* dims, int32_t act_dtype, const void* hq, int32_t batch, int32_t s_q, const void* W_DQ,
               const void* W_UQ, const void* W_UK, const mla_cache* cache, const int32_t* block_table,
               int32_t max_pages, const int32_t* seqlens, float softmax_scale, int32_t num_splits, void* ws,
               size_t ws_bytes, void* stream) {
  return decode_impl(dims, act_dtype, hq, batch, s_q, W_DQ, W_UQ, W_UK, cache, block_table, max_pages, seqlens,
                     softmax_scale, num_splits, ws, ws_bytes, stream, 3);
}

int mla_decode_query(const mla_dims* dims, int32_t act_dtype, const void* hq, int32_t batch, int32_t s_q,
                     const void* W_DQ, const void* W_UQ, const void* W_UK, const mla_cache* cache,
                     const int32_t* block_table, int32_t max_pages, const int32_t* seqlens, float softmax_scale,
                     int32_t num_splits, void* ws, size_t ws_bytes, void* stream) {
  return decode_impl(dims, act_dtype, hq, batch, s_q, W_DQ, W_UQ, W_UK, cache, block_table, max_pages, seqlens,
                     softmax_scale, num_splits, ws, ws_bytes, stream, 1);
}

int mla_decode_attend(const mla_dims* dims, int32_t act_dtype, const void* hq, int32_t batch, int32_t s_q,
                      const void* W_DQ, const void* W_UQ, const void* W_UK, const mla_cache* cache,
                      const int32_t* block_table, int32_t max_pages, const int32_t* seqlens, float softmax_scale,
                      int32_t num_splits, void* ws, size_t ws_bytes, void* stream) {
  return decode_impl(dims, act_dtype, hq, batch, s_q, W_DQ, W_UQ, W_UK, cache, block_table, max_pages, seqlens,
                     softmax_scale, num_splits, ws, ws_bytes, stream, 2);
}

int32_t mla_decode_splits(const mla_dims* dims, int32_t batch, int32_t s_q, int32_t max_pages, int32_t num_splits) {
  if (check_dims(dims) || batch <= 0 || s_q <= 0 || s_q > MAX_S_Q || max_pages <= 0 || num_splits < 0 ||
      num_splits > MAX_SPLITS)
    return 0;
  int S = 0, pps = 0;
  resolve_splits(dims, batch, s_q, max_pages, num_splits, &S, &pps);
  return S;
}

int mla_combine(const mla_dims* dims, int32_t act_dtype, int32_t batch, int32_t s_q, int32_t num_splits, void* ws,
                size_t ws_bytes, const void* W_UV, void* out, float* lse_out, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!valid_act(act_dtype)) return MLA_ERR_DTYPE;
  if (batch < 0 || s_q < 1 || s_q > MAX_S_Q || num_splits < 1 || num_splits > MAX_SPLITS) return MLA_ERR_DIMS;
  if (batch == 0) return MLA_OK;
  if (!ws || !W_UV || !out) return MLA_ERR_NULL;
  if (!aligned16(ws) || !aligned16(W_UV) || !aligned16(out) || (lse_out && !aligned16(lse_out))) return MLA_ERR_ALIGN;
  // The workspace must hold the plan of num_splits splits; the kernels read
  // exactly that many partials, so a too-small workspace is refused here.
  const WsLayout L = ws_layout(*dims, act_dtype, batch, s_q, num_splits);
  if (ws_bytes < L.total) return MLA_ERR_WORKSPACE;
  CombineArgs a;
  a.d = *dims; a.act = act_dtype; a.batch = batch; a.s_q = s_q; a.S = num_splits; a.ws = (uint8_t*)ws;
  a.W_UV = W_UV; a.out = out; a.lse_out = lse_out; a.stream = (hipStream_t)stream; a.L = L;
  hipError_t e;
  if (!force_generic() && fast_decode_supported(*dims, act_dtype, MLA_BF16, s_q)) e = fast_combine(a);
  else e = generic_combine(a);
  return hip_status(e);
}

size_t mla_decode_fp8w_workspace_bytes(const mla_dims* dims, int32_t batch, int32_t s_q, int32_t num_splits) {
  if (check_dims(dims) || batch <= 0 || s_q <= 0 || s_q > MAX_S_Q || num_splits <= 0 || num_splits > MAX_SPLITS ||
      !fp8w_supported(*dims))
    return 0;
  const WsLayout L = ws_layout(*dims, MLA_BF16, batch, s_q, num_splits);
  return fp8w_scratch_offset(L) + fp8w_scratch_bytes(*dims, batch * s_q);
}

static bool aligned4(const void* p) { return ((uintptr_t)p & 3) == 0; }

static int fp8w_decode_impl(const mla_dims* dims, const void* hq, int32_t batch, int32_t s_q, const void* W_DQ_codes,
                            const float* W_DQ_scales, const void* W_UQ_codes, const float* W_UQ_scales,
                            const void* W_UKT_codes, const float* W_UKT_scales, const mla_cache* cache,
                            const int32_t* block_table, int32_t max_pages, const int32_t* seqlens,
                            float softmax_scale, int32_t num_splits, void* ws, size_t ws_bytes, void* stream,
                            int parts) {
  int st = check_dims(dims);
  if (st) return st;
  if (batch < 0 || s_q < 1 || s_q > MAX_S_Q || num_splits < 0 || num_splits > MAX_SPLITS) return MLA_ERR_DIMS;
  if ((st = check_cache(dims, cache, block_table, max_pages))) return st;
  if (cache->dtype == MLA_F32) return MLA_ERR_DTYPE;
  if (!(softmax_scale == softmax_scale)) return MLA_ERR_DIMS;
  if (force_generic() || !fp8w_supported(*dims) || !fast_decode_supported(*dims, MLA_BF16, cache->dtype, s_q))
    return MLA_ERR_UNSUPPORTED;
  if (batch == 0) return MLA_OK;
  if (!seqlens || !ws) return MLA_ERR_NULL;
  if (!aligned16(seqlens) || !aligned16(ws)) return MLA_ERR_ALIGN;
  if (parts & 1) {
    if (!hq || !W_DQ_codes || !W_DQ_scales || !W_UQ_codes || !W_UQ_scales || !W_UKT_codes || !W_UKT_scales)
      return MLA_ERR_NULL;
    if (!aligned16(hq) || !aligned16(W_DQ_codes) || !aligned16(W_UQ_codes) || !aligned16(W_UKT_codes) ||
        !aligned4(W_DQ_scales) || !aligned4(W_UQ_scales) || !aligned4(W_UKT_scales))
      return MLA_ERR_ALIGN;
  }
  DecodeArgs a;
  a.d = *dims; a.act = MLA_BF16; a.cache_dtype = cache->dtype; a.hq = hq; a.batch = batch; a.s_q = s_q;
  a.W_DQ = nullptr; a.W_UQ = nullptr; a.W_UK = nullptr; a.pages = (const uint8_t*)cache->pages;
  a.g = make_geom(*dims, cache->dtype); a.block_table = block_table; a.max_pages = max_pages; a.seqlens = seqlens;
  a.scale = softmax_scale;
  resolve_splits(dims, batch, s_q, max_pages, num_splits, &a.S, &a.pages_per_split);
  a.L = ws_layout(*dims, MLA_BF16, batch, s_q, a.S);
  if (ws_bytes < fp8w_scratch_offset(a.L) + fp8w_scratch_bytes(*dims, batch * s_q)) return MLA_ERR_WORKSPACE;
  a.ws = (uint8_t*)ws; a.stream = (hipStream_t)stream;
  const Fp8Weights w{(const uint8_t*)W_DQ_codes, (const uint8_t*)W_UQ_codes, (const uint8_t*)W_UKT_codes,
                     W_DQ_scales, W_UQ_scales, W_UKT_scales};
  hipError_t e = hipSuccess;
  if (parts & 1) e = fp8w_query(a, w);
  if (e == hipSuccess && (parts & 2)) e = fast_attention(a);
  return hip_status(e);
}

int mla_decode_fp8w(const mla_dims* dims, const void* hq, int32_t batch, int32_t s_q, const void* W_DQ_codes,
                    const float* W_DQ_scales, const void* W_UQ_codes, const float* W_UQ_scales,
                    const void* W_UKT_codes, const float* W_UKT_scales, const mla_cache* cache,
                    const int32_t* block_table, int32_t max_pages, const int32_t* seqlens, float softmax_scale,
                    int32_t num_splits, void* ws, size_t ws_bytes, void* stream) {
  return fp8w_decode_impl(dims, hq, batch, s_q, W_DQ_codes, W_DQ_scales, W_UQ_codes, W_UQ_scales, W_UKT_codes,
                          W_UKT_scales, cache, block_table, max_pages, seqlens, softmax_scale, num_splits, ws,
                          ws_bytes, stream, 3);
}

int mla_decode_fp8w_query(const mla_dims* dims, const void* hq, int32_t batch, int32_t s_q, const void* W_DQ_codes,
                          const float* W_DQ_scales, const void* W_UQ_codes, const float* W_UQ_scales,
                          const void* W_UKT_codes, const float* W_UKT_scales, const mla_cache* cache,
                          const int32_t* block_table, int32_t max_pages, const int32_t* seqlens,
                          float softmax_scale, int32_t num_splits, void* ws, size_t ws_bytes, void* stream) {
  return fp8w_decode_impl(dims, hq, batch, s_q, W_DQ_codes, W_DQ_scales, W_UQ_codes, W_UQ_scales, W_UKT_codes,
                          W_UKT_scales, cache, block_table, max_pages, seqlens, softmax_scale, num_splits, ws,
                          ws_bytes, stream, 1);
}

int mla_combine_fp8w(const mla_dims* dims, int32_t batch, int32_t s_q, int32_t num_splits, void* ws,
                     size_t ws_bytes, const void* W_UV_codes, const float* W_UV_scales, void* out, float* lse_out,
                     void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (batch < 0 || s_q < 1 || s_q > MAX_S_Q || num_splits < 1 || num_splits > MAX_SPLITS) return MLA_ERR_DIMS;
  if (force_generic() || !fp8w_supported(*dims) || !fast_decode_supported(*dims, MLA_BF16, MLA_BF16, s_q))
    return MLA_ERR_UNSUPPORTED;
  if (batch == 0) return MLA_OK;
  if (!ws || !W_UV_codes || !W_UV_scales || !out) return MLA_ERR_NULL;
  if (!aligned16(ws) || !aligned16(W_UV_codes) || !aligned4(W_UV_scales) || !aligned16(out) ||
      (lse_out && !aligned16(lse_out)))
    return MLA_ERR_ALIGN;
  const WsLayout L = ws_layout(*dims, MLA_BF16, batch, s_q, num_splits);
  if (ws_bytes < L.total) return MLA_ERR_WORKSPACE;
  CombineArgs a;
  a.d = *dims; a.act = MLA_BF16; a.batch = batch; a.s_q = s_q; a.S = num_splits; a.ws = (uint8_t*)ws;
  a.W_UV = nullptr; a.out = out; a.lse_out = lse_out; a.stream = (hipStream_t)stream; a.L = L;
  return hip_status(fp8w_combine(a, (const uint8_t*)W_UV_codes, W_UV_scales));
}

int mla_decode_step_noalloc(const mla_dims* dims, int32_t act_dtype, const void* hq, int32_t batch, int32_t s_q,
                            const void* W_DQ, const void* W_UQ, const void* W_UK, const void* W_UV,
                            const mla_cache* cache, const int32_t* block_table, int32_t max_pages,
                            const int32_t* seqlens, float softmax_scale, int32_t num_splits, void* out,
                            float* lse_out, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!valid_act(act_dtype)) return MLA_ERR_DTYPE;
  if (batch < 0 || s_q < 1 || s_q > MAX_S_Q || num_splits < 0 || num_splits > MAX_SPLITS) return MLA_ERR_DIMS;
  if ((st = check_cache(dims, cache, block_table, max_pages))) return st;
  if (act_dtype == MLA_BF16 && cache->dtype == MLA_F32) return MLA_ERR_DTYPE;
  if (!(softmax_scale == softmax_scale)) return MLA_ERR_DIMS;
  if (force_generic() || !fast_decode_supported(*dims, act_dtype, cache->dtype, s_q)) return MLA_ERR_UNSUPPORTED;
  if (batch == 0) return MLA_OK;
  if (!hq || !W_UQ || !W_UK || !W_UV || !seqlens || !out) return MLA_ERR_NULL;
  if (!aligned16(hq) || !aligned16(W_UQ) || !aligned16(W_UK) || !aligned16(W_UV) || !aligned16(seqlens) ||
      !aligned16(out) || (W_DQ && !aligned16(W_DQ)) || (lse_out && !aligned16(lse_out)))
    return MLA_ERR_ALIGN;
  DecodeArgs a;
  a.d = *dims; a.act = act_dtype; a.cache_dtype = cache->dtype; a.hq = hq; a.batch = batch; a.s_q = s_q;
  a.W_DQ = W_DQ; a.W_UQ = W_UQ; a.W_UK = W_UK; a.pages = (const uint8_t*)cache->pages;
  a.g = make_geom(*dims, cache->dtype); a.block_table = block_table; a.max_pages = max_pages; a.seqlens = seqlens;
  a.scale = softmax_scale;
  resolve_splits(dims, batch, s_q, max_pages, num_splits, &a.S, &a.pages_per_split);
  a.L = noalloc_layout(*dims, batch, s_q, a.S);
  if (a.L.total > (size_t)MLA_NOALLOC_SCRATCH_BYTES) return MLA_ERR_WORKSPACE;
  a.stream = (hipStream_t)stream;
  CombineArgs c;
  c.d = *dims; c.act = act_dtype; c.batch = batch; c.s_q = s_q; c.S = a.S; c.L = a.L;
  c.W_UV = W_UV; c.out = out; c.lse_out = lse_out; c.stream = a.stream;
  return hip_status(noalloc_decode_step(a, c));
}

size_t mla_prefill_workspace_bytes(const mla_dims* dims, int32_t act_dtype, int32_t n_tok) {
  if (check_dims(dims) || !valid_act(act_dtype) || n_tok < 0 || n_tok > MAX_PREFILL_TOKENS) return 0;
  return prefill_layout(*dims, n_tok).total;
}

}  // extern "C"

namespace {
enum PrefillPart { PREFILL_ALL, PREFILL_PROJECT, PREFILL_ATTEND };

int prefill_common(PrefillPart part, const mla_dims* dims, int32_t act_dtype, const void* h, int32_t n_tok,
                   int32_t n_seq, const int32_t* cu_seqlens, int32_t max_seqlen, const void* W_DQ, const void* W_UQ,
                   const void* W_UK, const void* W_UV, const void* W_DKV, const void* W_KR, float softmax_scale,
                   void* out, float* lse_out, void* ws, size_t ws_bytes, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!valid_act(act_dtype)) return MLA_ERR_DTYPE;
  if (n_tok < 0 || n_tok > MAX_PREFILL_TOKENS || n_seq < 1 || n_seq > 65535 || max_seqlen < 1) return MLA_ERR_DIMS;
  if (n_tok == 0) return MLA_OK;
  if (!prefill_supported(*dims, act_dtype)) return MLA_ERR_UNSUPPORTED;
  if (!h || !cu_seqlens || !W_DQ || !W_UQ || !W_UK || !W_UV || !W_DKV || !W_KR || !out || !ws) return MLA_ERR_NULL;
  const void* ptrs[] = {h, cu_seqlens, W_DQ, W_UQ, W_UK, W_UV, W_DKV, W_KR, out, ws};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MLA_ERR_ALIGN;
  if (lse_out && ((uintptr_t)lse_out & 3)) return MLA_ERR_ALIGN;
  if (!(softmax_scale > 0.0f)) return MLA_ERR_DIMS;
  const PrefillLayout L = prefill_layout(*dims, n_tok);
  if (ws_bytes < L.total) return MLA_ERR_WORKSPACE;
  PrefillArgs a;
  // no sequence is longer than all tokens together
  a.d = *dims; a.h = (const bf16_t*)h; a.n_tok = n_tok; a.n_seq = n_seq; a.max_seqlen = std::min(max_seqlen, n_tok);
  a.cu_seqlens = cu_seqlens;
  a.W_DQ = (const bf16_t*)W_DQ; a.W_UQ = (const bf16_t*)W_UQ; a.W_UK = (const bf16_t*)W_UK;
  a.W_UV = (const bf16_t*)W_UV; a.W_DKV = (const bf16_t*)W_DKV; a.W_KR = (const bf16_t*)W_KR;
  a.scale = softmax_scale; a.out = (bf16_t*)out; a.lse_out = lse_out; a.ws = (uint8_t*)ws; a.L = L;
  a.stream = (hipStream_t)stream;
  switch (part) {
    case PREFILL_PROJECT: return hip_status(prefill_projections(a));
    case PREFILL_ATTEND: return hip_status(prefill_attention(a));
    default: return hip_status(fast_prefill(a));
  }
}
}  // namespace

extern "C" {

#define MLA_PREFILL_ARGS                                                                                          \
  const mla_dims *dims, int32_t act_dtype, const void *h, int32_t n_tok, int32_t n_seq, const int32_t *cu_seqlens, \
      int32_t max_seqlen, const void *W_DQ, const void *W_UQ, const void *W_UK, const void *W_UV,                 \
      const void *W_DKV, const void *W_KR, float softmax_scale, void *out, float *lse_out, void *ws,            \
      size_t ws_bytes, void *stream
#define MLA_PREFILL_PASS                                                                                        \
  dims, act_dtype, h, n_tok, n_seq, cu_seqlens, max_seqlen, W_DQ, W_UQ, W_UK, W_UV, W_DKV, W_KR, softmax_scale, \
      out, lse_out, ws, ws_bytes, stream

int mla_prefill(MLA_PREFILL_ARGS) { return prefill_common(PREFILL_ALL, MLA_PREFILL_PASS); }
int mla_prefill_project(MLA_PREFILL_ARGS) { return prefill_common(PREFILL_PROJECT, MLA_PREFILL_PASS); }
int mla_prefill_attend(MLA_PREFILL_ARGS) { return prefill_common(PREFILL_ATTEND, MLA_PREFILL_PASS); }

size_t mla_output_project_workspace_bytes(const mla_dims* dims, int32_t act_dtype, int32_t rows) {
  if (check_dims(dims) || !valid_act(act_dtype) || rows < 0 || rows > MAX_OUT_ROWS) return 0;
  return out_proj_ws_bytes(act_dtype, rows, dims->d_model, dims->n_heads * dims->d_head);
}

int mla_output_project(const mla_dims* dims, int32_t act_dtype, int32_t rows, const void* o, const void* W_O,
                       void* y, void* ws, size_t ws_bytes, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!valid_act(act_dtype)) return MLA_ERR_DTYPE;
  if (rows < 0 || rows > MAX_OUT_ROWS) return MLA_ERR_DIMS;
  if (rows == 0) return MLA_OK;
  if (!o || !W_O || !y) return MLA_ERR_NULL;
  if (!aligned16(o) || !aligned16(W_O) || !aligned16(y)) return MLA_ERR_ALIGN;
  OutProjArgs a;
  a.rows = rows; a.N = dims->d_model; a.K = dims->n_heads * dims->d_head; a.act = act_dtype;
  a.o = o; a.W_O = W_O; a.y = y; a.ws = (uint8_t*)ws; a.stream = (hipStream_t)stream;
  const size_t need = out_proj_ws_bytes(act_dtype, rows, a.N, a.K);
  if (need > 0 && (!ws || ws_bytes < need)) return MLA_ERR_WORKSPACE;
  if (need > 0 && !aligned16(ws)) return MLA_ERR_ALIGN;
  return hip_status(force_generic() ? generic_out_project(a) : out_project(a));
}

namespace {
int check_fp8_gemm_dims(int32_t N, int32_t K) {
  if (N < 1 || K < 1 || N > MAX_FP8_DIM || K > MAX_FP8_DIM) return MLA_ERR_DIMS;
  if (!fp8_gemm_supported(N, K)) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}
}  // namespace

int mla_fp8_quantize_weight(const void* W, int32_t N, int32_t K, void* codes, float* scales, void* stream) {
  if (N < 1 || K < 1 || N > MAX_FP8_DIM || K > MAX_FP8_DIM) return MLA_ERR_DIMS;
  if (N % 16 || K % 128) return MLA_ERR_UNSUPPORTED;
  if (!W || !codes || !scales) return MLA_ERR_NULL;
  if (!aligned16(W) || !aligned16(codes) || ((uintptr_t)scales & 3)) return MLA_ERR_ALIGN;
  return hip_status(fp8_quantize_weight(N, K, (const bf16_t*)W, (uint8_t*)codes, scales, (hipStream_t)stream));
}

int mla_fp8_quantize_weight_t(const void* W, int32_t batch, int32_t R, int32_t C, void* codes, float* scales,
                              void* stream) {
  if (batch < 1 || R < 1 || C < 1 || R > MAX_FP8_DIM || C > MAX_FP8_DIM || batch > MAX_FP8_DIM) return MLA_ERR_DIMS;
  if (R % 128 || C % 128) return MLA_ERR_UNSUPPORTED;
  if (!W || !codes || !scales) return MLA_ERR_NULL;
  if (!aligned16(W) || !aligned16(codes) || ((uintptr_t)scales & 3)) return MLA_ERR_ALIGN;
  return hip_status(
      fp8_quantize_weight_t(batch, R, C, (const bf16_t*)W, (uint8_t*)codes, scales, (hipStream_t)stream));
}

size_t mla_fp8_gemm_workspace_bytes(int32_t M, int32_t N, int32_t K) {
  if (M < 0 || M > MAX_OUT_ROWS || check_fp8_gemm_dims(N, K)) return 0;
  return fp8_plan(M, N, K).ws_bytes;
}

int mla_fp8_gemm(int32_t M, int32_t N, int32_t K, const void* X, const void* W_codes, const float* W_scales, void* Y,
                 void* ws, size_t ws_bytes, void* stream) {
  if (M < 0 || M > MAX_OUT_ROWS) return MLA_ERR_DIMS;
  const int st = check_fp8_gemm_dims(N, K);
  if (st) return st;
  if (M == 0) return MLA_OK;
  if (!X || !W_codes || !W_scales || !Y) return MLA_ERR_NULL;
  if (!aligned16(X) || !aligned16(W_codes) || !aligned16(Y) || ((uintptr_t)W_scales & 3)) return MLA_ERR_ALIGN;
  const size_t need = fp8_plan(M, N, K).ws_bytes;
  if (need > 0 && (!ws || ws_bytes < need)) return MLA_ERR_WORKSPACE;
  if (need > 0 && !aligned16(ws)) return MLA_ERR_ALIGN;
  return hip_status(fp8_gemm(M, N, K, (const bf16_t*)X, (const uint8_t*)W_codes, W_scales, (bf16_t*)Y, (uint8_t*)ws,
                             (hipStream_t)stream));
}

int mla_check_metadata(const mla_dims* dims, const mla_cache* cache, const int32_t* block_table, int32_t max_pages,
                       const int32_t* seqlens, int32_t batch, int32_t* bad, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (batch < 0) return MLA_ERR_DIMS;
  if ((st = check_cache(dims, cache, block_table, max_pages))) return st;
  if (!bad || (batch > 0 && !seqlens)) return MLA_ERR_NULL;
  if ((seqlens && !aligned16(seqlens)) || ((uintptr_t)bad & 3)) return MLA_ERR_ALIGN;
  return hip_status(check_metadata(batch, max_pages, dims->page_size, cache->num_pages, block_table, seqlens, bad,
                                   (hipStream_t)stream));
}

int mla_hbm_read_probe(const void* src, size_t bytes, int32_t* sink, void* stream) {
  if (bytes == 0) return MLA_OK;
  if (!src || !sink) return MLA_ERR_NULL;
  if (bytes % 16) return MLA_ERR_DIMS;
  if (!aligned16(src) || ((uintptr_t)sink & 3)) return MLA_ERR_ALIGN;
  return hip_status(read_probe(src, bytes, sink, (hipStream_t)stream));
}

int mla_mfma_probe(const void* ops, int32_t iters, float* sink, double* flops, void* stream) {
  if (iters < 0) return MLA_ERR_DIMS;
  if (flops) *flops = mfma_probe_flops(iters);
  if (iters == 0) return MLA_OK;
  if (!ops || !sink) return MLA_ERR_NULL;
  if (!aligned16(ops) || ((uintptr_t)sink & 3)) return MLA_ERR_ALIGN;
  return hip_status(mfma_probe(ops, iters, sink, (hipStream_t)stream));
}

double mla_mtp_tokens_per_step(double acceptance, int32_t depth) {
  if (!(acceptance >= 0.0 && acceptance <= 1.0) || depth < 0 || depth > MAX_S_Q - 1) return NAN;
  // Horner form of 1 + a + ... + a^depth: the draft chain's survival probabilities
  double t = 1.0;
  for (int k = 0; k < depth; ++k) t = 1.0 + acceptance * t;
  return t;
}

const char* mla_status_str(int s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL: return "required pointer is NULL";
    case MLA_ERR_DIMS: return "size out of range or inconsistent";
    case MLA_ERR_DTYPE: return "unsupported dtype or dtype combination";
    case MLA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case MLA_ERR_WORKSPACE: return "workspace missing or too small";
    case MLA_ERR_UNSUPPORTED: return "not implemented for these dims";
    case MLA_ERR_HIP: return "HIP runtime error while enqueueing";
    default: return "unknown status";
  }
}

const char* mla_last_hip_error(void) {
  return t_last_hip == hipSuccess ? "none" : hipGetErrorString(t_last_hip);
}

const char* mla_version(void) { return "libmla gfx950 (generic VALU + MFMA decode kernels)"; }

}  // extern "C"
