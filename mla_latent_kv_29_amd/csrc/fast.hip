// Dispatch of the MFMA path for the DeepSeek-V3 MLA shape (d_c 512, d_rope
// 64, 128 heads of 128, 64-token pages, bf16 activations).
#include "internal.hpp"

namespace mla {

static bool v3_shape(const mla_dims& d) {
  return d.d_c == 512 && d.d_rope == 64 && d.n_heads == 128 && d.d_head == 128 && d.page_size == 64 &&
         d.d_model % 32 == 0 && d.d_cq % 64 == 0;
}

bool fast_append_supported(const mla_dims& d, int act, int cache_dtype) {
  return fast_append_shape(d) && act == MLA_BF16 && (cache_dtype == MLA_BF16 || cache_dtype == MLA_FP8_E4M3);
}

bool fast_decode_supported(const mla_dims& d, int act, int cache_dtype, int s_q) {
  return v3_shape(d) && act == MLA_BF16 && (cache_dtype == MLA_BF16 || cache_dtype == MLA_FP8_E4M3) && s_q >= 1 &&
         s_q <= 8;
}

hipError_t fast_decode(const DecodeArgs& a) {
  hipError_t e = fast_query(a);
  if (e != hipSuccess) return e;
  return fast_attention(a);
}

hipError_t fast_attention(const DecodeArgs& a) { return fast_attention_b(a); }

hipError_t fast_combine(const CombineArgs& a) { return fast_combine_mfma(a); }

}  // namespace mla
