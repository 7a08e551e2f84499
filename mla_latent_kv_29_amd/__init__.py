"""MI355X-native MLA decode: DeepSeek-V3 Multi-head Latent Attention over a
paged latent cache (c^KV + shared k^R), with hand-written HIP kernels for
gfx950 behind the C ABI of include/mla.h (libmla.so); also the causal prefill
of fresh sequences in the non-absorbed form.

Python here only marshals arguments: `_lib` binds the C entry points by their
C names, `session` keeps the device buffers of one batch, `inputs` draws the
seeded synthetic inputs.
"""
from . import _lib
from ._lib import (mla_page_bytes, mla_cache_append, mla_cache_write, mla_default_splits, mla_plan_splits, mla_decode_splits,
                   mla_workspace_bytes, mla_decode, mla_decode_query, mla_decode_attend, mla_combine,
                   mla_prefill_workspace_bytes, mla_prefill, mla_prefill_project, mla_prefill_attend,
                   mla_output_project_workspace_bytes, mla_output_project, mla_fp8_quantize_weight,
                   mla_fp8_quantize_weight_t, mla_fp8_gemm_workspace_bytes, mla_fp8_gemm, mla_mtp_tokens_per_step,
                   mla_decode_fp8w_workspace_bytes, mla_decode_fp8w, mla_decode_fp8w_query, mla_combine_fp8w,
                   status_str, version, make_dims,
                   MLAError, MLA_F32, MLA_BF16, MLA_FP8_E4M3, MLA_FP8_E4M3_E8)

__all__ = ["mla_page_bytes", "mla_cache_append", "mla_cache_write", "mla_default_splits", "mla_plan_splits", "mla_decode_splits",
           "mla_workspace_bytes", "mla_decode", "mla_decode_query", "mla_decode_attend", "mla_combine",
           "mla_prefill_workspace_bytes", "mla_prefill", "mla_prefill_project", "mla_prefill_attend",
           "mla_output_project_workspace_bytes", "mla_output_project", "mla_fp8_quantize_weight",
           "mla_fp8_quantize_weight_t", "mla_fp8_gemm_workspace_bytes", "mla_fp8_gemm", "mla_mtp_tokens_per_step",
           "mla_decode_fp8w_workspace_bytes", "mla_decode_fp8w", "mla_decode_fp8w_query", "mla_combine_fp8w",
           "status_str", "version", "make_dims",
           "MLAError", "MLA_F32", "MLA_BF16", "MLA_FP8_E4M3", "MLA_FP8_E4M3_E8"]
