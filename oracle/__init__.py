"""Float64 CPU oracle for MLA decode -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import anything from this package.  The GPU library never calls it, and it
shares no code, tables or helpers with the GPU library: it is a plain, slow,
obviously-correct restatement of what the pages define.

Sources (cited by page title and section, never by file position):

* "Читаем техотчёт DeepSeek-V3 вместе" (ai.flicky.cc course lesson), section
  2.1.1 "MLA: что попадает в кэш" -- the latent-KV equations, the per-head key
  concatenation, the cache-size table and Question 2 (matrix absorption);
  section 3.3 "Обучение в FP8" -- E4M3/E5M2 ranges and 1x128 tile scaling;
  "Практика: перепроверяем числа статьи" -- the V3 shape dictionary, the MLA
  weight-shape docstring and the parameter breakdown table.
* "Báo cáo Kỹ thuật DeepSeek-V3" (xyznot.com paper summary), "Phương pháp",
  item 1 "Multi-head Latent Attention (MLA)" -- the same equations with the
  compressed query c^Q.
* The same lesson, section 2.2 "Multi-Token Prediction" and the
  `tokens_per_step` docstring of its practice part -- the verify-step model.

Parity status per function is listed in each module header.
"""
from .mla import (rope, kv_latents, queries, attend_nonabsorbed, attend_absorbed,
                  decode_from_latents, decode_from_h, softmax_lse, output_projection)
from .fp8 import (e4m3_decode, e4m3_encode, e4m3_values, e5m2_decode,
                  quantize_tiles, dequantize_tiles, pow2_ceil, quantize_blocks, dequantize_blocks,
                  gemm_block_scaled)
from .fp8w import decode_absorbed_exact, decode_fp8w_from_latents, bf16_round
from .sizes import (cache_values_per_token, mha_values_per_token, cache_bytes,
                    mla_params_per_layer)
from .mtp import tokens_per_step

__all__ = [
    "rope", "kv_latents", "queries", "attend_nonabsorbed", "attend_absorbed",
    "decode_from_latents", "decode_from_h", "softmax_lse", "output_projection",
    "e4m3_decode", "e4m3_encode", "e4m3_values", "e5m2_decode",
    "quantize_tiles", "dequantize_tiles", "pow2_ceil", "quantize_blocks", "dequantize_blocks", "gemm_block_scaled",
    "decode_absorbed_exact", "decode_fp8w_from_latents", "bf16_round",
    "cache_values_per_token", "mha_values_per_token", "cache_bytes",
    "mla_params_per_layer", "tokens_per_step",
]
