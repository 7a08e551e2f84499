"""Cache-size and weight-count arithmetic -- TEST INFRASTRUCTURE ONLY.

Sources: "Читаем техотчёт DeepSeek-V3 вместе", §2.1.1, the MHA-vs-MLA cache
table (numbers per token per layer, bytes over 61 layers in BF16, one 128K
sequence, binary units); "Практика: перепроверяем числа статьи", the
attention_params docstring (the five groups of MLA matrices) and the parameter
breakdown table (MLA attention, 61 layers: 11.4B).
"""


def cache_values_per_token(d_c, d_rope):
    """MLA caches only c^KV and the shared k^R: d_c + d_rope numbers."""
    return d_c + d_rope


def mha_values_per_token(n_heads, d_head):
    """Full multi-head K and V of the same shape: 2 * heads * d_head numbers."""
    return 2 * n_heads * d_head


def cache_bytes(values_per_token, n_layers, n_tokens, bytes_per_value=2):
    """Bytes for `n_tokens` tokens over `n_layers` layers."""
    return values_per_token * n_layers * n_tokens * bytes_per_value


def mla_params_per_layer(d, n_heads, d_head, d_rope, d_c, d_q):
    """Sum of the five MLA weight groups of one layer:
    W_DQ d x d_q; W_UQ d_q x heads*(d_head + d_rope); W_DKV and W_KR
    d x (d_c + d_rope); W_UK and W_UV d_c x heads*d_head each;
    W_O heads*d_head x d.
    """
    return (d * d_q
            + d_q * n_heads * (d_head + d_rope)
            + d * (d_c + d_rope)
            + 2 * d_c * n_heads * d_head
            + n_heads * d_head * d)
