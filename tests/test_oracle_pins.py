"""Pins for the float64 oracle: every check below is fixed by the pages or by
mathematics, not by re-running the oracle's own formula.

Pages: "Читаем техотчёт DeepSeek-V3 вместе" (ai.flicky.cc lesson) §2.1.1 and
§3.3, its practice section and quiz; "Báo cáo Kỹ thuật DeepSeek-V3"
(xyznot.com), Phương pháp item 1.
"""
import json
import os

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")
TINY = dict(d_model=32, n_heads=3, d_head=8, d_rope=6, d_c=12, d_cq=10, rope_theta=10000.0)


def tiny_weights(rng, dims=TINY, sigma=0.3):
    d, H, dh, dr, dc, dq = (dims[k] for k in ("d_model", "n_heads", "d_head", "d_rope", "d_c", "d_cq"))
    return {
        "W_DKV": rng.normal(0, sigma, (dc, d)),
        "W_KR": rng.normal(0, sigma, (dr, d)),
        "W_DQ": rng.normal(0, sigma, (dq, d)),
        "W_UQ": rng.normal(0, sigma, (H * (dh + dr), dq)),
        "W_UK": rng.normal(0, sigma, (H * dh, dc)),
        "W_UV": rng.normal(0, sigma, (H * dh, dc)),
    }


# ---------------------------------------------------------------- worked numbers

def test_cache_table_matches_printed_numbers():
    g = json.load(open(os.path.join(GOLD, "cache_table.json")))
    d, pr = g["dims"], g["printed"]
    mla = oracle.cache_values_per_token(d["d_c"], d["d_rope"])
    mha = oracle.mha_values_per_token(d["n_heads"], d["d_head"])
    assert mla == pr["mla_values_per_token_layer"]
    assert mha == pr["mha_values_per_token_layer"]
    KiB, MiB, GiB = 1024.0, 1024.0 ** 2, 1024.0 ** 3
    b_mla = oracle.cache_bytes(mla, d["n_layers"], 1, d["bytes_bf16"])
    b_mha = oracle.cache_bytes(mha, d["n_layers"], 1, d["bytes_bf16"])
    assert round(b_mla / KiB, 1) == pr["mla_bytes_per_token_61_layers_KiB_approx"]
    assert round(b_mha / MiB, 1) == pr["mha_bytes_per_token_61_layers_MiB_approx"]
    s_mla = oracle.cache_bytes(mla, d["n_layers"], d["seq_128k"], d["bytes_bf16"])
    s_mha = oracle.cache_bytes(mha, d["n_layers"], d["seq_128k"], d["bytes_bf16"])
    assert round(s_mla / GiB, 1) == pr["mla_128k_sequence_GiB_approx"]
    assert round(s_mha / GiB) == pr["mha_128k_sequence_GiB_approx"]
    assert round(mha / mla) == pr["ratio_approx"]


def test_weight_shapes_reproduce_mla_parameter_total():
    g = json.load(open(os.path.join(GOLD, "v3_shapes.json")))
    v = g["V3"]
    per_layer = oracle.mla_params_per_layer(v["d"], v["heads"], v["d_head"], v["d_rope"], v["d_c"], v["d_q"])
    assert round(per_layer * v["layers"] / 1e9, 1) == g["printed"]["mla_params_61_layers_billions_approx"]


# ---------------------------------------------------------------- fp8 codec

def test_fp8_format_maxima_match_pages():
    g = json.load(open(os.path.join(GOLD, "fp8_formats.json")))["printed"]
    v4 = oracle.e4m3_decode(np.arange(256))
    v5 = oracle.e5m2_decode(np.arange(256))
    assert np.nanmax(v4) == g["e4m3_max"]
    assert np.max(v5[np.isfinite(v5)]) == g["e5m2_max"]


def test_e4m3_table_structure():
    v = oracle.e4m3_decode(np.arange(256))
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.sum(np.isnan(v)) == 2                   # E4M3FN: only S.1111.111 is NaN
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)                   # codes 0..126 strictly increasing
    assert pos[1] == 2.0 ** -9                        # smallest subnormal
    assert pos[8] == 2.0 ** -6                        # smallest normal
    assert pos[0x38] == 1.0                           # exponent bias 7
    np.testing.assert_array_equal(v[0x80:0xFF], -pos)  # sign bit
    # spacing: 8 values per binade above the subnormals
    for e in range(1, 16):
        lo = 2.0 ** (e - 7)
        binade = pos[(pos >= lo) & (pos < 2 * lo)]
        assert len(binade) == (8 if e < 15 else 7)


def test_e4m3_encode_roundtrip_ties_and_saturation():
    codes = np.arange(0, 0x7F)
    vals = oracle.e4m3_decode(codes)
    np.testing.assert_array_equal(oracle.e4m3_encode(vals), codes)
    np.testing.assert_array_equal(oracle.e4m3_encode(-vals[1:]), codes[1:] | 0x80)
    mids = 0.5 * (vals[:-1] + vals[1:])               # exact midpoints -> even code
    enc = oracle.e4m3_encode(mids).astype(int)
    expect = np.where(codes[:-1] % 2 == 0, codes[:-1], codes[1:])
    np.testing.assert_array_equal(enc, expect)
    assert oracle.e4m3_encode(np.array([1e9, -1e9, 449.0, 460.0])).tolist() == [0x7E, 0xFE, 0x7E, 0x7E]
    # hand-worked examples: 1.0625 lies halfway between 1 (0x38) and 1.125 (0x39)
    assert oracle.e4m3_encode(np.array([1.0625, 1.1875, 3.0, 2.0 ** -10])).tolist() == [0x38, 0x3A, 0x44, 0x00]


def test_tile_quantisation_error_bound_and_amax():
    rng = np.random.default_rng(3)
    x = rng.normal(0, 0.5, (7, 256))
    x[2, :128] = 0.0                                   # an all-zero tile -> scale 1, codes 0
    codes, scales = oracle.quantize_tiles(x)
    xt = oracle.dequantize_tiles(codes, scales)
    assert scales[2, 0] == 1.0 and np.all(codes[2, :128] == 0)
    g = np.abs(x.reshape(7, 2, 128))
    amax = g.max(axis=2)
    # every value is within half an E4M3 step (2^-4 relative in the normal range,
    # 2^-10 * scale absolute in the subnormal range), saturation never triggers
    err = np.abs(xt - x).reshape(7, 2, 128)
    bound = np.maximum(g * 2.0 ** -4, 2.0 ** -10 * scales[:, :, None]) * (1 + 1e-6)
    assert np.all(err <= bound)
    # the amax element of each non-zero tile maps to the largest code
    for r in range(7):
        for t in range(2):
            if amax[r, t] > 0:
                k = np.argmax(g[r, t])
                assert codes[r, t * 128 + k] & 0x7F == 0x7E


def test_pow2_ceil_known_values():
    """Smallest power of two not below s (the UE8M0 scale rule), by hand."""
    s = np.array([1.0, 1.5, 0.75, 3.0e-3, 2.0 ** -130, 448.0], dtype=np.float32)
    got = oracle.pow2_ceil(s)
    np.testing.assert_array_equal(got, np.array([1.0, 2.0, 1.0, 2.0 ** -8, 2.0 ** -126, 512.0], dtype=np.float32))


def test_ue8m0_tiles_hand_worked():
    """amax 3 -> 3/448 = 0.0067 -> scale 2^-7; 3/2^-7 = 384 = 1.5 * 2^8 is code
    0x7C; -0.1/2^-7 = -12.8 rounds to -13 = -1.625 * 2^3, code 0xD5."""
    x = np.zeros((1, 128))
    x[0, 0], x[0, 1] = 3.0, -0.1
    codes, scales = oracle.quantize_tiles(x, scale_rule="ue8m0")
    assert scales[0, 0] == np.float32(2.0 ** -7)
    assert codes[0, 0] == 0x7C and codes[0, 1] == 0xD5 and np.all(codes[0, 2:] == 0)


def test_ue8m0_tiles_powers_of_two_no_saturation_bf16_exact():
    rng = np.random.default_rng(5)
    x = rng.normal(0, 0.7, (9, 512)) * np.exp(rng.normal(0, 3, (9, 1)))
    x[4, 128:256] = 0.0
    codes, scales = oracle.quantize_tiles(x, scale_rule="ue8m0")
    xt = oracle.dequantize_tiles(codes, scales)
    assert scales[4, 1] == 1.0 and np.all(codes[4, 128:256] == 0)
    g = np.abs(x.astype(np.float32).astype(np.float64)).reshape(9, 4, 128)
    amax = g.max(axis=2)
    m, _ = np.frexp(scales.astype(np.float64))
    assert np.all(m == 0.5)                                  # bare powers of two
    q = amax / 448.0
    nz = amax > 0
    assert np.all(scales[nz] >= q[nz] * (1 - 1e-6)) and np.all(scales[nz] / 2 < q[nz] * (1 + 1e-6))
    # no code saturates: every value within half an E4M3 step of its tile
    err = np.abs(xt - x).reshape(9, 4, 128)
    bound = np.maximum(g * 2.0 ** -4, 2.0 ** -10 * scales[:, :, None]) * (1 + 1e-6)
    assert np.all(err <= bound)
    # code * 2^k has at most 4 significant bits: exact in bfloat16
    f = xt.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), xt)
    assert np.all(f.view(np.uint32) & 0xFFFF == 0)


def test_ue8m0_equals_amax_rule_when_amax_over_448_is_a_power_of_two():
    rng = np.random.default_rng(6)
    x = rng.uniform(-1, 1, (3, 256))
    for r in range(3):
        for t in range(2):
            blk = x[r, 128 * t:128 * (t + 1)]
            k = np.argmax(np.abs(blk))
            blk[k] = np.sign(blk[k]) * 448.0 * 2.0 ** (-3 * r - t)
            blk[np.arange(128) != k] *= 0.9 * 448.0 * 2.0 ** (-3 * r - t)
    c1, s1 = oracle.quantize_tiles(x)
    c2, s2 = oracle.quantize_tiles(x, scale_rule="ue8m0")
    np.testing.assert_array_equal(s1, s2)
    np.testing.assert_array_equal(c1, c2)


# ---------------------------------------------------------------- RoPE

def test_rope_identity_norm_and_complex_form():
    rng = np.random.default_rng(0)
    x = rng.normal(size=(5, 16))
    np.testing.assert_array_equal(oracle.rope(x, np.zeros(5), 10000.0), x)
    pos = np.array([0, 1, 7, 4095, 131071])
    y = oracle.rope(x, pos, 10000.0)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    # textbook complex form: pair (x0, x1) as x0 + i x1, multiplied by e^{i pos w_m}
    z = x[:, 0::2] + 1j * x[:, 1::2]
    w = 10000.0 ** (-np.arange(8) * 2.0 / 16)
    zr = z * np.exp(1j * pos[:, None] * w[None, :])
    np.testing.assert_allclose(y[:, 0::2], zr.real, atol=1e-12)
    np.testing.assert_allclose(y[:, 1::2], zr.imag, atol=1e-12)


def test_rope_scores_depend_only_on_position_difference():
    rng = np.random.default_rng(1)
    q, k = rng.normal(size=16), rng.normal(size=16)
    for m, n in [(5, 2), (100, 37), (4000, 3999)]:
        base = oracle.rope(q[None], np.array([m]), 1e4)[0] @ oracle.rope(k[None], np.array([n]), 1e4)[0]
        for delta in (1, 17, 1000):
            sh = oracle.rope(q[None], np.array([m + delta]), 1e4)[0] @ oracle.rope(k[None], np.array([n + delta]), 1e4)[0]
            assert abs(sh - base) < 1e-10 * (1 + abs(base))


# ---------------------------------------------------------------- attention pins

def _setup(rng, T=9, s_q=1, dims=TINY):
    W = tiny_weights(rng, dims)
    h = rng.normal(size=(T, dims["d_model"]))
    return W, h


def test_softmax_rows_sum_to_one_and_lse_matches_library():
    rng = np.random.default_rng(2)
    s = rng.normal(0, 3, (4, 11))
    p, lse = oracle.softmax_lse(s)
    assert np.all(p >= 0)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, logsumexp(s, axis=1), rtol=1e-13)
    np.testing.assert_allclose(p, np.exp(s - logsumexp(s, axis=1, keepdims=True)), rtol=1e-12)
    p0, l0 = oracle.softmax_lse(np.zeros((2, 0)))
    assert p0.shape == (2, 0) and np.all(np.isneginf(l0))


def test_absorbed_equals_nonabsorbed():
    """§2.1.1 Question 2: q^T k^C = (q^T W^UK) c^KV, so folding W^UK into the
    query (and applying W^UV after the weighted sum) changes nothing."""
    rng = np.random.default_rng(4)
    W, h = _setup(rng, T=13)
    d = TINY
    c, kr = oracle.kv_latents(h, W["W_DKV"], W["W_KR"], np.arange(13), d["rope_theta"])
    qc, qr = oracle.queries(h[-1:], W["W_DQ"], W["W_UQ"], d["n_heads"], d["d_head"], d["d_rope"],
                            np.array([12]), d["rope_theta"])
    tau = 0.37
    o1, p1, l1 = oracle.attend_nonabsorbed(qc[0], qr[0], c, kr, W["W_UK"], W["W_UV"], d["d_head"], tau)
    o2, l2 = oracle.attend_absorbed(qc[0], qr[0], c, kr, W["W_UK"], W["W_UV"], d["d_head"], tau)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-12 * np.abs(o1).max())
    np.testing.assert_allclose(l1, l2, rtol=1e-12)


def test_one_token_cache_returns_value_row():
    rng = np.random.default_rng(5)
    W, h = _setup(rng, T=1)
    d = TINY
    o, lse = oracle.decode_from_h(h, W, d, seqlen=1, s_q=1, tau=0.5)
    c0 = W["W_DKV"] @ h[0]
    for i in range(d["n_heads"]):
        np.testing.assert_allclose(o[0, i], W["W_UV"][i * 8:(i + 1) * 8] @ c0, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("s_q", [1, 2, 3])
def test_zero_scale_gives_mean_of_visible_values(s_q):
    """tau = 0 makes the softmax uniform over the visible tokens, so each query
    j returns W^UV_i times the mean latent of tokens 0..L-s_q+j (causal)."""
    rng = np.random.default_rng(6)
    L = 10
    W, h = _setup(rng, T=L)
    d = TINY
    o, lse = oracle.decode_from_h(h, W, d, seqlen=L, s_q=s_q, tau=0.0)
    c = h @ W["W_DKV"].T
    for j in range(s_q):
        vis = L - s_q + j + 1
        mean_c = c[:vis].mean(axis=0)
        for i in range(d["n_heads"]):
            np.testing.assert_allclose(o[j, i], W["W_UV"][i * 8:(i + 1) * 8] @ mean_c, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse[j], np.log(vis), rtol=1e-13)


def test_planted_peak_through_content_and_rope_terms():
    """A token whose key aligns strongly with the query dominates the softmax:
    the output becomes that token's value row.  Planting through k^C checks the
    content term; planting through k^R alone checks the RoPE term and its sign."""
    rng = np.random.default_rng(7)
    d = TINY
    T, H, dh, dr = 20, d["n_heads"], d["d_head"], d["d_rope"]
    W = tiny_weights(rng)
    c = rng.normal(0, 0.1, (T, d["d_c"]))
    kr = rng.normal(0, 0.1, (T, dr))
    qc = rng.normal(size=(H, dh))
    qr = rng.normal(size=(H, dr))
    i, star = 1, 6
    W_UK_i = W["W_UK"][i * dh:(i + 1) * dh]
    # content route: c_star along W_UK_i^T q^C_i
    c1 = c.copy()
    c1[star] = 50.0 * (W_UK_i.T @ qc[i]) / np.linalg.norm(W_UK_i.T @ qc[i])
    o, p, _ = oracle.attend_nonabsorbed(qc, qr, c1, kr, W["W_UK"], W["W_UV"], dh, 1.0, heads=[i])
    assert p[0, star] > 0.999
    np.testing.assert_allclose(o[0], W["W_UV"][i * dh:(i + 1) * dh] @ c1[star], rtol=2e-3)
    # rope route: k^R_star along q^R_i, content untouched
    kr2 = kr.copy()
    kr2[star] = 40.0 * qr[i] / np.linalg.norm(qr[i])
    o2, p2, _ = oracle.attend_nonabsorbed(qc, qr, c, kr2, W["W_UK"], W["W_UV"], dh, 1.0, heads=[i])
    assert p2[0, star] > 0.999
    # and with the opposite sign the planted token is suppressed
    kr3 = kr.copy()
    kr3[star] = -40.0 * qr[i] / np.linalg.norm(qr[i])
    _, p3, _ = oracle.attend_nonabsorbed(qc, qr, c, kr3, W["W_UK"], W["W_UV"], dh, 1.0, heads=[i])
    assert p3[0, star] < 1e-6


def test_query_and_key_at_same_position_see_unrotated_rope_dot():
    """The last query sits at the same position as the last cached token, so
    its RoPE score term equals the dot product of the unrotated parts."""
    rng = np.random.default_rng(8)
    d = TINY
    L = 17
    W, h = _setup(rng, T=L)
    c, kr = oracle.kv_latents(h, W["W_DKV"], W["W_KR"], np.arange(L), d["rope_theta"])
    qc, qr = oracle.queries(h[-1:], W["W_DQ"], W["W_UQ"], d["n_heads"], d["d_head"], d["d_rope"],
                            np.array([L - 1]), d["rope_theta"])
    kr_raw = W["W_KR"] @ h[-1]
    u = (W["W_UQ"] @ (W["W_DQ"] @ h[-1])).reshape(d["n_heads"], -1)
    for i in range(d["n_heads"]):
        np.testing.assert_allclose(qr[0, i] @ kr[-1], u[i, d["d_head"]:] @ kr_raw, rtol=1e-11)


def test_shared_rope_key_gives_equal_heads_equal_outputs():
    rng = np.random.default_rng(9)
    d = TINY
    W, h = _setup(rng, T=8)
    dh, dr = d["d_head"], d["d_rope"]
    # make head 2 an exact copy of head 0 in every per-head weight
    W["W_UK"][2 * dh:3 * dh] = W["W_UK"][0:dh]
    W["W_UV"][2 * dh:3 * dh] = W["W_UV"][0:dh]
    w = dh + dr
    W["W_UQ"][2 * w:3 * w] = W["W_UQ"][0:w]
    o, lse = oracle.decode_from_h(h, W, d, seqlen=8, s_q=1, tau=0.8)
    np.testing.assert_allclose(o[0, 2], o[0, 0], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse[0, 2], lse[0, 0], rtol=1e-13)


def test_empty_sequence_gives_zero_output_and_neg_inf_lse():
    rng = np.random.default_rng(10)
    W = tiny_weights(rng)
    d = TINY
    qc = rng.normal(size=(3, 8))
    qr = rng.normal(size=(3, 6))
    o, p, lse = oracle.attend_nonabsorbed(qc, qr, np.zeros((0, 12)), np.zeros((0, 6)),
                                          W["W_UK"], W["W_UV"], 8, 1.0)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_cq_input_equals_h_input():
    """W_DQ = None means the caller passes c^Q directly (same result)."""
    rng = np.random.default_rng(11)
    d = TINY
    W, h = _setup(rng, T=6)
    qc1, qr1 = oracle.queries(h[-2:], W["W_DQ"], W["W_UQ"], 3, 8, 6, np.array([4, 5]), 1e4)
    cq = h[-2:] @ W["W_DQ"].T
    qc2, qr2 = oracle.queries(cq, None, W["W_UQ"], 3, 8, 6, np.array([4, 5]), 1e4)
    np.testing.assert_allclose(qc1, qc2, rtol=1e-13)
    np.testing.assert_allclose(qr1, qr2, rtol=1e-13)


def test_head_subset_matches_all_heads():
    rng = np.random.default_rng(12)
    d = TINY
    W, h = _setup(rng, T=11)
    o_all, l_all = oracle.decode_from_h(h, W, d, seqlen=11, s_q=2, tau=0.6)
    o_sub, l_sub = oracle.decode_from_h(h, W, d, seqlen=11, s_q=2, tau=0.6, heads=[2, 0])
    np.testing.assert_allclose(o_sub[:, 0], o_all[:, 2], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(o_sub[:, 1], o_all[:, 0], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(l_sub[:, 1], l_all[:, 0], rtol=1e-13)


@pytest.mark.parametrize("L,chunk", [(4, 4096), (7, 3)])
def test_brute_force_loops_tiny(L, chunk):
    """Scalar-loop evaluation of one (query, head) on a short cache, with the
    key assembled element by element as [k^C; k^R] and every token rotated at
    its absolute position.  With chunk=3 the oracle builds the latents of
    tokens 3.. in later chunks, so a position offset slipped at a chunk
    boundary would fail here."""
    rng = np.random.default_rng(13)
    d = TINY
    W, h = _setup(rng, T=L)
    tau = 0.45
    o, lse = oracle.decode_from_h(h, W, d, seqlen=L, s_q=1, tau=tau, chunk=chunk)
    i = 1
    dh, dr, dc, dm = d["d_head"], d["d_rope"], d["d_c"], d["d_model"]
    import math
    c = [[sum(W["W_DKV"][a][m] * h[t][m] for m in range(dm)) for a in range(dc)] for t in range(L)]
    kraw = [[sum(W["W_KR"][a][m] * h[t][m] for m in range(dm)) for a in range(dr)] for t in range(L)]

    def rot(v, pos):
        out = list(v)
        for mm in range(dr // 2):
            a = pos * 10000.0 ** (-2.0 * mm / dr)
            out[2 * mm] = v[2 * mm] * math.cos(a) - v[2 * mm + 1] * math.sin(a)
            out[2 * mm + 1] = v[2 * mm] * math.sin(a) + v[2 * mm + 1] * math.cos(a)
        return out

    cq = [sum(W["W_DQ"][a][m] * h[L - 1][m] for m in range(dm)) for a in range(d["d_cq"])]
    row0 = i * (dh + dr)
    u = [sum(W["W_UQ"][row0 + a][m] * cq[m] for m in range(d["d_cq"])) for a in range(dh + dr)]
    q = u[:dh] + rot(u[dh:], L - 1)
    scores = []
    for t in range(L):
        key = [sum(W["W_UK"][i * dh + a][m] * c[t][m] for m in range(dc)) for a in range(dh)] + rot(kraw[t], t)
        scores.append(tau * sum(q[a] * key[a] for a in range(dh + dr)))
    mx = max(scores)
    z = sum(math.exp(s - mx) for s in scores)
    out = [sum(math.exp(scores[t] - mx) / z * sum(W["W_UV"][i * dh + a][m] * c[t][m] for m in range(dc))
               for t in range(L)) for a in range(dh)]
    np.testing.assert_allclose(o[0, i], out, rtol=1e-11, atol=1e-13)
    assert abs(lse[0, i] - (mx + math.log(z))) < 1e-12


@pytest.mark.parametrize("chunk", [1, 3, 4, 9])
def test_chunked_latents_equal_one_chunk(chunk):
    """The chunk loop of decode_from_h only bounds memory: any chunk length
    gives the single-chunk result (10 tokens, three causal query rows)."""
    rng = np.random.default_rng(21)
    W, h = _setup(rng, T=10)
    o1, l1 = oracle.decode_from_h(h, W, TINY, seqlen=10, s_q=3, tau=0.8)
    o2, l2 = oracle.decode_from_h(h, W, TINY, seqlen=10, s_q=3, tau=0.8, chunk=chunk)
    assert float(np.max(np.abs(o1 - o2))) <= 1e-12
    assert float(np.max(np.abs(l1 - l2))) <= 1e-12


# ---------------------------------------------------------------- MTP verify model

def test_tokens_per_step_matches_printed_numbers():
    """Depth-1 MTP at 85% and 90% acceptance gives the 1.85 and 1.9 tokens per
    step that the lesson prints (section 2.2, quiz item 5, summary)."""
    g = json.load(open(os.path.join(GOLD, "mtp_tokens_per_step.json")))
    for row in g["printed"]:
        assert abs(oracle.tokens_per_step(row["acceptance"], row["depth"]) - row["tokens_per_step"]) < 1e-12


@pytest.mark.parametrize("depth", [0, 1, 2, 3, 7])
def test_tokens_per_step_limits_and_geometric_series(depth):
    """Acceptance 0: only the main model's token; acceptance 1: every draft
    counts; in between, the k-th draft survives with probability a^k, so the
    mean is the geometric series 1 + a + ... + a^depth."""
    assert oracle.tokens_per_step(0.0, depth) == 1.0
    assert oracle.tokens_per_step(1.0, depth) == 1.0 + depth
    for a in (0.3, 0.85, 0.97):
        series = sum(a ** k for k in range(depth + 1))
        assert abs(oracle.tokens_per_step(a, depth) - series) < 1e-12


def test_tokens_per_step_by_simulation():
    """A Monte Carlo run of the draft chain (accept each draft with
    probability a, stop at the first rejection) agrees within 4 standard
    errors."""
    rng = np.random.default_rng(7)
    a, depth, n = 0.8, 4, 200000
    acc = rng.random((n, depth)) < a
    first_reject = np.where(acc.all(1), depth, np.argmin(acc, 1))
    emitted = 1 + first_reject
    se = emitted.std() / np.sqrt(n)
    assert abs(emitted.mean() - oracle.tokens_per_step(a, depth)) < 4 * se


# ---------------------------------------------------------------- W^O

def test_output_projection_brute_force_and_head_order():
    """y[r][n] = sum over heads i and channels a of W_O[n][i*d_head + a] *
    o[r][i][a], by explicit loops; a W_O that picks one head's block returns
    exactly that head (pins the head-major concatenation); an identity W_O
    (d_model = H * d_head) returns the concatenated heads."""
    rng = np.random.default_rng(11)
    R, H, dh, dm = 3, 4, 5, 7
    o = rng.normal(size=(R, H, dh))
    W = rng.normal(size=(dm, H * dh))
    y = oracle.output_projection(o, W)
    assert y.shape == (R, dm)
    for r in range(R):
        for n in range(dm):
            ref = 0.0
            for i in range(H):
                for a in range(dh):
                    ref += W[n][i * dh + a] * o[r][i][a]
            assert abs(y[r][n] - ref) < 1e-12
    for i in range(H):
        P = np.zeros((dh, H * dh))
        P[:, i * dh:(i + 1) * dh] = np.eye(dh)
        np.testing.assert_array_equal(oracle.output_projection(o, P), o[:, i, :])
    np.testing.assert_array_equal(oracle.output_projection(o, np.eye(H * dh)), o.reshape(R, H * dh))


# ---------------------------------------------------------------- FP8 weight blocks and the block-scaled GEMM

def test_weight_blocks_reduce_to_the_tile_rule():
    """A 128 x 128 block is quantised exactly like one tile holding all of its
    values (the pinned 1 x 128 rule with the tile widened); the short last
    row-block (n = 200: rows 128..199) likewise."""
    rng = np.random.default_rng(3)
    w = rng.normal(0, 0.02, (200, 256))
    codes, scales = oracle.quantize_blocks(w)
    assert codes.shape == (200, 256) and scales.shape == (2, 2)
    for i, (r0, r1) in enumerate(((0, 128), (128, 200))):
        for j in range(2):
            blk = w[r0:r1, 128 * j:128 * (j + 1)]
            c1, s1 = oracle.quantize_tiles(blk.reshape(1, -1), tile=blk.size)
            assert s1[0, 0] == scales[i, j]
            np.testing.assert_array_equal(c1.reshape(blk.shape), codes[r0:r1, 128 * j:128 * (j + 1)])


def test_weight_blocks_scale_error_bound_and_outlier_isolation():
    """amax of every block decodes to +-448 x scale; the dequantised weight is
    within half an E4M3 step (2^-4 relative; 2^-10 x scale absolute near 0);
    a power-of-two factor on one block changes only that block's scale; an
    outlier spoils only its own block (§3.3 item 2)."""
    rng = np.random.default_rng(4)
    w = rng.normal(0, 0.01, (256, 384))
    codes, scales = oracle.quantize_blocks(w)
    deq = oracle.dequantize_blocks(codes, scales)
    s_full = np.repeat(np.repeat(scales.astype(np.float64), 128, 0), 128, 1)
    assert np.all(np.abs(deq - w) <= np.maximum(np.abs(w) * 2.0 ** -4, s_full * 2.0 ** -10) * (1 + 1e-9))
    for i in range(2):
        for j in range(3):
            blk = oracle.e4m3_decode(codes[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)])
            assert np.abs(blk).max() == 448.0
    w2 = w.copy()
    w2[128:256, 0:128] *= 4.0
    c2, s2 = oracle.quantize_blocks(w2)
    np.testing.assert_array_equal(c2, codes)
    assert s2[1, 0] == 4 * scales[1, 0] and np.all(np.delete(s2.ravel(), 3) == np.delete(scales.ravel(), 3))
    w3 = w.copy()
    w3[5, 300] = 50.0
    c3, s3 = oracle.quantize_blocks(w3)
    changed = np.argwhere(s3 != scales)
    assert changed.tolist() == [[0, 2]]
    mask = np.ones_like(codes, dtype=bool)
    mask[0:128, 256:384] = False
    np.testing.assert_array_equal(c3[mask], codes[mask])


def test_block_scaled_gemm_by_promoted_partial_sums():
    """Y by the route of §3.3 item 3 written out: for every 128-wide k-block
    the integer-grid partial sum of code values is scaled by the activation
    tile's and the weight block's scales and promoted into the running sum;
    equals the oracle's dequantise-then-multiply, and stays within the FP8
    error bound of the unquantised product."""
    rng = np.random.default_rng(5)
    m, n, k = 3, 130, 384
    x = rng.normal(0, 1.0, (m, k))
    w = rng.normal(0, 0.02, (n, k))
    wc, ws = oracle.quantize_blocks(w)
    y, xc, xs = oracle.gemm_block_scaled(x, wc, ws)
    xv, wv = oracle.e4m3_decode(xc), oracle.e4m3_decode(wc)
    for r in range(m):
        for c in range(n):
            acc = 0.0
            for kb in range(k // 128):
                part = float(np.dot(xv[r, 128 * kb:128 * (kb + 1)], wv[c, 128 * kb:128 * (kb + 1)]))
                acc += part * float(xs[r, kb]) * float(ws[c // 128, kb])
            assert abs(acc - y[r, c]) <= 1e-12 * max(1.0, abs(acc))
    exact = x @ w.T
    bound = (np.abs(x) @ np.abs(w).T) * (2 * 2.0 ** -4 + 2.0 ** -8) + 1e-6
    assert np.all(np.abs(y - exact) <= bound)


# ---------------------------------------------------------------- decode with FP8 projection weights

FP8W_DIMS = dict(d_model=256, n_heads=2, d_head=128, d_rope=64, d_c=256, d_cq=128, page_size=64, rope_theta=10000.0)


def _fp8w_case(rng, T):
    d = FP8W_DIMS
    H, dh, dr, dc, dq, dm = d["n_heads"], d["d_head"], d["d_rope"], d["d_c"], d["d_cq"], d["d_model"]
    W = {"W_DQ": rng.normal(0, 0.06, (dq, dm)), "W_UQ": rng.normal(0, 0.09, (H * (dh + dr), dq)),
         "W_UK": rng.normal(0, 0.06, (H * dh, dc)), "W_UV": rng.normal(0, 0.06, (H * dh, dc)),
         "W_DKV": rng.normal(0, 0.06, (dc, dm)), "W_KR": rng.normal(0, 0.06, (dr, dm))}
    h = rng.normal(0, 1.0, (T, dm))
    c, kr = oracle.kv_latents(h, W["W_DKV"], W["W_KR"], np.arange(T), d["rope_theta"])
    return d, W, h, c, kr


@pytest.mark.parametrize("T,s_q", [(40, 1), (40, 3), (3, 3)])
def test_fp8w_steps_with_exact_projections_equal_nonabsorbed_decode(T, s_q):
    """The absorbed step sequence of the FP8-weight decode, with exact
    projections, is the non-absorbed decode of §2.1.1 (keys and values built
    per head): every head slice, transpose, RoPE position and scale of its
    plumbing.  T = 3, s_q = 3: the first query row sees one token."""
    d, W, h, c, kr = _fp8w_case(np.random.default_rng(20 + T + s_q), T)
    tau = 1.0 / np.sqrt(d["d_head"] + d["d_rope"])
    hq = h[T - s_q:T]
    o_ref, l_ref = oracle.decode_from_latents(c, kr, hq, W["W_DQ"], W["W_UQ"], W["W_UK"], W["W_UV"], d, T, s_q, tau)
    o, lse = oracle.decode_absorbed_exact(c, kr, hq, W, d, T, s_q, tau)
    assert np.max(np.abs(o - o_ref)) <= 1e-10 * max(1.0, np.max(np.abs(o_ref)))
    fin = np.isfinite(l_ref)
    np.testing.assert_array_equal(np.isfinite(lse), fin)
    assert np.all(np.abs(lse[fin] - l_ref[fin]) <= 1e-10)


def test_fp8w_quantised_steps_stay_within_the_fp8_error():
    """With every projection the block-scaled FP8 GEMM (§3.3 items 2-3), the
    output differs from the exact step sequence (the quantisation is applied)
    by no more than the error of four chained E4M3 GEMMs: each rounds a
    typical operand by 2-4% (3 mantissa bits; a Gaussian block's amax maps to
    448, its typical values to about 100, where the step is 8), and these
    inputs measure 5.8% of the largest output (4-10% over other seeds)."""
    d, W, h, c, kr = _fp8w_case(np.random.default_rng(31), 48)
    tau = 1.0 / np.sqrt(d["d_head"] + d["d_rope"])
    s_q = 2
    hq = h[48 - s_q:48]
    Wq = {k: oracle.quantize_blocks(W[k]) for k in ("W_DQ", "W_UQ", "W_UK", "W_UV")}
    o_q, l_q = oracle.decode_fp8w_from_latents(c, kr, hq, Wq, d, 48, s_q, tau)
    o_e, l_e = oracle.decode_absorbed_exact(c, kr, hq, W, d, 48, s_q, tau)
    err = np.max(np.abs(o_q - o_e)) / np.max(np.abs(o_e))
    assert 1e-3 < err < 0.1, err
    assert np.max(np.abs(l_q - l_e)) < 5e-2


def test_fp8w_uses_each_heads_own_weight_blocks():
    """Scaling head 1's W^UK and W^UV blocks by powers of two (which the
    block quantisation absorbs into the scales exactly) changes only head 1:
    its scores scale by the W^UK factor and its output by the W^UV factor,
    head 0 stays bit-identical.  A wrong head slice or scale row fails."""
    d, W, h, c, kr = _fp8w_case(np.random.default_rng(32), 24)
    tau = 1.0 / np.sqrt(d["d_head"] + d["d_rope"])
    hq = h[23:24]
    dh = d["d_head"]
    Wq = {k: oracle.quantize_blocks(W[k]) for k in ("W_DQ", "W_UQ", "W_UK", "W_UV")}
    o1, l1 = oracle.decode_fp8w_from_latents(c, kr, hq, Wq, d, 24, 1, tau)
    W2 = dict(W)
    W2["W_UK"] = W["W_UK"].copy()
    W2["W_UV"] = W["W_UV"].copy()
    W2["W_UV"][dh:2 * dh] *= 8.0
    Wq2 = dict(Wq)
    Wq2["W_UV"] = oracle.quantize_blocks(W2["W_UV"])
    o2, l2 = oracle.decode_fp8w_from_latents(c, kr, hq, Wq2, d, 24, 1, tau)
    np.testing.assert_array_equal(o2[:, 0], o1[:, 0])
    np.testing.assert_array_equal(l2, l1)
    assert np.max(np.abs(o2[:, 1] - 8.0 * o1[:, 1])) <= 1e-12 * np.max(np.abs(o1[:, 1])) * 8
    # W^UK of head 1 doubled: the content scores of head 1 double, head 0 is unchanged
    W2["W_UK"][dh:2 * dh] *= 2.0
    Wq3 = dict(Wq)
    Wq3["W_UK"] = oracle.quantize_blocks(W2["W_UK"])
    o3, l3 = oracle.decode_fp8w_from_latents(c, kr, hq, Wq3, d, 24, 1, tau)
    np.testing.assert_array_equal(o3[:, 0], o1[:, 0])
    assert np.max(np.abs(o3[:, 1] - o1[:, 1])) > 1e-6


def test_bf16_round_ties_and_independent_conversion():
    """Round to nearest bf16, ties to an even mantissa: 1 + 2^-8 lies halfway
    between 1 and 1 + 2^-7 and goes to 1; 1 + 3 2^-8 lies halfway between
    1 + 2^-7 (odd) and 1 + 2^-6 (even) and goes up; anything above a tie
    rounds up; the sign is kept; and on random values it agrees with torch's
    own float32 -> bfloat16 conversion."""
    import torch
    r = oracle.bf16_round
    assert r(1.0 + 2.0 ** -8) == 1.0
    assert r(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert r(1.0 + 2.0 ** -8 + 2.0 ** -20) == 1.0 + 2.0 ** -7
    assert r(-(1.0 + 3 * 2.0 ** -8)) == -(1.0 + 2.0 ** -6)
    assert r(0.0) == 0.0 and r(2.0 ** -130) == r(2.0 ** -130)
    x = np.random.default_rng(7).normal(0, 3.0, 10000)
    t = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(r(x), t)
