"""Absorbed decode with FP8 block-scaled projection weights, float64 --
TEST INFRASTRUCTURE ONLY.

Sources: "Читаем техотчёт DeepSeek-V3 вместе", §2.1.1 (the latent-KV
equations and Question 2: W^UK folded into the query, W^UV applied after the
softmax-weighted sum of latents) and §3.3 "Обучение в FP8", items 2-4 (each
GEMM on E4M3 inputs: weights in 128 x 128 blocks, activations in 1 x 128
tiles, one scale per group, products summed in high precision).

Reading (stated because the pages describe FP8 for training GEMMs, not for
a decode step): the scheme applies to the four projections of the absorbed
decode step exactly as the step executes them, each as Y = Q(X) Q(W)^T:
    c^Q = W^DQ h,   u = W^UQ c^Q = [q^C_i ; q^R_i],
    q_abs_i = W^UK_i^T q^C_i  (X = q^C_i, the weight W^UK_i^T [d_c, d_head]),
    out_i = W^UV_i O_lat_i     (X = O_lat_i).
The cached latents, the scores and the softmax stay in float64 (the
attention is not an FP8 GEMM on the pages).  Each GEMM's activation input
is taken as a stored bf16 tensor, the storage of the decode step between
its kernels: h is bf16 already, and c^Q, u and O_lat are rounded to bf16
(round to nearest, ties to even) before they are tile-quantised, so that the
codes are decided from the same values the device quantises.  The 128 x 128 blocks of
W^UK_i^T are the transposes of W^UK's own blocks (d_head = 128), so W^UK is
quantised once in its stored orientation [H * d_head, d_c].

Parity: pinned in tests/test_oracle_pins.py by (a) the same step sequence
with exact projections equalling the non-absorbed decode of mla.py to 1e-10
(every transpose, head slice, RoPE position and scale of the plumbing),
(b) the quantised step staying within the FP8 error of the exact one on
random inputs while differing from it (the quantisation is really applied),
(c) each head using only its own weight blocks, and (d) bf16_round against
worked ties and an independent bf16 conversion.
"""
import numpy as np

from .fp8 import gemm_block_scaled
from .mla import rope, softmax_lse


def bf16_round(x):
    """x rounded to the nearest bf16 value (8 exponent bits, 7 stored mantissa
    bits; ties to an even mantissa), via float32: the low 16 bits of the
    float32 pattern are rounded off.  Returned as float64."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    keep = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + keep) >> np.uint64(16)) << np.uint64(16)
    out = (r & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(np.float32).astype(np.float64)
    return np.where(np.isfinite(f), out, f.astype(np.float64))


def _absorbed_steps(c, kr, hq, dims, seqlen, s_q, tau, heads, dq, uq, uk, uv, store=lambda x: x):
    """The absorbed decode of s_q query rows of one sequence with the four
    projections given as functions: dq(x), uq(x), uk(x, i), uv(x, i), each
    mapping rows x [r, k] to [r, n]; store(x) is applied to c^Q, u and O_lat
    (the stored form of an intermediate)."""
    H, dh, dr = dims["n_heads"], dims["d_head"], dims["d_rope"]
    c = np.asarray(c, dtype=np.float64)
    kr = np.asarray(kr, dtype=np.float64)
    d_c = c.shape[1]
    heads = list(range(H)) if heads is None else list(heads)
    pos_q = np.arange(seqlen - s_q, seqlen)
    cq = store(dq(np.asarray(hq, dtype=np.float64)))
    u = store(uq(cq)).reshape(s_q, H, dh + dr)
    qc = u[:, :, :dh]
    qr = rope(u[:, :, dh:], pos_q[:, None], dims["rope_theta"])
    o = np.zeros((s_q, len(heads), dh))
    lse = np.zeros((s_q, len(heads)))
    for j in range(s_q):
        vis = max(0, seqlen - s_q + j + 1)
        for n, i in enumerate(heads):
            q_abs = uk(qc[j, i][None, :], i)[0]                     # [d_c]
            s = tau * (c[:vis] @ q_abs + kr[:vis] @ qr[j, i])
            p, lse[j, n] = softmax_lse(s)
            o_lat = store(p @ c[:vis]) if vis > 0 else np.zeros(d_c)
            o[j, n] = uv(o_lat[None, :], i)[0]
    return o, lse


def decode_absorbed_exact(c, kr, hq, W, dims, seqlen, s_q, tau, heads=None):
    """The step sequence above with exact float64 projections of the given
    weights (W: dict of W_DQ [d_cq, d_model], W_UQ [H(d_head + d_rope), d_cq],
    W_UK, W_UV [H d_head, d_c]).  Returns o [s_q, h, d_head], lse [s_q, h]."""
    dh = dims["d_head"]
    Wd = {k: np.asarray(W[k], dtype=np.float64) for k in ("W_DQ", "W_UQ", "W_UK", "W_UV")}
    return _absorbed_steps(
        c, kr, hq, dims, seqlen, s_q, tau, heads,
        dq=lambda x: x @ Wd["W_DQ"].T,
        uq=lambda x: x @ Wd["W_UQ"].T,
        uk=lambda x, i: x @ Wd["W_UK"][i * dh:(i + 1) * dh],
        uv=lambda x, i: x @ Wd["W_UV"][i * dh:(i + 1) * dh].T)


def decode_fp8w_from_latents(c, kr, hq, Wq, dims, seqlen, s_q, tau, heads=None):
    """The step sequence with every projection the block-scaled FP8 GEMM of
    fp8.gemm_block_scaled, its bf16-stored intermediates rounded as stated
    above.  Wq: dict of (codes, scales) from
    fp8.quantize_blocks for W_DQ, W_UQ, W_UK (stored [H d_head, d_c]) and
    W_UV.  Requires d_head == 128 (one block row of W^UK and W^UV per head).
    Returns o [s_q, h, d_head], lse [s_q, h]."""
    dh = dims["d_head"]
    assert dh == 128
    ukc, uks = Wq["W_UK"]
    uvc, uvs = Wq["W_UV"]
    return _absorbed_steps(
        c, kr, hq, dims, seqlen, s_q, tau, heads,
        dq=lambda x: gemm_block_scaled(x, *Wq["W_DQ"])[0],
        uq=lambda x: gemm_block_scaled(x, *Wq["W_UQ"])[0],
        uk=lambda x, i: gemm_block_scaled(x, ukc[i * dh:(i + 1) * dh].T, uks[i:i + 1].T)[0],
        uv=lambda x, i: gemm_block_scaled(x, uvc[i * dh:(i + 1) * dh], uvs[i:i + 1])[0],
        store=bf16_round)
