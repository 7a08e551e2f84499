"""Parity of the causal prefill (mla_prefill) with the float64 oracle.

The oracle's decode of a sequence with s_q equal to its length is exactly the
prefill of that sequence: every token is a query at its own position and sees
tokens 0..j, with explicit per-head k^C = W^UK c^KV and v^C = W^UV c^KV (the
non-absorbed form).  Inputs are the seeded hidden states and weights of the
decode tests, sequences packed back to back.
"""
import numpy as np
import pytest
import torch

import oracle
import mla_latent_kv_29_amd as m
from mla_latent_kv_29_amd import inputs
from gpu_common import DEV, tau_of, to_np, max_abs

pytestmark = pytest.mark.gpu

V3 = inputs.V3_DIMS
TOL_BF16 = 2e-2
HEADS = [0, 57, 127]


def run_prefill(lengths, kappa, seed=0, wl=3, sigma=0.006, lse=True):
    dims = V3
    W = inputs.weights(dims, sigma, torch.bfloat16, DEV, seed, wl)
    hs = [inputs.hidden(dims, b, 0, int(L), torch.bfloat16, DEV, seed, wl) for b, L in enumerate(lengths)]
    h = torch.cat(hs, 0).contiguous()
    n = h.shape[0]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device=DEV)
    d = m.make_dims(dims)
    wsb = m.mla_prefill_workspace_bytes(d, m.MLA_BF16, n)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    out = torch.full((n, dims["n_heads"], dims["d_head"]), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse_t = torch.full((n, dims["n_heads"]), float("nan"), dtype=torch.float32, device=DEV) if lse else None
    tau = kappa * tau_of(dims)
    m.mla_prefill(d, m.MLA_BF16, h, n, len(lengths), cu, int(max(lengths)), W["W_DQ"], W["W_UQ"], W["W_UK"],
                  W["W_UV"], W["W_DKV"], W["W_KR"], tau, out, lse_t, ws, wsb)
    torch.cuda.synchronize()
    return dims, W, hs, to_np(out), (to_np(lse_t) if lse else None), tau


def check(lengths, kappa, heads=HEADS):
    dims, W, hs, out, lse, tau = run_prefill(lengths, kappa)
    Wn = {k: to_np(v) for k, v in W.items()}
    row = 0
    for b, L in enumerate(lengths):
        L = int(L)
        o_ref, l_ref = oracle.decode_from_h(to_np(hs[b]), Wn, dims, L, L, tau, heads)
        got = out[row:row + L][:, heads]
        ref = float(np.max(np.abs(o_ref)))
        err = max_abs(got, o_ref)
        assert err <= TOL_BF16 * ref, (b, L, kappa, err, ref)
        gl = lse[row:row + L][:, heads]
        assert max_abs(gl, l_ref) <= TOL_BF16 * max(1.0, float(np.max(np.abs(l_ref)))), (b, L, kappa)
        row += L
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))


@pytest.mark.parametrize("kappa", [1.0, 56.0])
def test_prefill_ragged_sequences(kappa):
    """One token, exactly one tile, three tiles with a ragged tail, one tile plus one."""
    check([1, 64, 190, 65], kappa)


def test_prefill_long_sequence_streams_many_key_tiles():
    """640 tokens: ten query tiles, the last of which streams ten key tiles
    through the two LDS buffers; plus a short neighbour."""
    check([640, 3], 1.0)


def test_prefill_rows_past_the_end_are_not_written():
    """Query rows of a block beyond its sequence are computed on clamped rows
    and never stored: the next sequence's rows come out right (covered above),
    and no output row is left unwritten (no NaN survives the fill)."""
    dims, W, hs, out, lse, tau = run_prefill([5, 70, 1], 1.0)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))


def test_prefill_halves_equal_the_whole_call():
    """mla_prefill_project then mla_prefill_attend (the benchmark's two timed
    halves) give exactly what mla_prefill gives, on ragged sequences that take
    the 256 x 256 projections (300 tokens) and the 64 x 64 ones (40)."""
    for lengths in ([130, 7, 163], [33, 7]):
        dims = V3
        W = inputs.weights(dims, 0.006, torch.bfloat16, DEV, 0, 3)
        h = torch.cat([inputs.hidden(dims, b, 0, int(L), torch.bfloat16, DEV, 0, 3) for b, L in enumerate(lengths)],
                      0).contiguous()
        n = h.shape[0]
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device=DEV)
        d = m.make_dims(dims)
        wsb = m.mla_prefill_workspace_bytes(d, m.MLA_BF16, n)
        outs = []
        for split in (False, True):
            ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
            out = torch.full((n, dims["n_heads"], dims["d_head"]), float("nan"), dtype=torch.bfloat16, device=DEV)
            lse = torch.full((n, dims["n_heads"]), float("nan"), dtype=torch.float32, device=DEV)
            args = (d, m.MLA_BF16, h, n, len(lengths), cu, int(max(lengths)), W["W_DQ"], W["W_UQ"], W["W_UK"],
                    W["W_UV"], W["W_DKV"], W["W_KR"], tau_of(dims), out, lse, ws, wsb)
            if split:
                m.mla_prefill_project(*args)
                m.mla_prefill_attend(*args)
            else:
                m.mla_prefill(*args)
            torch.cuda.synchronize()
            outs.append((out.clone(), lse.clone()))
        assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1]), lengths
        assert bool(torch.isfinite(outs[0][0].float()).all())


@pytest.mark.parametrize("kappa", [1.0, 56.0])
def test_prefill_benchmark_shape_sampled_rows(kappa):
    """The benchmarked prefill: 4 sequences x 4096 tokens packed (the bench's
    seeds and launch), so every query tile, the XCD placement of all 16384
    work items and the 256 x 256 projection epilogues run at full size.  Row
    j of a sequence is the oracle's decode with one query row and seqlen
    j + 1; rows 0, 127, 128, 2047 and 4095 of the first and the last
    sequence, three heads."""
    spec = inputs.PREFILL_WORKLOADS["prefill_v3_bf16_b4_l4096"]
    dims, wl = spec["dims"], spec["index"]
    lengths = inputs.seqlens(spec["lengths"], spec["batch"], 0, wl)
    W = inputs.weights(dims, spec["sigma"], torch.bfloat16, DEV, 0, wl)
    hs = [inputs.hidden(dims, b, 0, int(L), torch.bfloat16, DEV, 0, wl) for b, L in enumerate(lengths)]
    h = torch.cat(hs, 0).contiguous()
    n = h.shape[0]
    cu_np = np.concatenate([[0], np.cumsum(lengths)])
    cu = torch.tensor(cu_np, dtype=torch.int32, device=DEV)
    d = m.make_dims(dims)
    wsb = m.mla_prefill_workspace_bytes(d, m.MLA_BF16, n)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    out = torch.full((n, dims["n_heads"], dims["d_head"]), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((n, dims["n_heads"]), float("nan"), dtype=torch.float32, device=DEV)
    tau = kappa * tau_of(dims)
    args = (d, m.MLA_BF16, h, n, len(lengths), cu, int(max(lengths)), W["W_DQ"], W["W_UQ"], W["W_UK"], W["W_UV"],
            W["W_DKV"], W["W_KR"], tau, out, lse, ws, wsb)
    m.mla_prefill_project(*args)
    m.mla_prefill_attend(*args)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out.float()).all()) and bool(torch.isfinite(lse).all())
    Wn = {k: to_np(v) for k, v in W.items()}
    rows = [0, 127, 128, 2047, 4095]
    for b in (0, len(lengths) - 1):
        hb = to_np(hs[b])
        c, kr = oracle.kv_latents(hb, Wn["W_DKV"], Wn["W_KR"], np.arange(hb.shape[0]), dims["rope_theta"])
        for j in rows:
            o_ref, l_ref = oracle.decode_from_latents(c[:j + 1], kr[:j + 1], hb[j:j + 1], Wn["W_DQ"], Wn["W_UQ"],
                                                      Wn["W_UK"], Wn["W_UV"], dims, j + 1, 1, tau, HEADS)
            g = int(cu_np[b]) + j
            got = to_np(out[g, HEADS])
            got_l = to_np(lse[g, HEADS])
            ref = float(np.max(np.abs(o_ref)))
            assert max_abs(got, o_ref[0]) <= TOL_BF16 * ref, (b, j, kappa)
            assert max_abs(got_l, l_ref[0]) <= TOL_BF16 * max(1.0, float(np.max(np.abs(l_ref)))), (b, j, kappa)
