"""GPU parity at DeepSeek-V3 shapes (hidden 7168, 128 heads of 128, RoPE 64,
d_c 512, d_c' 1536, weights N(0, 0.006^2)) on small batches the oracle
finishes in seconds: ragged lengths spanning several pages and a partial last
page, shuffled block tables, several split counts, bf16 and fp8 caches.
Tolerance: max|delta| <= 2e-2 * max|ref| (bf16), 5e-2 * max|ref| (fp8 cache),
max|ref| over the whole compared tensor."""
import os

import numpy as np
import pytest
import torch

from mla_latent_kv_29_amd import inputs
from gpu_common import Case, tau_of, max_abs, to_np, DEV

pytestmark = pytest.mark.gpu
V3 = inputs.V3_DIMS
TOL_BF16 = 2e-2


def check_all(case, out, lse, tau, tol_rel, heads=None, fp8=False):
    for b, Lb in enumerate(case.lengths):
        if Lb == 0:
            assert np.all(out[b] == 0) and np.all(np.isneginf(lse[b]))
            continue
        o, l = case.oracle(b, tau, heads=heads, fp8=fp8)
        got = out[b] if heads is None else out[b][:, heads]
        gl = lse[b] if heads is None else lse[b][:, heads]
        ref = float(np.abs(o).max())
        err = max_abs(got, o)
        assert err <= tol_rel * ref, (b, int(Lb), err, ref)
        assert max_abs(gl, l) <= tol_rel * max(1.0, float(np.abs(l).max()))


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("kappa", [1.0, 56.0])
def test_v3_bf16_ragged(splits, kappa):
    case = Case(V3, "bf16", "bf16", [300, 1, 129, 64], s_q=1, table="shuffled", wl=1, num_splits=splits)
    tau = tau_of(V3) * kappa
    out, lse, _ = case.run(tau)
    check_all(case, out, lse, tau, TOL_BF16)


@pytest.mark.parametrize("cache", ["bf16", "fp8", "fp8e8"])
def test_v3_bf16_fast_matches_generic(cache):
    """The MFMA path and the generic VALU path agree (same inputs, the same
    cache bytes: the generic path dequantises FP8 codes in fp32)."""
    case = Case(V3, "bf16", cache, [200, 77], s_q=1, table="shuffled", wl=1, num_splits=2)
    tau = tau_of(V3) * 30.0
    fast, lfast, _ = case.run(tau)
    os.environ["MLA_FORCE_GENERIC"] = "1"
    try:
        gen, lgen, _ = case.run(tau)
    finally:
        del os.environ["MLA_FORCE_GENERIC"]
    assert max_abs(fast, gen) <= 1e-2 * float(np.abs(gen).max())
    assert max_abs(lfast, lgen) <= 1e-2 * float(np.abs(lgen).max())


@pytest.mark.parametrize("s_q", [2])
def test_v3_bf16_causal_two_queries(s_q):
    case = Case(V3, "bf16", "bf16", [200, 65, 2], s_q=s_q, table="shuffled", wl=4, num_splits=2)
    tau = tau_of(V3) * 56.0
    out, lse, _ = case.run(tau)
    check_all(case, out, lse, tau, TOL_BF16)


@pytest.mark.parametrize("s_q", [3, 4, 8])
def test_v3_bf16_deeper_mtp_verify(s_q):
    """Verify of s_q - 1 chained drafts: s_q causal query rows per sequence.
    The last sequence holds exactly s_q tokens, so its first query sees one."""
    case = Case(V3, "bf16", "bf16", [200, 65, s_q], s_q=s_q, table="shuffled", wl=6, num_splits=2)
    tau = tau_of(V3) * 56.0
    out, lse, _ = case.run(tau)
    check_all(case, out, lse, tau, TOL_BF16)


def test_v3_bf16_verify_more_than_64_rows():
    """9 sequences x 8 query rows = 72 rows: the query projection and the
    combine take their many-row kernels; default split plan."""
    lengths = [70 + 37 * i for i in range(9)]
    case = Case(V3, "bf16", "bf16", lengths, s_q=8, table="shuffled", wl=6)
    tau = tau_of(V3) * 20.0
    out, lse, _ = case.run(tau)
    check_all(case, out, lse, tau, TOL_BF16, heads=[0, 63, 127])


@pytest.mark.parametrize("lengths,s_q", [([65] + [40 + i for i in range(64)], 1),
                                         ([5 + 3 * i for i in range(43)], 3),
                                         ([4 + i for i in range(100)], 3)])
def test_v3_bf16_many_row_query_block_edges(lengths, s_q):
    """The many-row query kernel (128 rows a block) at 65 rows (one block,
    63 clamped rows), 129 rows (a second block with one row) and 300 rows
    (three blocks, the last partly filled); ragged lengths, default plan."""
    case = Case(V3, "bf16", "bf16", lengths, s_q=s_q, table="shuffled", wl=8)
    tau = tau_of(V3) * 20.0
    out, lse, _ = case.run(tau)
    check_all(case, out, lse, tau, TOL_BF16, heads=[0, 63, 127])


def test_v3_planted_latents_sharp():
    """Cache written directly (std 0.5, the scale of W^DKV h at these
    weights), queries from h; sharpened softmax."""
    case = Case(V3, "bf16", "bf16", [257, 64, 31], s_q=1, table="shuffled", wl=1, num_splits=2,
                planted=(0.5, 0.5))
    tau = tau_of(V3) * 56.0
    out, lse, hq = case.run(tau)
    for b in range(3):
        o, l = case.oracle(b, tau, hq=hq)
        assert max_abs(out[b], o) <= TOL_BF16 * float(np.abs(o).max())


@pytest.mark.parametrize("cache", ["bf16", "fp8", "fp8e8"])
def test_v3_score_far_above_first_stage_max(cache):
    """A token in a later pipeline stage whose score exceeds the first
    stage's maximum by ~2^150 (log2 units): the kernel must redo the item
    against the exact maximum and still match the oracle (for the FP8
    caches, the oracle on the same quantised latents)."""
    import oracle
    from gpu_common import to_np
    case = Case(V3, "bf16", cache, [300], s_q=1, table="shuffled", wl=1, num_splits=1, planted=(0.05, 0.05))
    tau = tau_of(V3)
    hq = case.hq()
    Wn = case.weights_np()
    qc, qr = oracle.queries(to_np(hq), Wn["W_DQ"], Wn["W_UQ"], 128, 128, 64, np.array([299]), 1e4)
    q_abs = Wn["W_UK"][0:128].T @ qc[0, 0]
    star = 200
    c, r = case.lat[0]
    c = c.clone()
    c[star] = torch.from_numpy(q_abs / np.linalg.norm(q_abs) * (100.0 / tau / np.linalg.norm(q_abs))).to(c)
    case.lat[0] = (c, r)
    case.sess.write(c[star:star + 1].contiguous(), r[star:star + 1].contiguous(), 0, star)
    torch.cuda.synchronize()
    out, lse, _ = case.run(tau)
    o, l = case.oracle(0, tau, hq=hq, fp8=cache != "bf16")
    assert max_abs(out[0], o) <= TOL_BF16 * float(np.abs(o).max())
    assert abs(lse[0, 0, 0] - l[0, 0]) <= 1e-2 * abs(l[0, 0])


@pytest.mark.parametrize("splits", [1, 2])
def test_v3_bf16_bytes_past_the_end_are_ignored(splits):
    """Page slots past a sequence's length hold NaN bf16 patterns (0xFFFF):
    the tokens they would be are not visible, so the output must not change."""
    from gpu_common import bf16_page_off
    case = Case(V3, "bf16", "bf16", [300, 129, 64], s_q=1, table="shuffled", wl=1, num_splits=splits)
    ps, D = V3["page_size"], V3["d_c"] + V3["d_rope"]
    t = np.arange(ps)[:, None]
    ch = np.arange(D)[None, :]
    raw = case.sess.pages.cpu().numpy()
    for b, Lb in enumerate(case.lengths):
        last = int(case.bt[b, (int(Lb) - 1) // ps])
        tail = t[int(Lb) % ps:] if Lb % ps else t[:0]
        off = bf16_page_off(tail, ch, ps)
        raw[last, off.ravel()] = 0xFF
        raw[last, off.ravel() + 1] = 0xFF
    case.sess.pages.copy_(torch.from_numpy(raw))
    torch.cuda.synchronize()
    tau = tau_of(V3) * 56.0
    out, lse, _ = case.run(tau)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    check_all(case, out, lse, tau, TOL_BF16)


@pytest.mark.parametrize("s_q", [1, 2])
def test_v3_bf16_compressed_query_input(s_q):
    """W_DQ = NULL: the caller passes c^Q = W^DQ h (here the float64 oracle's,
    rounded to bf16) instead of h; the output matches the oracle decoded
    from h."""
    case = Case(V3, "bf16", "bf16", [300, 129, 70], s_q=s_q, table="shuffled", wl=1, num_splits=2)
    tau = tau_of(V3)
    Wn = case.weights_np()
    hq = case.hq()
    cq = torch.from_numpy(to_np(hq) @ Wn["W_DQ"].T).to(torch.bfloat16).to(DEV).contiguous()
    out, lse = case.sess.decode(cq, case.W, tau, use_dq=False)
    torch.cuda.synchronize()
    out, lse = to_np(out), to_np(lse)
    for b in range(3):
        o, l = case.oracle(b, tau)
        assert max_abs(out[b], o) <= TOL_BF16 * float(np.abs(o).max()), b
        assert max_abs(lse[b], l) <= TOL_BF16 * max(1.0, float(np.abs(l).max())), b


def test_v3_bf16_many_rows_two_row_blocks():
    """48 query rows (24 sequences x 2 queries): the combine's second row block
    is partly empty and each wave merges several rows; ragged lengths down to
    two tokens (the two new ones) and three splits."""
    lengths = [2, 2, 65, 300, 129, 64, 17, 200, 33, 250, 80, 5, 140, 96, 63, 190, 7, 111, 222, 40, 66, 130, 3, 280]
    case = Case(V3, "bf16", "bf16", lengths, s_q=2, table="shuffled", wl=1, num_splits=3)
    tau = tau_of(V3)
    out, lse, _ = case.run(tau)
    check_all(case, out, lse, tau, TOL_BF16, heads=[0, 77, 127])


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_decode_halves_equal_the_whole_call(cache):
    """mla_decode_query then mla_decode_attend (the benchmark's timed halves),
    then mla_combine, give exactly what mla_decode + mla_combine give."""
    from mla_latent_kv_29_amd import _lib as L
    case = Case(V3, "bf16", cache, [200, 65, 3], s_q=2, table="shuffled", wl=4, num_splits=2)
    tau = tau_of(V3) * 20.0
    hq = case.hq()
    s = case.sess
    W = case.W
    s.decode(hq, W, tau)
    torch.cuda.synchronize()
    whole = (s.out.clone(), s.lse.clone())
    s.out.fill_(float("nan"))
    s.lse.fill_(float("nan"))
    args = (s.cdims, s.act, hq, s.batch, s.s_q, W["W_DQ"], W["W_UQ"], W["W_UK"], s.cache, s.block_table,
            s.max_pages, s.seqlens, tau, s.num_splits, s.ws, s.ws_bytes, None)
    L.mla_decode_query(*args)
    L.mla_decode_attend(*args)
    L.mla_combine(s.cdims, s.act, s.batch, s.s_q, s.num_splits, s.ws, s.ws_bytes, W["W_UV"], s.out, s.lse, None)
    torch.cuda.synchronize()
    assert torch.equal(whole[0], s.out) and torch.equal(whole[1], s.lse)


def test_v3_sequence_is_independent_of_its_batch_mates():
    """Sequence 0 (same seed, same length) decoded beside different batch-mates
    and at a different place in the page pool gives the same bits: no row of
    the query projections, attention items or merge reads another sequence."""
    tau = tau_of(V3) * 20.0
    outs = []
    for lengths, table in (([300, 129, 64], "inorder"), ([300, 7], "shuffled"), ([300], "inorder")):
        case = Case(V3, "bf16", "bf16", lengths, s_q=2, table=table, wl=1, num_splits=3)
        out, lse, _ = case.run(tau)
        outs.append((out[0], lse[0]))
    for o, l in outs[1:]:
        assert np.array_equal(o, outs[0][0]) and np.array_equal(l, outs[0][1])


def test_v3_split_counts_agree_with_each_other():
    """The same batch with 1, 2, 3 and 7 splits per sequence: each split count
    is an exact rewrite of the softmax, so the outputs agree far more closely
    than either agrees with the float64 oracle (1e-2 max|o|, against 2e-2)."""
    case = Case(V3, "bf16", "bf16", [300, 129, 448, 64], s_q=1, table="shuffled", wl=1, num_splits=1)
    tau = tau_of(V3) * 30.0
    ref, lref, _ = case.run(tau, num_splits=1)
    for splits in (2, 3, 7):
        out, lse, _ = case.run(tau, num_splits=splits)
        assert case.sess.num_splits == splits
        assert max_abs(out, ref) <= 1e-2 * float(np.abs(ref).max()), splits
        assert max_abs(lse, lref) <= 1e-4 * float(np.abs(lref).max()), splits


def test_v3_empty_sequence_in_a_batch():
    """A sequence of length 0 beside others, through the MFMA query, attention
    and merge kernels: its output is 0 and its lse -inf; the others match the
    oracle."""
    case = Case(V3, "bf16", "bf16", [200, 0, 65], s_q=1, table="shuffled", wl=1, num_splits=2)
    tau = tau_of(V3) * 10.0
    out, lse, _ = case.run(tau)
    check_all(case, out, lse, tau, TOL_BF16)


@pytest.mark.parametrize("lengths,s_q", [([70 + 37 * i for i in range(9)], 8), ([300, 65, 9], 1)])
def test_attend_and_combine_rerun_on_the_same_workspace(lengths, s_q):
    """query, attend, combine, then attend and combine again on the same
    workspace give identical bytes: the combine writes only its own region
    (the merged latent rows), never the queries the attention reads.  72 rows
    (the many-row combine) and 3 rows (the fused one)."""
    from mla_latent_kv_29_amd import _lib as L
    case = Case(V3, "bf16", "bf16", lengths, s_q=s_q, table="shuffled", wl=6)
    sess = case.sess
    hq = case.hq()
    tau = tau_of(V3)
    W = case.W
    args = (sess.cdims, sess.act, hq, sess.batch, s_q, W["W_DQ"], W["W_UQ"], W["W_UK"], sess.cache,
            sess.block_table, sess.max_pages, sess.seqlens, tau, sess.num_splits, sess.ws, sess.ws_bytes)
    comb = lambda: L.mla_combine(sess.cdims, sess.act, sess.batch, s_q, sess.num_splits, sess.ws, sess.ws_bytes,
                                 W["W_UV"], sess.out, sess.lse)
    L.mla_decode_query(*args)
    L.mla_decode_attend(*args)
    comb()
    o1, l1 = sess.out.clone(), sess.lse.clone()
    L.mla_decode_attend(*args)
    comb()
    torch.cuda.synchronize()
    assert torch.equal(sess.out, o1) and torch.equal(sess.lse, l1)
