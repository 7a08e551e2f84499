"""The decode step replayed from a captured HIP graph (torch.cuda.CUDAGraph
over the C ABI calls): the library enqueues only kernels on the caller's
stream (no allocation, memset or copy), so a captured step must give the
eager step's bytes on every replay.  Each test replays three times with
other eager library work and a synchronisation between the replays."""
import numpy as np
import pytest
import torch

from mla_latent_kv_29_amd import inputs
from mla_latent_kv_29_amd.session import DecodeSession
from gpu_common import DEV, tau_of

pytestmark = pytest.mark.gpu
V3 = inputs.V3_DIMS


def make_session(lengths, s_q, seed, cache="bf16"):
    lengths = np.asarray(lengths, dtype=np.int64)
    W = inputs.weights(V3, 0.006, torch.bfloat16, DEV, seed, 12)
    bt, pool = inputs.block_table(lengths, V3["page_size"], "shuffled", seed, 12)
    sess = DecodeSession(V3, "bf16", cache, lengths, bt, pool, s_q, 0, DEV)
    gen_h = lambda b, t0, t1: inputs.hidden(V3, b, t0, t1, torch.bfloat16, DEV, seed, 12)
    sess.build_from_h(gen_h, W)
    hq = torch.cat([gen_h(b, int(L) - s_q, int(L)) for b, L in enumerate(lengths)], 0).contiguous()
    return sess, W, hq


def replay_and_check(sess, run, other):
    """run(): one step into sess.out / sess.lse; other(): unrelated eager work."""
    run()
    torch.cuda.synchronize()
    ref_o, ref_l = sess.out.clone(), sess.lse.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for _ in range(3):
        sess.out.zero_()
        sess.lse.zero_()
        other()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(sess.out, ref_o) and torch.equal(sess.lse, ref_l)


@pytest.mark.parametrize("lengths,s_q", [([300, 65, 1, 1000], 1), ([70 + 37 * i for i in range(9)], 8)])
def test_bf16_decode_step_from_a_graph(lengths, s_q):
    """4 rows (the skinny query and the fused combine) and 72 rows (the
    many-row query kernel and the combine's row groups)."""
    sess, W, hq = make_session(lengths, s_q, 3)
    other_sess, W2, hq2 = make_session([200, 33], 1, 4)
    tau = tau_of(V3)
    replay_and_check(sess, lambda: sess.decode(hq, W, tau), lambda: other_sess.decode(hq2, W2, tau))


def test_fp8w_decode_step_from_a_graph():
    """The FP8-weight step (fused W^UQ + absorption, fused merge + W^UV)."""
    sess, W, hq = make_session([300, 65, 1, 1000], 1, 5)
    Wq = sess.quantize_fp8w(W)
    other_sess, W2, hq2 = make_session([200, 33], 1, 6)
    tau = tau_of(V3)
    sess.fp8w_workspace()
    replay_and_check(sess, lambda: sess.decode_fp8w(hq, Wq, tau), lambda: other_sess.decode(hq2, W2, tau))


@pytest.mark.parametrize("cache", ["fp8", "fp8e8"])
def test_fp8_cache_decode_step_from_a_graph(cache):
    """Both FP8 cache formats (the two-barrier and the one-barrier attention)
    at 2 query rows a sequence."""
    sess, W, hq = make_session([300, 65, 2, 1000], 2, 7, cache)
    other_sess, W2, hq2 = make_session([200, 33], 1, 8)
    tau = tau_of(V3)
    replay_and_check(sess, lambda: sess.decode(hq, W, tau), lambda: other_sess.decode(hq2, W2, tau))
