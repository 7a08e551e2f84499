"""The allocation-free decode step (mla_decode_step_noalloc) against the two
entry points it stands for (mla_decode + mla_combine with a caller
workspace), through the C ABI on the GPU: the same kernels on the same
inputs, so the outputs and lse must agree bit for bit (stricter than the
bf16 tolerance of the oracle comparisons).  Two calls in a row, the second
with a smaller batch, so the second call reuses the array the first one left
behind."""
import numpy as np
import pytest
import torch

from mla_latent_kv_29_amd import inputs
from mla_latent_kv_29_amd import _lib as L
from gpu_common import Case, tau_of

pytestmark = pytest.mark.gpu
V3 = inputs.V3_DIMS


def noalloc_outputs(case, tau):
    s = case.sess
    hq = case.hq()
    out = torch.full_like(s.out, float("nan"))
    lse = torch.full_like(s.lse, float("nan"))
    L.mla_decode_step_noalloc(s.cdims, s.act, hq, s.batch, s.s_q, case.W["W_DQ"], case.W["W_UQ"], case.W["W_UK"],
                              case.W["W_UV"], s.cache, s.block_table, s.max_pages, s.seqlens, tau, s.num_splits,
                              out, lse)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("cache", ["bf16", "fp8", "fp8e8"])
def test_noalloc_decode_step_equals_decode_and_combine(cache):
    tau = tau_of(V3) * 20.0
    cases = [Case(V3, "bf16", cache, [1024] * 48 + [700, 3, 0, 65], s_q=1, table="shuffled", wl=1, num_splits=0),
             Case(V3, "bf16", cache, [300, 129, 64], s_q=2, table="inorder", wl=4, num_splits=3)]
    for case in cases:
        out_n, lse_n = noalloc_outputs(case, tau)
        out_r, lse_r = case.sess.decode(case.hq(), case.W, tau)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(out_n.float()).all())
        assert torch.equal(out_n, out_r) and torch.equal(lse_n, lse_r), (cache, case.lengths.tolist())
