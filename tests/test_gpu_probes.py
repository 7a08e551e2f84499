"""The two measurement probes of the library (no part of the MLA maths) run
through the C ABI: they finish, report their work, and leave the sink
untouched.  Each writes its sink only when its result equals one particular
value; zero inputs keep the results at zero, so that never happens here."""
import pytest
import torch

from mla_latent_kv_29_amd import _lib as m

pytestmark = pytest.mark.gpu

DEV = "cuda"


def test_hbm_read_probe_runs_and_writes_nothing():
    src = torch.zeros(1 << 20, device=DEV)  # 4 MiB
    sink = torch.zeros(4, dtype=torch.int32, device=DEV)
    assert m.mla_hbm_read_probe(src, src.numel() * 4, sink) == m.MLA_OK
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0


def test_mfma_probe_runs_and_reports_its_flops():
    ops = torch.zeros(12 * 64 * 8, dtype=torch.bfloat16, device=DEV)
    sink = torch.zeros(4, dtype=torch.float32, device=DEV)
    st, flops = m.mla_mfma_probe(ops, 4, sink)
    torch.cuda.synchronize()
    assert st == m.MLA_OK
    # 4096 waves x 4 iterations x 32 MFMAs of 32 x 32 x 16 multiply-adds
    assert flops == 4096 * 4 * 32 * (32 * 32 * 16 * 2)
    assert float(sink.abs().sum()) == 0.0
