"""Parity of the output projection y = W^O [o_1; ...; o_H] (mla_output_project)
with the float64 oracle, on seeded per-head outputs o ~ N(0, 0.05^2) and
W^O ~ N(0, 0.006^2) at the DeepSeek-V3 shape (d_model 7168, 128 heads of 128):
the weight-streaming kernel (at most 64 rows), the general GEMM with and
without K splits (more rows), the generic fp32 path on the tiny shape, and
decode -> combine -> W^O end to end.  Tolerances: bf16 max|d| <= 2e-2 max|ref|,
fp32 max|d| <= 1e-4 max(1, max|ref|)."""
import os

import numpy as np
import pytest
import torch

import oracle
import mla_latent_kv_29_amd as m
from mla_latent_kv_29_amd import inputs
from gpu_common import Case, DEV, tau_of, to_np, max_abs

pytestmark = pytest.mark.gpu
V3, TINY = inputs.V3_DIMS, inputs.TINY_DIMS
TOL_BF16 = 2e-2


def project(dims, act, rows, wl=7, std=0.05, sigma=0.006):
    tdt = torch.float32 if act == m.MLA_F32 else torch.bfloat16
    o = inputs.head_outputs(dims, rows, std, tdt, DEV, 0, wl)
    W = inputs.out_weight(dims, sigma, tdt, DEV, 0, wl)
    y = torch.full((rows, dims["d_model"]), float("nan"), dtype=tdt, device=DEV)
    d = m.make_dims(dims)
    wsb = m.mla_output_project_workspace_bytes(d, act, rows)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=DEV)
    m.mla_output_project(d, act, rows, o, W, y, ws, wsb)
    torch.cuda.synchronize()
    return o, W, to_np(y)


def check_rows(o, W, y, rows_checked, tol):
    ref = oracle.output_projection(to_np(o[rows_checked]), to_np(W))
    got = y[rows_checked]
    assert np.all(np.isfinite(y))
    assert max_abs(got, ref) <= tol * float(np.abs(ref).max()), (max_abs(got, ref), float(np.abs(ref).max()))


@pytest.mark.parametrize("rows", [1, 37, 64])
def test_output_project_few_rows_streaming_kernel(rows):
    o, W, y = project(V3, m.MLA_BF16, rows)
    check_rows(o, W, y, list(range(rows)), TOL_BF16)


@pytest.mark.parametrize("rows", [65, 300])
def test_output_project_many_rows_split_k(rows):
    """65 rows: two row tiles with a ragged second one, five K splits; 300
    rows: five row tiles, two K splits."""
    o, W, y = project(V3, m.MLA_BF16, rows)
    check_rows(o, W, y, list(range(rows)), TOL_BF16)


def test_output_project_many_rows_256_tiles():
    """2600 rows: the 256 x 256-tile kernel (11 row tiles x 28 column tiles),
    a ragged last row tile; sampled rows against the oracle."""
    o, W, y = project(V3, m.MLA_BF16, 2600)
    check_rows(o, W, y, [0, 255, 256, 1300, 2559, 2560, 2599], TOL_BF16)


def test_output_project_large_rows_single_pass():
    """1100 rows fill the chip without splitting K; sampled rows (first, last
    of a tile, ragged tail) against the oracle, all rows finite."""
    o, W, y = project(V3, m.MLA_BF16, 1100)
    check_rows(o, W, y, [0, 63, 64, 555, 1087, 1099], TOL_BF16)


@pytest.mark.parametrize("rows", [3, 70])
def test_output_project_fp32_tiny(rows):
    o, W, y = project(TINY, m.MLA_F32, rows, std=0.5, sigma=0.05)
    ref = oracle.output_projection(to_np(o), to_np(W))
    assert max_abs(y, ref) <= 1e-4 * max(1.0, float(np.abs(ref).max()))


def test_output_project_generic_matches_fast():
    """MLA_FORCE_GENERIC takes the VALU path for the same bf16 inputs."""
    o, W, y_fast = project(V3, m.MLA_BF16, 5)
    os.environ["MLA_FORCE_GENERIC"] = "1"
    try:
        _, _, y_gen = project(V3, m.MLA_BF16, 5)
    finally:
        del os.environ["MLA_FORCE_GENERIC"]
    check_rows(o, W, y_gen, list(range(5)), TOL_BF16)
    assert max_abs(y_fast, y_gen) <= 1e-2 * float(np.abs(y_gen).max())


def test_decode_combine_output_projection_end_to_end():
    """Two sequences with two query rows each: decode and combine through the
    session, then W^O on the combine's output rows, against the oracle's
    decode followed by its output projection."""
    case = Case(V3, "bf16", "bf16", [150, 70], s_q=2, table="shuffled", wl=7, num_splits=2)
    tau = tau_of(V3) * 20.0
    out, lse = case.sess.decode(case.hq(), case.W, tau)
    rows = out.shape[0] * out.shape[1]
    W = inputs.out_weight(V3, 0.006, torch.bfloat16, DEV, 0, 7)
    y = torch.empty((rows, V3["d_model"]), dtype=torch.bfloat16, device=DEV)
    d = m.make_dims(V3)
    wsb = m.mla_output_project_workspace_bytes(d, m.MLA_BF16, rows)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    m.mla_output_project(d, m.MLA_BF16, rows, out.contiguous(), W, y, ws, wsb)
    torch.cuda.synchronize()
    y = to_np(y)
    Wn = to_np(W)
    for b in range(2):
        o_ref, _ = case.oracle(b, tau)
        ref = oracle.output_projection(o_ref, Wn)
        got = y[2 * b:2 * b + 2]
        assert max_abs(got, ref) <= TOL_BF16 * float(np.abs(ref).max()), b
