"""FP8 (E4M3FN) latent cache at DeepSeek-V3 shapes.

Pages: the reading lesson "Читаем техотчёт DeepSeek-V3 вместе", §3.3: E4M3
(max 448) for all tensors, one scale per 1x128 activation tile.  Codes and
scales written by the library must equal the oracle's encoder bit for bit on
the same float32 inputs; decode outputs must match the oracle within
5e-2 * max|ref| against the unquantized oracle and 2e-2 * max|ref| against the
fp8-emulating oracle."""
import numpy as np
import pytest
import torch

import oracle
from mla_latent_kv_29_amd import inputs
from gpu_common import Case, tau_of, to_np, max_abs, read_fp8_rows, read_bf16_rows, DEV

pytestmark = pytest.mark.gpu
V3 = inputs.V3_DIMS


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_fp8_write_codes_and_scales_bit_exact(act):
    case = Case(V3, act, "fp8", [131, 64], s_q=1, table="shuffled", wl=4, planted=(0.5, 0.5))
    for b in range(2):
        c, r = case.lat[b]
        Lb = int(case.lengths[b])
        npg = (Lb + 63) // 64
        codes, scales, rope = read_fp8_rows(case.sess.pages, case.bt[b, :npg], V3)
        ref_codes, ref_scales = oracle.quantize_tiles(to_np(c))
        np.testing.assert_array_equal(codes[:Lb], ref_codes)
        np.testing.assert_array_equal(scales[:Lb], ref_scales)
        np.testing.assert_array_equal(rope[:Lb], to_np(r.to(torch.bfloat16)))


def test_fp8_append_from_h_matches_oracle_latents():
    case = Case(V3, "bf16", "fp8", [200], s_q=1, table="inorder", wl=4)
    Wn = case.weights_np()
    h = to_np(case.h(0, 0, 200))
    c, kr = oracle.kv_latents(h, Wn["W_DKV"], Wn["W_KR"], np.arange(200), V3["rope_theta"])
    codes, scales, rope = read_fp8_rows(case.sess.pages, case.bt[0, :4], V3)
    deq = oracle.dequantize_tiles(codes[:200], scales[:200])
    # within one E4M3 step of the exact latent (half a step of quantisation
    # plus the difference between fp32 and fp64 accumulation)
    g = np.abs(c).reshape(200, 4, 128)
    step = np.maximum(g * 2.0 ** -3, 2.0 ** -9 * scales[:200, :, None])
    assert np.all(np.abs(deq - c).reshape(200, 4, 128) <= step)
    assert max_abs(rope[:200], kr) <= 2e-2 * np.abs(kr).max()


def test_bf16_append_rows_match_oracle_latents():
    case = Case(V3, "bf16", "bf16", [150, 70], s_q=1, table="shuffled", wl=1)
    Wn = case.weights_np()
    for b in range(2):
        Lb = int(case.lengths[b])
        h = to_np(case.h(b, 0, Lb))
        c, kr = oracle.kv_latents(h, Wn["W_DKV"], Wn["W_KR"], np.arange(Lb), V3["rope_theta"])
        rows = read_bf16_rows(case.sess.pages, case.bt[b, :(Lb + 63) // 64], V3)[:Lb]
        ref = np.concatenate([c, kr], 1)
        assert max_abs(rows, ref) <= 1e-2 * np.abs(ref).max()


@pytest.mark.parametrize("s_q,kappa,splits", [(2, 1.0, 2), (2, 56.0, 3), (1, 56.0, 1), (4, 56.0, 2)])
def test_fp8_decode_parity(s_q, kappa, splits):
    case = Case(V3, "bf16", "fp8", [300, 65, 128], s_q=s_q, table="shuffled", wl=4, num_splits=splits)
    tau = tau_of(V3) * kappa
    out, lse, _ = case.run(tau)
    for b in range(3):
        o_q, l_q = case.oracle(b, tau, fp8=True)      # fp8-emulating oracle
        o, l = case.oracle(b, tau)                    # unquantized oracle
        assert max_abs(out[b], o_q) <= 2e-2 * float(np.abs(o_q).max()), (b, "emulated")
        assert max_abs(out[b], o) <= 5e-2 * float(np.abs(o).max()), (b, "unquantized")
        assert max_abs(lse[b], l) <= 5e-2 * max(1.0, float(np.abs(l).max()))


def test_fp8_planted_decode_vs_emulated_oracle():
    case = Case(V3, "bf16", "fp8", [257, 33], s_q=2, table="shuffled", wl=4, num_splits=2, planted=(0.5, 0.5))
    tau = tau_of(V3) * 56.0
    out, lse, hq = case.run(tau)
    for b in range(2):
        o_q, _ = case.oracle(b, tau, hq=hq, fp8=True)
        assert max_abs(out[b], o_q) <= 2e-2 * float(np.abs(o_q).max())


@pytest.mark.parametrize("splits", [1, 2])
def test_fp8_bytes_past_the_end_are_ignored(splits):
    """Page slots past a sequence's length hold NaN patterns in all three
    blocks (E4M3 code 0xFF, fp32 scale 0xFFFFFFFF, bf16 k^R 0xFFFF): those
    tokens are not visible, so the output must stay finite and unchanged."""
    from gpu_common import slot_x
    case = Case(V3, "bf16", "fp8", [300, 129, 64], s_q=1, table="shuffled", wl=4, num_splits=splits)
    ps, dc, dr = V3["page_size"], V3["d_c"], V3["d_rope"]
    s_off = ps * dc
    r_off = s_off + ps * (dc // 128) * 4
    raw = case.sess.pages.cpu().numpy()
    for b, Lb in enumerate(case.lengths):
        if Lb % ps == 0:
            continue
        last = int(case.bt[b, (int(Lb) - 1) // ps])
        t = np.arange(int(Lb) % ps, ps)[:, None]
        ch = np.arange(dc)[None, :]
        C = ch // 16
        raw[last, (16 * (C * ps + (t ^ slot_x(C))) + ch % 16).ravel()] = 0xFF
        raw[last, (s_off + 16 * t + np.arange(16)[None, :]).ravel()] = 0xFF
        m = np.arange(dr)[None, :]
        Cm = m // 8
        roff = (r_off + 16 * (Cm * ps + (t ^ slot_x(Cm))) + 2 * (m % 8)).ravel()
        raw[last, roff] = 0xFF
        raw[last, roff + 1] = 0xFF
    case.sess.pages.copy_(torch.from_numpy(raw))
    torch.cuda.synchronize()
    tau = tau_of(V3) * 56.0
    out, lse, _ = case.run(tau)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    for b in range(3):
        o_q, _ = case.oracle(b, tau, fp8=True)
        assert max_abs(out[b], o_q) <= 2e-2 * float(np.abs(o_q).max()), b
