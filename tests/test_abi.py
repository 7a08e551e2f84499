"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every symbol include/mla.h declares, computes sizes as documented and rejects
invalid arguments before enqueueing anything (stream argument 0, no device
pointer is ever dereferenced on these paths)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

import mla_latent_kv_29_amd as m
from mla_latent_kv_29_amd import _lib as L
from mla_latent_kv_29_amd import inputs


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "mla.h")).read()
    return set(re.findall(r"MLA_API\s+[\w\s\*]+?\b(mla_\w+)\s*\(", src))


def test_header_declarations_are_all_exported():
    decl = declared_symbols()
    assert decl == set(L.EXPORTS), decl ^ set(L.EXPORTS)
    lib = ctypes.CDLL(L.LIB_PATH)
    for name in decl:
        assert hasattr(lib, name), name


def test_status_strings_and_version():
    assert m.status_str(0) == "ok"
    for s in range(-7, 0):
        assert m.status_str(s) and m.status_str(s) != "unknown status"
    assert "gfx950" in m.version()


def test_page_bytes_layouts():
    d = m.make_dims(inputs.V3_DIMS)
    assert m.mla_page_bytes(d, m.MLA_BF16) == 64 * 576 * 2
    assert m.mla_page_bytes(d, m.MLA_F32) == 64 * 576 * 4
    assert m.mla_page_bytes(d, m.MLA_FP8_E4M3) == 64 * (512 + 4 * 4 + 2 * 64)  # 41 984
    t = m.make_dims(inputs.TINY_DIMS)
    assert m.mla_page_bytes(t, m.MLA_FP8_E4M3) == 0       # d_c % 128 != 0
    assert m.mla_page_bytes(t, 7) == 0


def test_default_splits_and_workspace():
    d = m.make_dims(inputs.V3_DIMS)
    for batch, s_q, mp in [(64, 1, 64), (4, 1, 2048), (128, 2, 128), (1, 1, 1)]:
        s = m.mla_default_splits(d, batch, s_q, mp)
        assert 1 <= s <= mp
        assert m.mla_workspace_bytes(d, m.MLA_BF16, batch, s_q, s) > 0
    assert m.mla_workspace_bytes(d, m.MLA_BF16, 64, 9, 1) == 0
    assert m.mla_workspace_bytes(d, m.MLA_BF16, 64, 1, 0) == 0
    w1 = m.mla_workspace_bytes(d, m.MLA_BF16, 64, 1, 1)
    w4 = m.mla_workspace_bytes(d, m.MLA_BF16, 64, 1, 4)
    assert w4 - w1 >= 3 * 64 * 128 * 512 * 4


FAKE = 1 << 40  # aligned non-null value; never dereferenced on the paths below


def _dims(**kw):
    d = dict(inputs.V3_DIMS)
    d.update(kw)
    return m.make_dims(d)


@pytest.mark.parametrize("kw,expect", [
    (dict(d_c=0), L.MLA_ERR_DIMS), (dict(d_rope=7), L.MLA_ERR_DIMS), (dict(page_size=63), L.MLA_ERR_DIMS),
    (dict(d_rope=256), L.MLA_ERR_DIMS), (dict(rope_theta=0.0), L.MLA_ERR_DIMS),
])
def test_decode_rejects_bad_dims(kw, expect):
    d = _dims(**kw)
    cache = L.cache_struct(FAKE, m.MLA_BF16, 10)
    st = m.mla_decode(d, m.MLA_BF16, FAKE, 1, 1, FAKE, FAKE, FAKE, cache, FAKE, 4, FAKE, 0.1, 1, FAKE,
                      1 << 30, stream=0, check=False)
    assert st == expect


def test_decode_argument_errors():
    d = _dims()
    cache = L.cache_struct(FAKE, m.MLA_BF16, 10)
    args = lambda **o: dict(dict(act=m.MLA_BF16, hq=FAKE, batch=2, s_q=1, wdq=FAKE, cache=cache, bt=FAKE,
                                 mp=4, sl=FAKE, ns=1, ws=FAKE, wsb=1 << 34), **o)

    def call(a):
        return m.mla_decode(d, a["act"], a["hq"], a["batch"], a["s_q"], a["wdq"], FAKE, FAKE, a["cache"], a["bt"],
                            a["mp"], a["sl"], 0.1, a["ns"], a["ws"], a["wsb"], stream=0, check=False)

    assert call(args(act=5)) == L.MLA_ERR_DTYPE
    assert call(args(s_q=0)) == L.MLA_ERR_DIMS
    assert call(args(s_q=9)) == L.MLA_ERR_DIMS
    assert call(args(hq=None)) == L.MLA_ERR_NULL
    assert call(args(ws=None)) == L.MLA_ERR_NULL
    assert call(args(bt=None)) == L.MLA_ERR_NULL
    assert call(args(hq=FAKE + 2)) == L.MLA_ERR_ALIGN
    assert call(args(wsb=1000)) == L.MLA_ERR_WORKSPACE
    assert call(args(mp=0)) == L.MLA_ERR_DIMS
    assert call(args(cache=L.cache_struct(FAKE, m.MLA_F32, 10))) == L.MLA_ERR_DTYPE   # bf16 act, f32 cache
    assert call(args(cache=L.cache_struct(FAKE, 9, 10))) == L.MLA_ERR_DTYPE
    assert call(args(batch=0)) == L.MLA_OK                                            # no-op
    t = m.make_dims(inputs.TINY_DIMS)
    st = m.mla_decode(t, m.MLA_F32, FAKE, 1, 1, FAKE, FAKE, FAKE, L.cache_struct(FAKE, m.MLA_FP8_E4M3, 4), FAKE, 4,
                      FAKE, 0.1, 1, FAKE, 1 << 30, stream=0, check=False)
    assert st == L.MLA_ERR_UNSUPPORTED                                               # fp8 needs d_c % 128 == 0


def test_append_and_combine_argument_errors():
    d = _dims()
    cache = L.cache_struct(FAKE, m.MLA_BF16, 10)
    assert m.mla_cache_append(d, m.MLA_BF16, FAKE, 0, FAKE, FAKE, FAKE, FAKE, cache, FAKE, 4, stream=0,
                              check=False) == L.MLA_OK
    assert m.mla_cache_append(d, m.MLA_BF16, None, 3, FAKE, FAKE, FAKE, FAKE, cache, FAKE, 4, stream=0,
                              check=False) == L.MLA_ERR_NULL
    assert m.mla_cache_append(d, m.MLA_BF16, FAKE, -1, FAKE, FAKE, FAKE, FAKE, cache, FAKE, 4, stream=0,
                              check=False) == L.MLA_ERR_DIMS
    assert m.mla_cache_append(d, m.MLA_BF16, FAKE, 3, FAKE, FAKE + 4, FAKE, FAKE, cache, FAKE, 4, stream=0,
                              check=False) == L.MLA_ERR_ALIGN
    assert m.mla_cache_write(d, m.MLA_BF16, FAKE, None, 3, FAKE, FAKE, cache, FAKE, 4, stream=0,
                             check=False) == L.MLA_ERR_NULL
    assert m.mla_combine(d, m.MLA_BF16, 2, 1, FAKE, 10, FAKE, FAKE, None, stream=0, check=False) == \
        L.MLA_ERR_WORKSPACE
    assert m.mla_combine(d, m.MLA_BF16, 2, 1, FAKE, 1 << 34, None, FAKE, None, stream=0, check=False) == \
        L.MLA_ERR_NULL
    assert m.mla_combine(d, m.MLA_BF16, 0, 1, None, 0, None, None, None, stream=0, check=False) == L.MLA_OK


def test_prefill_workspace_and_argument_errors():
    d = _dims()
    w1 = m.mla_prefill_workspace_bytes(d, m.MLA_BF16, 1)
    w100 = m.mla_prefill_workspace_bytes(d, m.MLA_BF16, 100)
    # RoPE frequencies (256 B), then per token: position, 32 (cos, sin) pairs, c^KV, k^R, c^Q,
    # q, k^C and v^C (bf16), 256-byte aligned regions
    per_tok = 4 + 32 * 8 + 2 * (512 + 64 + 1536 + 128 * 192 + 2 * 128 * 128)
    assert w100 >= 256 + 100 * per_tok and w100 < 256 + 100 * per_tok + 8 * 256
    assert 0 < w1 < w100
    assert m.mla_prefill_workspace_bytes(d, m.MLA_BF16, -1) == 0

    def call(**o):
        a = dict(act=m.MLA_BF16, h=FAKE, n=100, ns=2, cu=FAKE, mx=64, wuv=FAKE, out=FAKE, lse=None, ws=FAKE,
                 wsb=w100, dims=d, tau=0.1)
        a.update(o)
        return m.mla_prefill(a["dims"], a["act"], a["h"], a["n"], a["ns"], a["cu"], a["mx"], FAKE, FAKE, FAKE,
                             a["wuv"], FAKE, FAKE, a["tau"], a["out"], a["lse"], a["ws"], a["wsb"], stream=0,
                             check=False)

    assert call(n=0) == L.MLA_OK                                   # no-op
    assert call(act=7) == L.MLA_ERR_DTYPE
    assert call(ns=0) == L.MLA_ERR_DIMS
    assert call(mx=0) == L.MLA_ERR_DIMS
    assert call(n=-3) == L.MLA_ERR_DIMS
    assert call(h=None) == L.MLA_ERR_NULL
    assert call(cu=None) == L.MLA_ERR_NULL
    assert call(wuv=None) == L.MLA_ERR_NULL
    assert call(out=FAKE + 8) == L.MLA_ERR_ALIGN
    assert call(lse=FAKE + 2) == L.MLA_ERR_ALIGN
    assert call(wsb=w100 - 1) == L.MLA_ERR_WORKSPACE
    assert call(tau=0.0) == L.MLA_ERR_DIMS
    assert call(act=m.MLA_F32) == L.MLA_ERR_UNSUPPORTED             # bf16 activations only
    assert call(dims=m.make_dims(inputs.TINY_DIMS)) == L.MLA_ERR_UNSUPPORTED


def test_mtp_tokens_per_step_matches_oracle():
    """Host arithmetic of the C ABI against the oracle's enumeration; invalid
    arguments give NaN."""
    import math
    import oracle
    for depth in range(0, 8):
        for a in (0.0, 0.5, 0.85, 0.9, 1.0):
            assert abs(m.mla_mtp_tokens_per_step(a, depth) - oracle.tokens_per_step(a, depth)) < 1e-12
    for a, depth in ((-0.1, 1), (1.1, 1), (float("nan"), 1), (0.5, -1), (0.5, 8)):
        assert math.isnan(m.mla_mtp_tokens_per_step(a, depth))


def test_output_project_workspace_and_argument_errors():
    d = _dims()
    K, N = 128 * 128, 7168
    # at most 64 rows: 16 k-groups of 1024 fp32 partials; more rows: K splits of the general GEMM
    assert m.mla_output_project_workspace_bytes(d, m.MLA_BF16, 1) == 16 * 1 * N * 4
    assert m.mla_output_project_workspace_bytes(d, m.MLA_BF16, 64) == 16 * 64 * N * 4
    assert m.mla_output_project_workspace_bytes(d, m.MLA_BF16, 72) == 5 * 72 * N * 4
    assert m.mla_output_project_workspace_bytes(d, m.MLA_BF16, 4096) == 4096 * N * 4
    assert m.mla_output_project_workspace_bytes(d, m.MLA_F32, 10) == 0
    assert m.mla_output_project_workspace_bytes(d, m.MLA_BF16, -1) == 0
    assert m.mla_output_project_workspace_bytes(d, 9, 10) == 0
    w = m.mla_output_project_workspace_bytes(d, m.MLA_BF16, 10)

    def call(**o):
        a = dict(act=m.MLA_BF16, rows=10, o=FAKE, w=FAKE, y=FAKE, ws=FAKE, wsb=w)
        a.update(o)
        return m.mla_output_project(d, a["act"], a["rows"], a["o"], a["w"], a["y"], a["ws"], a["wsb"], stream=0,
                                    check=False)

    assert call(rows=0) == L.MLA_OK                               # no-op
    assert call(act=7) == L.MLA_ERR_DTYPE
    assert call(act=m.MLA_FP8_E4M3) == L.MLA_ERR_DTYPE
    assert call(rows=-1) == L.MLA_ERR_DIMS
    assert call(rows=(1 << 17) + 1) == L.MLA_ERR_DIMS
    assert call(o=None) == L.MLA_ERR_NULL
    assert call(w=None) == L.MLA_ERR_NULL
    assert call(y=None) == L.MLA_ERR_NULL
    assert call(y=FAKE + 8) == L.MLA_ERR_ALIGN
    assert call(ws=None) == L.MLA_ERR_WORKSPACE
    assert call(wsb=w - 1) == L.MLA_ERR_WORKSPACE
    assert call(ws=FAKE + 4) == L.MLA_ERR_ALIGN


def test_fp8_gemm_workspace_and_argument_errors():
    # activation codes and scales of one 64-row chunk (256-byte aligned regions), then the
    # fp32 partials of the k-groups: W^DQ has 7 k-groups of 1024; K = 512 and K = 1536 are
    # one k-group each (no partials)
    def x_part(rows, K):
        return (rows * K + 255) // 256 * 256 + (rows * (K // 128) * 4 + 255) // 256 * 256
    assert m.mla_fp8_gemm_workspace_bytes(64, 1536, 7168) == x_part(64, 7168) + 7 * 64 * 1536 * 4
    assert m.mla_fp8_gemm_workspace_bytes(100, 1536, 7168) == x_part(64, 7168) + 7 * 64 * 1536 * 4
    assert m.mla_fp8_gemm_workspace_bytes(64, 16384, 512) == x_part(64, 512)
    assert m.mla_fp8_gemm_workspace_bytes(8, 24576, 1536) == x_part(8, 1536)
    assert m.mla_fp8_gemm_workspace_bytes(64, 7168, 16384) == x_part(64, 16384) + 16 * 64 * 7168 * 4
    assert m.mla_fp8_gemm_workspace_bytes(8, 24576, 1000) == 0                     # unsupported K
    assert m.mla_fp8_gemm_workspace_bytes(-1, 64, 512) == 0
    w = m.mla_fp8_gemm_workspace_bytes(10, 1536, 7168)

    def gemm(**o):
        a = dict(M=10, N=1536, K=7168, x=FAKE, wc=FAKE, wsc=FAKE, y=FAKE, ws=FAKE, wsb=w)
        a.update(o)
        return m.mla_fp8_gemm(a["M"], a["N"], a["K"], a["x"], a["wc"], a["wsc"], a["y"], a["ws"], a["wsb"],
                              stream=0, check=False)

    assert gemm(M=0) == L.MLA_OK
    assert gemm(M=-1) == L.MLA_ERR_DIMS
    assert gemm(N=0) == L.MLA_ERR_DIMS
    assert gemm(K=1 << 17) == L.MLA_ERR_DIMS
    assert gemm(N=40) == L.MLA_ERR_UNSUPPORTED
    assert gemm(K=640) == L.MLA_ERR_UNSUPPORTED
    assert gemm(x=None) == L.MLA_ERR_NULL
    assert gemm(wsc=None) == L.MLA_ERR_NULL
    assert gemm(y=FAKE + 2) == L.MLA_ERR_ALIGN
    assert gemm(wsc=FAKE + 2) == L.MLA_ERR_ALIGN
    assert gemm(ws=None) == L.MLA_ERR_WORKSPACE
    assert gemm(wsb=w - 4) == L.MLA_ERR_WORKSPACE

    def quant(**o):
        a = dict(w=FAKE, N=1536, K=7168, c=FAKE, s=FAKE)
        a.update(o)
        return m.mla_fp8_quantize_weight(a["w"], a["N"], a["K"], a["c"], a["s"], stream=0, check=False)

    assert quant(N=0) == L.MLA_ERR_DIMS
    assert quant(N=40) == L.MLA_ERR_UNSUPPORTED
    assert quant(K=100) == L.MLA_ERR_UNSUPPORTED
    assert quant(c=None) == L.MLA_ERR_NULL
    assert quant(w=FAKE + 8) == L.MLA_ERR_ALIGN
