"""ctypes binding of libmla.so (the C ABI declared in include/mla.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of the library.  Torch tensors are accepted for device memory and
streams; their data pointers are passed straight through.  If the library is
missing the import fails loudly -- there is no fallback implementation.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla.so")

MLA_OK, MLA_ERR_NULL, MLA_ERR_DIMS, MLA_ERR_DTYPE = 0, -1, -2, -3
MLA_ERR_ALIGN, MLA_ERR_WORKSPACE, MLA_ERR_UNSUPPORTED, MLA_ERR_HIP = -4, -5, -6, -7
MLA_F32, MLA_BF16, MLA_FP8_E4M3, MLA_FP8_E4M3_E8 = 0, 1, 2, 3

EXPORTS = ("mla_page_bytes", "mla_cache_append", "mla_append_workspace_bytes", "mla_cache_append_ws", "mla_cache_write", "mla_default_splits", "mla_plan_splits", "mla_decode_splits",
           "mla_workspace_bytes", "mla_decode", "mla_decode_query", "mla_decode_attend", "mla_combine",
           "mla_prefill_workspace_bytes", "mla_prefill", "mla_prefill_project", "mla_prefill_attend",
           "mla_output_project_workspace_bytes", "mla_output_project", "mla_fp8_quantize_weight",
           "mla_fp8_quantize_weight_t", "mla_fp8_gemm_workspace_bytes", "mla_fp8_gemm", "mla_mtp_tokens_per_step",
           "mla_decode_step_noalloc", "mla_decode_fp8w_workspace_bytes", "mla_decode_fp8w",
           "mla_decode_fp8w_query", "mla_combine_fp8w", "mla_check_metadata", "mla_hbm_read_probe", "mla_mfma_probe", "mla_status_str",
           "mla_last_hip_error", "mla_version")


class mla_dims(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("d_head", ctypes.c_int32),
                ("d_rope", ctypes.c_int32), ("d_c", ctypes.c_int32), ("d_cq", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("rope_theta", ctypes.c_float)]


class mla_cache(ctypes.Structure):
    _fields_ = [("pages", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("num_pages", ctypes.c_int32)]


class MLAError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        msg = f"{fn} failed: {status} ({status_str(status)})"
        if status == MLA_ERR_HIP:
            msg += ": " + _lib.mla_last_hip_error().decode()
        super().__init__(msg)


def _load():
    # torch ships its own HIP runtime under the same soname as ROCm's.  Loading
    # it first makes libmla.so bind to that runtime too, so that the library and
    # the torch tensors it is handed live in one HIP context.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run python mla_latent_kv_29_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    D = ctypes.POINTER(mla_dims)
    C = ctypes.POINTER(mla_cache)
    sig = {
        "mla_page_bytes": (SZ, [D, I32]),
        "mla_cache_append": (ctypes.c_int, [D, I32, P, I32, P, P, P, P, C, P, I32, P]),
        "mla_append_workspace_bytes": (SZ, [D, I32, I32]),
        "mla_cache_append_ws": (ctypes.c_int, [D, I32, P, I32, P, P, P, P, C, P, I32, P, SZ, P]),
        "mla_cache_write": (ctypes.c_int, [D, I32, P, P, I32, P, P, C, P, I32, P]),
        "mla_default_splits": (I32, [D, I32, I32, I32]),
        "mla_plan_splits": (I32, [D, I32, I32, I32, P]),
        "mla_decode_splits": (I32, [D, I32, I32, I32, I32]),
        "mla_workspace_bytes": (SZ, [D, I32, I32, I32, I32]),
        "mla_decode": (ctypes.c_int, [D, I32, P, I32, I32, P, P, P, C, P, I32, P, F, I32, P, SZ, P]),
        "mla_decode_query": (ctypes.c_int, [D, I32, P, I32, I32, P, P, P, C, P, I32, P, F, I32, P, SZ, P]),
        "mla_decode_attend": (ctypes.c_int, [D, I32, P, I32, I32, P, P, P, C, P, I32, P, F, I32, P, SZ, P]),
        "mla_combine": (ctypes.c_int, [D, I32, I32, I32, I32, P, SZ, P, P, P, P]),
        "mla_prefill_workspace_bytes": (SZ, [D, I32, I32]),
        "mla_prefill": (ctypes.c_int, [D, I32, P, I32, I32, P, I32, P, P, P, P, P, P, F, P, P, P, SZ, P]),
        "mla_prefill_project": (ctypes.c_int, [D, I32, P, I32, I32, P, I32, P, P, P, P, P, P, F, P, P, P, SZ, P]),
        "mla_prefill_attend": (ctypes.c_int, [D, I32, P, I32, I32, P, I32, P, P, P, P, P, P, F, P, P, P, SZ, P]),
        "mla_output_project_workspace_bytes": (SZ, [D, I32, I32]),
        "mla_output_project": (ctypes.c_int, [D, I32, I32, P, P, P, P, SZ, P]),
        "mla_fp8_quantize_weight": (ctypes.c_int, [P, I32, I32, P, P, P]),
        "mla_fp8_quantize_weight_t": (ctypes.c_int, [P, I32, I32, I32, P, P, P]),
        "mla_fp8_gemm_workspace_bytes": (SZ, [I32, I32, I32]),
        "mla_fp8_gemm": (ctypes.c_int, [I32, I32, I32, P, P, P, P, P, SZ, P]),
        "mla_mtp_tokens_per_step": (ctypes.c_double, [ctypes.c_double, I32]),
        "mla_decode_step_noalloc": (ctypes.c_int, [D, I32, P, I32, I32, P, P, P, P, C, P, I32, P, F, I32, P, P, P]),
        "mla_decode_fp8w_workspace_bytes": (SZ, [D, I32, I32, I32]),
        "mla_decode_fp8w": (ctypes.c_int, [D, P, I32, I32, P, P, P, P, P, P, C, P, I32, P, F, I32, P, SZ, P]),
        "mla_decode_fp8w_query": (ctypes.c_int, [D, P, I32, I32, P, P, P, P, P, P, C, P, I32, P, F, I32, P, SZ, P]),
        "mla_combine_fp8w": (ctypes.c_int, [D, I32, I32, I32, P, SZ, P, P, P, P, P]),
        "mla_check_metadata": (ctypes.c_int, [D, C, P, I32, P, I32, P, P]),
        "mla_hbm_read_probe": (ctypes.c_int, [P, SZ, P, P]),
        "mla_mfma_probe": (ctypes.c_int, [P, ctypes.c_int32, P, ctypes.POINTER(ctypes.c_double), P]),
        "mla_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "mla_version": (ctypes.c_char_p, []),
        "mla_last_hip_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()


def lib():
    return _lib


def status_str(status):
    return _lib.mla_status_str(int(status)).decode()


def version():
    return _lib.mla_version().decode()


def make_dims(d):
    """mla_dims from a dict with d_model, n_heads, d_head, d_rope, d_c, d_cq,
    page_size, rope_theta."""
    return mla_dims(int(d["d_model"]), int(d["n_heads"]), int(d["d_head"]), int(d["d_rope"]),
                    int(d["d_c"]), int(d["d_cq"]), int(d["page_size"]), float(d["rope_theta"]))


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn, st):
    if st != MLA_OK:
        raise MLAError(fn, st)


def mla_page_bytes(dims, cache_dtype):
    return int(_lib.mla_page_bytes(ctypes.byref(dims), int(cache_dtype)))


def mla_append_workspace_bytes(dims, act, n_tok):
    return int(_lib.mla_append_workspace_bytes(ctypes.byref(dims), int(act), int(n_tok)))


def mla_cache_append_ws(dims, act_dtype, h, n_tok, seq_id, pos, W_DKV, W_KR, cache, block_table, max_pages, ws,
                        ws_bytes, stream=None, check=True):
    st = _lib.mla_cache_append_ws(ctypes.byref(dims), int(act_dtype), _ptr(h), int(n_tok), _ptr(seq_id), _ptr(pos),
                                  _ptr(W_DKV), _ptr(W_KR), ctypes.byref(cache), _ptr(block_table), int(max_pages),
                                  _ptr(ws), int(ws_bytes), _stream(stream))
    if check:
        _check("mla_cache_append_ws", st)
    return st


def mla_output_project_workspace_bytes(dims, act, rows):
    return int(_lib.mla_output_project_workspace_bytes(ctypes.byref(dims), int(act), int(rows)))


def mla_output_project(dims, act, rows, o, W_O, y, ws, ws_bytes, stream=None, check=True):
    st = _lib.mla_output_project(ctypes.byref(dims), int(act), int(rows), _ptr(o), _ptr(W_O), _ptr(y), _ptr(ws),
                                 int(ws_bytes), _stream(stream))
    if check:
        _check("mla_output_project", st)
    return st


def mla_fp8_quantize_weight(W, N, K, codes, scales, stream=None, check=True):
    st = _lib.mla_fp8_quantize_weight(_ptr(W), int(N), int(K), _ptr(codes), _ptr(scales), _stream(stream))
    if check:
        _check("mla_fp8_quantize_weight", st)
    return st


def mla_fp8_quantize_weight_t(W, batch, R, C, codes, scales, stream=None, check=True):
    st = _lib.mla_fp8_quantize_weight_t(_ptr(W), int(batch), int(R), int(C), _ptr(codes), _ptr(scales),
                                        _stream(stream))
    if check:
        _check("mla_fp8_quantize_weight_t", st)
    return st


def mla_fp8_gemm_workspace_bytes(M, N, K):
    return int(_lib.mla_fp8_gemm_workspace_bytes(int(M), int(N), int(K)))


def mla_fp8_gemm(M, N, K, X, W_codes, W_scales, Y, ws, ws_bytes, stream=None, check=True):
    st = _lib.mla_fp8_gemm(int(M), int(N), int(K), _ptr(X), _ptr(W_codes), _ptr(W_scales), _ptr(Y), _ptr(ws),
                           int(ws_bytes), _stream(stream))
    if check:
        _check("mla_fp8_gemm", st)
    return st


def mla_mtp_tokens_per_step(acceptance, depth):
    return float(_lib.mla_mtp_tokens_per_step(float(acceptance), int(depth)))


def mla_default_splits(dims, batch, s_q, max_pages):
    return int(_lib.mla_default_splits(ctypes.byref(dims), int(batch), int(s_q), int(max_pages)))


def mla_plan_splits(dims, batch, s_q, max_pages, seqlens):
    """seqlens: host lengths (any int sequence), passed as an int32 array."""
    import numpy as np
    arr = np.ascontiguousarray(np.asarray(seqlens), dtype=np.int32)
    if arr.shape != (int(batch),):
        raise ValueError("seqlens must hold batch lengths")
    return int(_lib.mla_plan_splits(ctypes.byref(dims), int(batch), int(s_q), int(max_pages),
                                    arr.ctypes.data_as(ctypes.c_void_p)))


def mla_decode_splits(dims, batch, s_q, max_pages, num_splits):
    return int(_lib.mla_decode_splits(ctypes.byref(dims), int(batch), int(s_q), int(max_pages), int(num_splits)))


def mla_workspace_bytes(dims, act_dtype, batch, s_q, num_splits):
    return int(_lib.mla_workspace_bytes(ctypes.byref(dims), int(act_dtype), int(batch), int(s_q), int(num_splits)))


def cache_struct(pages, cache_dtype, num_pages):
    return mla_cache(ctypes.c_void_p(_ptr(pages)), int(cache_dtype), int(num_pages))


def mla_cache_append(dims, act_dtype, h, n_tok, seq_id, pos, W_DKV, W_KR, cache, block_table, max_pages,
                     stream=None, check=True):
    st = _lib.mla_cache_append(ctypes.byref(dims), int(act_dtype), _ptr(h), int(n_tok), _ptr(seq_id), _ptr(pos),
                               _ptr(W_DKV), _ptr(W_KR), ctypes.byref(cache), _ptr(block_table), int(max_pages),
                               _stream(stream))
    if check:
        _check("mla_cache_append", st)
    return st


def mla_cache_write(dims, act_dtype, c_kv, k_rope, n_tok, seq_id, pos, cache, block_table, max_pages,
                    stream=None, check=True):
    st = _lib.mla_cache_write(ctypes.byref(dims), int(act_dtype), _ptr(c_kv), _ptr(k_rope), int(n_tok),
                              _ptr(seq_id), _ptr(pos), ctypes.byref(cache), _ptr(block_table), int(max_pages),
                              _stream(stream))
    if check:
        _check("mla_cache_write", st)
    return st


def mla_decode(dims, act_dtype, hq, batch, s_q, W_DQ, W_UQ, W_UK, cache, block_table, max_pages, seqlens,
               softmax_scale, num_splits, ws, ws_bytes, stream=None, check=True):
    st = _lib.mla_decode(ctypes.byref(dims), int(act_dtype), _ptr(hq), int(batch), int(s_q), _ptr(W_DQ),
                         _ptr(W_UQ), _ptr(W_UK), ctypes.byref(cache), _ptr(block_table), int(max_pages),
                         _ptr(seqlens), float(softmax_scale), int(num_splits), _ptr(ws), int(ws_bytes),
                         _stream(stream))
    if check:
        _check("mla_decode", st)
    return st


def _decode_call(name, dims, act_dtype, hq, batch, s_q, W_DQ, W_UQ, W_UK, cache, block_table, max_pages, seqlens,
                 softmax_scale, num_splits, ws, ws_bytes, stream=None, check=True):
    st = getattr(_lib, name)(ctypes.byref(dims), int(act_dtype), _ptr(hq), int(batch), int(s_q), _ptr(W_DQ),
                             _ptr(W_UQ), _ptr(W_UK), ctypes.byref(cache), _ptr(block_table), int(max_pages),
                             _ptr(seqlens), float(softmax_scale), int(num_splits), _ptr(ws), int(ws_bytes),
                             _stream(stream))
    if check:
        _check(name, st)
    return st


def mla_decode_query(*args, **kw):
    return _decode_call("mla_decode_query", *args, **kw)


def mla_decode_attend(*args, **kw):
    return _decode_call("mla_decode_attend", *args, **kw)


def mla_combine(dims, act_dtype, batch, s_q, num_splits, ws, ws_bytes, W_UV, out, lse_out=None, stream=None,
                check=True):
    st = _lib.mla_combine(ctypes.byref(dims), int(act_dtype), int(batch), int(s_q), int(num_splits), _ptr(ws),
                          int(ws_bytes), _ptr(W_UV), _ptr(out), _ptr(lse_out), _stream(stream))
    if check:
        _check("mla_combine", st)
    return st


def mla_decode_fp8w_workspace_bytes(dims, batch, s_q, num_splits):
    return int(_lib.mla_decode_fp8w_workspace_bytes(ctypes.byref(dims), int(batch), int(s_q), int(num_splits)))


def _fp8w_call(name, dims, hq, batch, s_q, W_DQ, W_UQ, W_UKT, cache, block_table, max_pages, seqlens,
               softmax_scale, num_splits, ws, ws_bytes, stream=None, check=True):
    """W_DQ, W_UQ, W_UKT: (codes, scales) pairs of mla_fp8_quantize_weight."""
    st = getattr(_lib, name)(ctypes.byref(dims), _ptr(hq), int(batch), int(s_q), _ptr(W_DQ[0]), _ptr(W_DQ[1]),
                             _ptr(W_UQ[0]), _ptr(W_UQ[1]), _ptr(W_UKT[0]), _ptr(W_UKT[1]), ctypes.byref(cache),
                             _ptr(block_table), int(max_pages), _ptr(seqlens), float(softmax_scale),
                             int(num_splits), _ptr(ws), int(ws_bytes), _stream(stream))
    if check:
        _check(name, st)
    return st


def mla_decode_fp8w(*args, **kw):
    return _fp8w_call("mla_decode_fp8w", *args, **kw)


def mla_decode_fp8w_query(*args, **kw):
    return _fp8w_call("mla_decode_fp8w_query", *args, **kw)


def mla_combine_fp8w(dims, batch, s_q, num_splits, ws, ws_bytes, W_UV, out, lse_out=None, stream=None, check=True):
    """W_UV: (codes, scales) of mla_fp8_quantize_weight."""
    st = _lib.mla_combine_fp8w(ctypes.byref(dims), int(batch), int(s_q), int(num_splits), _ptr(ws), int(ws_bytes),
                               _ptr(W_UV[0]), _ptr(W_UV[1]), _ptr(out), _ptr(lse_out), _stream(stream))
    if check:
        _check("mla_combine_fp8w", st)
    return st


def mla_check_metadata(dims, cache, block_table, max_pages, seqlens, batch, bad, stream=None, check=True):
    """Enqueues the metadata check; bad (device int32[2]) holds the counts once the stream has run."""
    st = _lib.mla_check_metadata(ctypes.byref(dims), ctypes.byref(cache), _ptr(block_table), int(max_pages),
                                 _ptr(seqlens), int(batch), _ptr(bad), _stream(stream))
    if check:
        _check("mla_check_metadata", st)
    return st


NOALLOC_SCRATCH_BYTES = 64 << 20  # MLA_NOALLOC_SCRATCH_BYTES of include/mla.h


def mla_decode_step_noalloc(dims, act_dtype, hq, batch, s_q, W_DQ, W_UQ, W_UK, W_UV, cache, block_table, max_pages,
                            seqlens, softmax_scale, num_splits, out, lse_out=None, stream=None, check=True):
    st = _lib.mla_decode_step_noalloc(ctypes.byref(dims), int(act_dtype), _ptr(hq), int(batch), int(s_q), _ptr(W_DQ),
                                      _ptr(W_UQ), _ptr(W_UK), _ptr(W_UV), ctypes.byref(cache), _ptr(block_table),
                                      int(max_pages), _ptr(seqlens), float(softmax_scale), int(num_splits),
                                      _ptr(out), _ptr(lse_out), _stream(stream))
    if check:
        _check("mla_decode_step_noalloc", st)
    return st


def mla_mfma_probe(ops, iters, sink, stream=None, check=True):
    """Returns (status, flops of the launch)."""
    fl = ctypes.c_double(0.0)
    st = _lib.mla_mfma_probe(_ptr(ops), int(iters), _ptr(sink), ctypes.byref(fl), _stream(stream))
    if check:
        _check("mla_mfma_probe", st)
    return st, fl.value


def mla_hbm_read_probe(src, nbytes, sink, stream=None, check=True):
    st = _lib.mla_hbm_read_probe(_ptr(src), int(nbytes), _ptr(sink), _stream(stream))
    if check:
        _check("mla_hbm_read_probe", st)
    return st


def mla_prefill_workspace_bytes(dims, act_dtype, n_tok):
    return int(_lib.mla_prefill_workspace_bytes(ctypes.byref(dims), int(act_dtype), int(n_tok)))


def _prefill_call(name, dims, act_dtype, h, n_tok, n_seq, cu_seqlens, max_seqlen, W_DQ, W_UQ, W_UK, W_UV, W_DKV,
                  W_KR, softmax_scale, out, lse_out, ws, ws_bytes, stream=None, check=True):
    st = getattr(_lib, name)(ctypes.byref(dims), int(act_dtype), _ptr(h), int(n_tok), int(n_seq), _ptr(cu_seqlens),
                             int(max_seqlen), _ptr(W_DQ), _ptr(W_UQ), _ptr(W_UK), _ptr(W_UV), _ptr(W_DKV),
                             _ptr(W_KR), float(softmax_scale), _ptr(out), _ptr(lse_out), _ptr(ws), int(ws_bytes),
                             _stream(stream))
    if check:
        _check(name, st)
    return st


def mla_prefill(*args, **kw):
    return _prefill_call("mla_prefill", *args, **kw)


def mla_prefill_project(*args, **kw):
    return _prefill_call("mla_prefill_project", *args, **kw)


def mla_prefill_attend(*args, **kw):
    return _prefill_call("mla_prefill_attend", *args, **kw)
