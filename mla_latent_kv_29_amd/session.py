"""Device-buffer bookkeeping around the C ABI for one decode workload.

`DecodeSession` owns (as torch tensors) the paged cache, block table,
seqlens, workspace and output buffers of a batch, builds the cache through
mla_cache_append and runs mla_decode + mla_combine.  It does no arithmetic of
its own: every number is produced by libmla.so.
"""
import numpy as np
import torch

from . import _lib as L

ACT = {"f32": L.MLA_F32, "bf16": L.MLA_BF16}
CACHE = {"f32": L.MLA_F32, "bf16": L.MLA_BF16, "fp8": L.MLA_FP8_E4M3, "fp8e8": L.MLA_FP8_E4M3_E8}


class DecodeSession:
    def __init__(self, dims, act, cache_dtype, lengths, table, num_pages, s_q, num_splits=0, device="cuda"):
        """dims: dict of model dims; act: 'f32'|'bf16'; cache_dtype: 'f32'|'bf16'|'fp8'|'fp8e8';
        lengths: int array [batch] (seqlens, including the s_q query tokens);
        table: int32 numpy [batch, max_pages]; num_pages: size of the page pool."""
        self.dims = dict(dims)
        self.cdims = L.make_dims(dims)
        self.act_name, self.cache_name = act, cache_dtype
        self.act, self.cache_dtype = ACT[act], CACHE[cache_dtype]
        self.tdtype = torch.float32 if act == "f32" else torch.bfloat16
        self.device = device
        self.batch = len(lengths)
        self.s_q = s_q
        self.lengths = np.asarray(lengths, dtype=np.int64)
        self.max_pages = int(table.shape[1])
        self.num_pages = int(num_pages)
        self.page_bytes = L.mla_page_bytes(self.cdims, self.cache_dtype)
        if self.page_bytes == 0:
            raise ValueError("invalid dims / cache dtype")
        self.pages = torch.zeros((self.num_pages, self.page_bytes), dtype=torch.uint8, device=device)
        self.cache = L.cache_struct(self.pages, self.cache_dtype, self.num_pages)
        self.block_table = torch.from_numpy(np.ascontiguousarray(table, dtype=np.int32)).to(device)
        self.seqlens = torch.from_numpy(self.lengths.astype(np.int32)).to(device)
        self.set_splits(num_splits)
        H, dh = dims["n_heads"], dims["d_head"]
        self.out = torch.empty((self.batch, s_q, H, dh), dtype=self.tdtype, device=device)
        self.lse = torch.empty((self.batch, s_q, H), dtype=torch.float32, device=device)

    def set_splits(self, num_splits):
        """Split plan: num_splits per sequence (0 = the library's plan from the
        batch's lengths, mla_plan_splits), as mla_decode resolves it; the
        combine takes the same count."""
        if num_splits == 0 and self.batch > 0:
            num_splits = L.mla_plan_splits(self.cdims, self.batch, self.s_q, self.max_pages, self.lengths)
        s = L.mla_decode_splits(self.cdims, self.batch, self.s_q, self.max_pages, num_splits)
        if s <= 0:
            raise ValueError("invalid split request")
        self.num_splits = s
        self.ws_bytes = L.mla_workspace_bytes(self.cdims, self.act, self.batch, self.s_q, s)
        if self.ws_bytes == 0:
            raise ValueError("invalid workspace request")
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)

    # ---------------------------------------------------------------- cache
    def append(self, h, b, t0, W, stream=None):
        """Append rows h [n, d_model] as tokens t0..t0+n-1 of sequence b."""
        n = h.shape[0]
        seq_id = torch.full((n,), b, dtype=torch.int32, device=self.device)
        pos = torch.arange(t0, t0 + n, dtype=torch.int32, device=self.device)
        L.mla_cache_append(self.cdims, self.act, h, n, seq_id, pos, W["W_DKV"], W["W_KR"], self.cache,
                           self.block_table, self.max_pages, stream)

    def append_rows(self, h, seq_id, pos, W, stream=None, ws=False):
        """Append rows h at (seq_id[r], pos[r]); ws=True takes the workspace
        entry point (mla_cache_append_ws) with a workspace of its own."""
        n = h.shape[0]
        if not ws:
            L.mla_cache_append(self.cdims, self.act, h, n, seq_id, pos, W["W_DKV"], W["W_KR"], self.cache,
                               self.block_table, self.max_pages, stream)
            return
        need = L.mla_append_workspace_bytes(self.cdims, self.act, n)
        if need and (getattr(self, "append_ws", None) is None or self.append_ws.numel() < need):
            self.append_ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        buf = self.append_ws if need else None
        L.mla_cache_append_ws(self.cdims, self.act, h, n, seq_id, pos, W["W_DKV"], W["W_KR"], self.cache,
                              self.block_table, self.max_pages, buf, need, stream)

    def write(self, c_kv, k_rope, b, t0, stream=None):
        n = c_kv.shape[0]
        seq_id = torch.full((n,), b, dtype=torch.int32, device=self.device)
        pos = torch.arange(t0, t0 + n, dtype=torch.int32, device=self.device)
        L.mla_cache_write(self.cdims, self.act, c_kv, k_rope, n, seq_id, pos, self.cache, self.block_table,
                          self.max_pages, stream)

    def build_from_h(self, gen_h, W, chunk=16384, stream=None):
        """Append every token of every sequence; gen_h(b, t0, t1) -> h rows."""
        for b in range(self.batch):
            Lb = int(self.lengths[b])
            for t0 in range(0, Lb, chunk):
                t1 = min(Lb, t0 + chunk)
                self.append(gen_h(b, t0, t1), b, t0, W, stream)

    # ---------------------------------------------------------------- decode
    def decode(self, hq, W, softmax_scale, use_dq=True, stream=None):
        """hq: [batch*s_q, d_model] hidden states (or c^Q [batch*s_q, d_cq] with use_dq=False)."""
        L.mla_decode(self.cdims, self.act, hq, self.batch, self.s_q, W["W_DQ"] if use_dq else None, W["W_UQ"],
                     W["W_UK"], self.cache, self.block_table, self.max_pages, self.seqlens, softmax_scale,
                     self.num_splits, self.ws, self.ws_bytes, stream)
        L.mla_combine(self.cdims, self.act, self.batch, self.s_q, self.num_splits, self.ws, self.ws_bytes, W["W_UV"],
                      self.out, self.lse, stream)
        return self.out, self.lse

    # ---------------------------------------------------------------- FP8 projection weights
    def quantize_fp8w(self, W, stream=None):
        """E4M3 codes and 128 x 128-block scales of W^DQ, W^UQ, W^UK (transposed
        per head, the layout mla_decode_fp8w takes) and W^UV, made by the
        library: {name: (codes, scales)}."""
        d = self.dims
        H, dh, dr, dc = d["n_heads"], d["d_head"], d["d_rope"], d["d_c"]

        def q(w, N, K):
            codes = torch.empty((N, K), dtype=torch.uint8, device=self.device)
            scales = torch.empty(((N + 127) // 128, K // 128), dtype=torch.float32, device=self.device)
            L.mla_fp8_quantize_weight(w, N, K, codes, scales, stream)
            return codes, scales

        ukt = (torch.empty((H * dc, dh), dtype=torch.uint8, device=self.device),
               torch.empty((H * dc // 128, dh // 128), dtype=torch.float32, device=self.device))
        L.mla_fp8_quantize_weight_t(W["W_UK"], H, dh, dc, ukt[0], ukt[1], stream)
        return {"W_DQ": q(W["W_DQ"], d["d_cq"], d["d_model"]), "W_UQ": q(W["W_UQ"], H * (dh + dr), d["d_cq"]),
                "W_UKT": ukt, "W_UV": q(W["W_UV"], H * dh, dc)}

    def fp8w_workspace(self):
        """Grow the workspace to what mla_decode_fp8w needs for the current split plan."""
        need = L.mla_decode_fp8w_workspace_bytes(self.cdims, self.batch, self.s_q, self.num_splits)
        if need == 0:
            raise ValueError("the FP8-weight decode does not support these dims")
        if self.ws_bytes < need:
            self.ws_bytes = need
            self.ws = torch.empty(need, dtype=torch.uint8, device=self.device)

    def decode_fp8w(self, hq, Wq, softmax_scale, stream=None):
        """The decode step on FP8 weights (Wq from quantize_fp8w): mla_decode_fp8w + mla_combine_fp8w."""
        self.fp8w_workspace()
        L.mla_decode_fp8w(self.cdims, hq, self.batch, self.s_q, Wq["W_DQ"], Wq["W_UQ"], Wq["W_UKT"], self.cache,
                          self.block_table, self.max_pages, self.seqlens, softmax_scale, self.num_splits, self.ws,
                          self.ws_bytes, stream)
        L.mla_combine_fp8w(self.cdims, self.batch, self.s_q, self.num_splits, self.ws, self.ws_bytes, Wq["W_UV"],
                           self.out, self.lse, stream)
        return self.out, self.lse

    # ---------------------------------------------------------------- inspection
    def page_view(self):
        """Raw pages as uint8 [num_pages, page_bytes] (for layout tests)."""
        return self.pages
