"""Seeded synthetic inputs for the MLA decode workloads.

This module holds no MLA arithmetic: it only draws random numbers, rounds them
to the storage dtype and lays out sequence lengths and block tables.  Both the
GPU path (through the C ABI) and the float64 oracle consume what it produces,
so the two sides always see identical input values.

Every tensor is drawn from its own torch.Generator whose seed is derived from
(seed, workload, tensor, sequence, block), so any part of any sequence can be
regenerated independently of the rest (hidden states come in blocks of
H_BLOCK tokens).  Values are drawn in float32 and rounded once to the
workload's dtype (round-to-nearest-even for bf16); the oracle upcasts those
exact values.
"""
import numpy as np
import torch

H_BLOCK = 4096

TINY_DIMS = dict(d_model=256, n_heads=4, d_head=32, d_rope=16, d_c=64, d_cq=96, page_size=64, rope_theta=10000.0)
V3_DIMS = dict(d_model=7168, n_heads=128, d_head=128, d_rope=64, d_c=512, d_cq=1536, page_size=64,
               rope_theta=10000.0)

# The decode workloads: a tiny float32 one, then DeepSeek-V3 shapes.
WORKLOADS = {
    "tiny_f32_b2_l256": dict(index=0, dims=TINY_DIMS, act="f32", cache="f32", batch=2, s_q=1,
                             lengths=("fixed", 256), table="inorder", sigma=0.02),
    "v3_bf16_b64_l4096": dict(index=1, dims=V3_DIMS, act="bf16", cache="bf16", batch=64, s_q=1,
                              lengths=("fixed", 4096), table="inorder", sigma=0.006),
    "v3_bf16_b128_var32k_paged": dict(index=2, dims=V3_DIMS, act="bf16", cache="bf16", batch=128, s_q=1,
                                      lengths=("uniform", 1, 32768), table="shuffled", sigma=0.006),
    "v3_bf16_b4_l128k": dict(index=3, dims=V3_DIMS, act="bf16", cache="bf16", batch=4, s_q=1,
                             lengths=("fixed", 131072), table="inorder", sigma=0.006),
    "v3_fp8_b128_l8192_sq2": dict(index=4, dims=V3_DIMS, act="bf16", cache="fp8", batch=128, s_q=2,
                                  lengths=("fixed", 8192), table="inorder", sigma=0.006),
    # the inputs of v3_fp8_b128_l8192_sq2 (the same index, so the same values) in the FP8 cache
    # format with power-of-two (UE8M0) tile scales
    "v3_fp8e8_b128_l8192_sq2": dict(index=4, dims=V3_DIMS, act="bf16", cache="fp8e8", batch=128, s_q=2,
                                    lengths=("fixed", 8192), table="inorder", sigma=0.006),
    # the headline batch with W^DQ, W^UQ, W^UK and W^UV in E4M3 (128 x 128-block scales)
    "v3_fp8w_b64_l4096": dict(index=11, dims=V3_DIMS, act="bf16", cache="bf16", batch=64, s_q=1,
                              lengths=("fixed", 4096), table="inorder", sigma=0.006, weights="fp8"),
    # speculative verify of three chained MTP drafts (s_q = 1 + 3)
    "v3_bf16_b64_l4096_sq4": dict(index=6, dims=V3_DIMS, act="bf16", cache="bf16", batch=64, s_q=4,
                                  lengths=("fixed", 4096), table="inorder", sigma=0.006),
}

# Decode through a stack of attention layers, each with its own cache and
# weights (W^O included): the per-layer cache of the whole model.
LAYER_WORKLOADS = {
    "v3_bf16_b64_l4096_61layers": dict(index=8, dims=V3_DIMS, act="bf16", cache="bf16", batch=64, s_q=1,
                                       lengths=("fixed", 4096), table="inorder", sigma=0.006, layers=61),
}

# FP8 block-scaled projections (mla_fp8_gemm) at decode row counts: every
# MLA weight of one layer, W^O included, as (name, N, K).
FP8_PROJECTIONS = (("W_DKV", 512, 7168), ("W_KR", 64, 7168), ("W_DQ", 1536, 7168), ("W_UQ", 24576, 1536),
                   ("W_UK", 16384, 512), ("W_UV", 16384, 512), ("W_O", 7168, 16384))
FP8_WORKLOADS = {
    "fp8_proj_v3_r64": dict(index=10, rows=64, sigma=0.006),
}

# Prefill of fresh sequences (mla_prefill): batch sequences of the given lengths, packed.
PREFILL_WORKLOADS = {
    "prefill_v3_bf16_b4_l4096": dict(index=5, dims=V3_DIMS, act="bf16", batch=4, lengths=("fixed", 4096),
                                     sigma=0.006),
}

TENSORS = {"W_DKV": 1, "W_KR": 2, "W_DQ": 3, "W_UQ": 4, "W_UK": 5, "W_UV": 6, "h": 7, "len": 8, "table": 9,
           "latent": 10, "rope": 11, "W_O": 12, "o": 13, "gemm_x": 14, "gemm_w": 15}


def seed_of(seed, workload_index, tensor, b=0, block=0):
    ss = np.random.SeedSequence([int(seed), int(workload_index), TENSORS[tensor], int(b), int(block)])
    return int(ss.generate_state(1, np.uint64)[0] & np.uint64(0x7FFFFFFFFFFFFFFF))


def torch_dtype(name):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def weight_shapes(d):
    H, dh, dr = d["n_heads"], d["d_head"], d["d_rope"]
    return {
        "W_DKV": (d["d_c"], d["d_model"]),
        "W_KR": (dr, d["d_model"]),
        "W_DQ": (d["d_cq"], d["d_model"]),
        "W_UQ": (H * (dh + dr), d["d_cq"]),
        "W_UK": (H * dh, d["d_c"]),
        "W_UV": (H * dh, d["d_c"]),
    }


def normal(shape, std, seed, device, dtype):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def weights(dims, sigma, dtype, device, seed=0, workload_index=0):
    """Weights N(0, sigma^2), stored [out, in] in `dtype`."""
    return {k: normal(s, sigma, seed_of(seed, workload_index, k), device, dtype)
            for k, s in weight_shapes(dims).items()}


def out_weight(dims, sigma, dtype, device, seed=0, workload_index=0):
    """W^O ~ N(0, sigma^2), stored [out, in] = [d_model, n_heads * d_head]."""
    shape = (dims["d_model"], dims["n_heads"] * dims["d_head"])
    return normal(shape, sigma, seed_of(seed, workload_index, "W_O"), device, dtype)


def head_outputs(dims, rows, std, dtype, device, seed=0, workload_index=0):
    """Per-head attention outputs o ~ N(0, std^2), [rows, n_heads, d_head]."""
    shape = (rows, dims["n_heads"], dims["d_head"])
    return normal(shape, std, seed_of(seed, workload_index, "o"), device, dtype)


def gemm_operands(M, N, K, sigma, dtype, device, seed=0, workload_index=0):
    """A projection's activations X ~ N(0, 1) [M, K] and weight W ~ N(0,
    sigma^2) [N, K] (stored [out, in])."""
    X = normal((M, K), 1.0, seed_of(seed, workload_index, "gemm_x", N, K), device, dtype)
    W = normal((N, K), sigma, seed_of(seed, workload_index, "gemm_w", N, K), device, dtype)
    return X, W


def hidden(dims, b, t0, t1, dtype, device, seed=0, workload_index=0):
    """Hidden states h of tokens t0..t1-1 of sequence b, N(0, 1), [t1-t0, d_model]."""
    out = torch.empty((t1 - t0, dims["d_model"]), dtype=dtype, device=device)
    k0, k1 = t0 // H_BLOCK, (t1 - 1) // H_BLOCK if t1 > t0 else t0 // H_BLOCK - 1
    for k in range(k0, k1 + 1):
        blk = normal((H_BLOCK, dims["d_model"]), 1.0, seed_of(seed, workload_index, "h", b, k), device, dtype)
        a, z = max(t0, k * H_BLOCK), min(t1, (k + 1) * H_BLOCK)
        out[a - t0:z - t0] = blk[a - k * H_BLOCK:z - k * H_BLOCK]
    return out


def latents(dims, n, std_c, std_r, dtype, device, seed=0, workload_index=0, b=0):
    """Directly planted cache rows: c^KV ~ N(0, std_c^2) [n, d_c] and an
    already-rotated k^R ~ N(0, std_r^2) [n, d_rope]."""
    c = normal((n, dims["d_c"]), std_c, seed_of(seed, workload_index, "latent", b), device, dtype)
    r = normal((n, dims["d_rope"]), std_r, seed_of(seed, workload_index, "rope", b), device, dtype)
    return c, r


def seqlens(spec, batch, seed=0, workload_index=0):
    """int64 numpy lengths: ('fixed', L) or ('uniform', lo, hi) inclusive integers."""
    if spec[0] == "fixed":
        return np.full(batch, spec[1], dtype=np.int64)
    rng = np.random.default_rng(seed_of(seed, workload_index, "len"))
    return rng.integers(spec[1], spec[2] + 1, size=batch).astype(np.int64)


def block_table(lengths, page_size, kind, seed=0, workload_index=0):
    """int32 numpy [batch, max_pages] table and the pool size.  'inorder' gives
    sequence b consecutive pages after those of b-1; 'shuffled' hands out a
    random permutation of the pool.  Unused entries hold page 0."""
    npages = [(int(L) + page_size - 1) // page_size for L in lengths]
    max_pages = max(1, max(npages))
    pool = sum(npages)
    ids = np.arange(pool, dtype=np.int64)
    if kind == "shuffled":
        ids = np.random.default_rng(seed_of(seed, workload_index, "table")).permutation(pool)
    bt = np.zeros((len(lengths), max_pages), dtype=np.int32)
    o = 0
    for b, n in enumerate(npages):
        bt[b, :n] = ids[o:o + n]
        o += n
    return bt, max(pool, 1)


def sample_sequences(lengths, k, seed=0, workload_index=0):
    """k seeded sequence indices, always including the shortest and longest."""
    B = len(lengths)
    if k >= B:
        return list(range(B))
    rng = np.random.default_rng(seed_of(seed, workload_index, "len", 1))
    pick = {int(np.argmin(lengths)), int(np.argmax(lengths))}
    for b in rng.permutation(B):
        if len(pick) >= k:
            break
        pick.add(int(b))
    return sorted(pick)
