"""Float64 MLA decode, written out the slow way -- TEST INFRASTRUCTURE ONLY.

What is computed (all arithmetic in float64, numpy; matmul is the only library
primitive used):

* Latents, "Читаем техотчёт DeepSeek-V3 вместе", §2.1.1, KV equations (and
  "Báo cáo Kỹ thuật DeepSeek-V3", Phương pháp item 1):
      c_t^KV = W^DKV h_t            k_t^R = RoPE(W^KR h_t)
* Query side, "Báo cáo Kỹ thuật DeepSeek-V3", Phương pháp item 1 (c^Q) and the
  W_DQ / W_UQ shapes of the attention_params docstring in the V3 practice
  section of the lesson: c^Q = W^DQ h, then W^UQ c^Q gives, per head, a
  content part q^C and a RoPE part q^R.
* Per-head key [k^C_{t,i}; k^R_t] with k^C = W^UK c^KV and value
  v^C = W^UV c^KV, built EXPLICITLY per head (§2.1.1) -- no absorption here.
* Scaled softmax attention over the visible tokens (the pages print the score
  q^T k but not the softmax; the plain reading of "multi-head attention").
* Output projection W^O of the concatenated heads (the W_O shape of the
  attention_params docstring; its result is the u_t of §2.1.2).

`attend_absorbed` is a second, independent route through the same maths (the
absorption of W^UK into the query from §2.1.1 Question 2, and W^UV applied after
the weighted sum of latents by linearity).  It exists only as a pin: the two
routes must agree to rounding.

Conventions that no page fixes (parity unpinned beyond these conventions):
RoPE pairs adjacent channels (2m, 2m+1) with frequency theta^(-2m/d_rope); the
softmax scale tau is a caller argument; W^UQ rows are head-major with
[content d_head | rope d_rope] per head; weights are stored [out, in];
positions are 0-based and query j of a sequence of length L sits at
L - s_q + j and sees tokens 0..L - s_q + j.
"""
import numpy as np


def rope(x, pos, theta):
    """Rotary embedding of the last axis of `x` (length d_rope, even).

    Channel pair (2m, 2m+1) is rotated by angle pos * theta^(-2m/d_rope).
    `pos` broadcasts against x[..., 0] (e.g. shape [n] for x of shape [n, d]
    or [n, H, d] with pos[:, None]).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    assert d % 2 == 0
    m = np.arange(d // 2, dtype=np.float64)
    omega = np.power(float(theta), -2.0 * m / d)            # [d/2]
    ang = np.asarray(pos, dtype=np.float64)[..., None] * omega
    cos, sin = np.cos(ang), np.sin(ang)
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * cos - xo * sin
    out[..., 1::2] = xe * sin + xo * cos
    return out


def kv_latents(h, W_DKV, W_KR, positions, theta):
    """c^KV_t = W^DKV h_t and k^R_t = RoPE(W^KR h_t, t) for every row of h.

    h [n, d_model]; W_DKV [d_c, d_model]; W_KR [d_rope, d_model];
    positions [n] -> (c [n, d_c], kr [n, d_rope]), float64.
    """
    h = np.asarray(h, dtype=np.float64)
    c = h @ np.asarray(W_DKV, dtype=np.float64).T
    kr = rope(h @ np.asarray(W_KR, dtype=np.float64).T, np.asarray(positions), theta)
    return c, kr


def queries(hq, W_DQ, W_UQ, n_heads, d_head, d_rope, positions, theta):
    """Per-head query parts for rows of hq.

    If W_DQ is None, hq already is c^Q [n, d_cq]; otherwise c^Q = W^DQ hq.
    u = W^UQ c^Q is split head-major into [content d_head | rope d_rope]; the
    rope part is rotated at the query's position.
    Returns qc [n, H, d_head], qr [n, H, d_rope].
    """
    hq = np.asarray(hq, dtype=np.float64)
    cq = hq if W_DQ is None else hq @ np.asarray(W_DQ, dtype=np.float64).T
    u = cq @ np.asarray(W_UQ, dtype=np.float64).T
    u = u.reshape(u.shape[0], n_heads, d_head + d_rope)
    qc = u[:, :, :d_head]
    qr = rope(u[:, :, d_head:], np.asarray(positions)[:, None], theta)
    return qc, qr


def softmax_lse(s):
    """Softmax along the last axis and its log-sum-exp, max-shifted.

    An empty last axis gives an empty p and lse = -inf.
    """
    s = np.asarray(s, dtype=np.float64)
    if s.shape[-1] == 0:
        return s.copy(), np.full(s.shape[:-1], -np.inf)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=-1, keepdims=True)
    return e / z, (m + np.log(z))[..., 0]


def attend_nonabsorbed(qc, qr, c, kr, W_UK, W_UV, d_head, tau, heads=None):
    """One query token attending over T visible cached tokens, per head.

    qc [H, d_head], qr [H, d_rope]: this query's parts (qr already rotated).
    c [T, d_c], kr [T, d_rope]: the visible latents (kr already rotated).
    For each head i: k^C_{t,i} = W^UK_i c_t and v^C_{t,i} = W^UV_i c_t, built
    explicitly; key_{t,i} = [k^C_{t,i}; k^R_t]; score = tau * q_i . key_{t,i};
    p = softmax(score over t); o_i = sum_t p_t v^C_{t,i}.
    `heads` selects a subset of head indices (default all).
    Returns (o [h, d_head], p [h, T], lse [h]).
    """
    c = np.asarray(c, dtype=np.float64)
    kr = np.asarray(kr, dtype=np.float64)
    W_UK = np.asarray(W_UK, dtype=np.float64)
    W_UV = np.asarray(W_UV, dtype=np.float64)
    H = qc.shape[0]
    heads = list(range(H)) if heads is None else list(heads)
    T = c.shape[0]
    o = np.zeros((len(heads), d_head))
    p_all = np.zeros((len(heads), T))
    lse = np.zeros(len(heads))
    for n, i in enumerate(heads):
        W_UK_i = W_UK[i * d_head:(i + 1) * d_head]       # [d_head, d_c]
        W_UV_i = W_UV[i * d_head:(i + 1) * d_head]
        kC = c @ W_UK_i.T                                 # [T, d_head]
        vC = c @ W_UV_i.T                                 # [T, d_head]
        key = np.concatenate([kC, kr], axis=1)            # [T, d_head + d_rope]
        q = np.concatenate([qc[i], qr[i]])                # [d_head + d_rope]
        s = tau * (key @ q)                               # [T]
        p, lse[n] = softmax_lse(s)
        p_all[n] = p
        o[n] = p @ vC if T > 0 else 0.0
    return o, p_all, lse


def attend_absorbed(qc, qr, c, kr, W_UK, W_UV, d_head, tau):
    """The same attention with W^UK folded into the query and W^UV applied
    after the softmax-weighted sum of latents (§2.1.1 Question 2; linearity
    of v^C = W^UV c^KV).  A second route used only to pin the first.
    """
    c = np.asarray(c, dtype=np.float64)
    kr = np.asarray(kr, dtype=np.float64)
    W_UK = np.asarray(W_UK, dtype=np.float64)
    W_UV = np.asarray(W_UV, dtype=np.float64)
    H = qc.shape[0]
    d_c = c.shape[1]
    o = np.zeros((H, d_head))
    lse = np.zeros(H)
    for i in range(H):
        W_UK_i = W_UK[i * d_head:(i + 1) * d_head]
        W_UV_i = W_UV[i * d_head:(i + 1) * d_head]
        q_abs = W_UK_i.T @ qc[i]                          # [d_c]: q^T W^UK once
        s = tau * (c @ q_abs + kr @ qr[i])
        p, lse[i] = softmax_lse(s)
        o_lat = p @ c if c.shape[0] > 0 else np.zeros(d_c)
        o[i] = W_UV_i @ o_lat
    return o, lse


def decode_from_latents(c, kr, hq, W_DQ, W_UQ, W_UK, W_UV, dims, seqlen, s_q,
                        tau, heads=None):
    """Decode s_q query tokens of one sequence from its cached latents.

    c [>=seqlen, d_c], kr [>=seqlen, d_rope]: latents of tokens 0..seqlen-1.
    hq [s_q, d_model] (or c^Q [s_q, d_cq] when W_DQ is None): the hidden
    states of the last s_q tokens, which sit at positions seqlen-s_q+j.
    dims: dict with n_heads, d_head, d_rope, rope_theta.
    Query j sees tokens 0..seqlen-s_q+j (causal).
    Returns o [s_q, h, d_head], lse [s_q, h].
    """
    H, dh, dr = dims["n_heads"], dims["d_head"], dims["d_rope"]
    pos_q = np.arange(seqlen - s_q, seqlen)
    qc, qr = queries(hq, W_DQ, W_UQ, H, dh, dr, pos_q, dims["rope_theta"])
    nh = H if heads is None else len(list(heads))
    o = np.zeros((s_q, nh, dh))
    lse = np.zeros((s_q, nh))
    for j in range(s_q):
        vis = max(0, seqlen - s_q + j + 1)
        o[j], _, lse[j] = attend_nonabsorbed(qc[j], qr[j], c[:vis], kr[:vis],
                                             W_UK, W_UV, dh, tau, heads)
    return o, lse


def decode_from_h(h, W, dims, seqlen, s_q, tau, heads=None, chunk=4096):
    """End-to-end decode of one sequence from its hidden states.

    h [seqlen, d_model]: hidden states of tokens 0..seqlen-1 (the last s_q
    rows are the queries).  W: dict of W_DKV, W_KR, W_DQ, W_UQ, W_UK, W_UV.
    Latents are computed chunk by chunk (memory only; the arithmetic is the
    same as one call).  Returns o [s_q, h, d_head], lse [s_q, h].
    """
    d_c, d_r = dims["d_c"], dims["d_rope"]
    c = np.zeros((seqlen, d_c))
    kr = np.zeros((seqlen, d_r))
    for t0 in range(0, seqlen, chunk):
        t1 = min(seqlen, t0 + chunk)
        c[t0:t1], kr[t0:t1] = kv_latents(h[t0:t1], W["W_DKV"], W["W_KR"],
                                         np.arange(t0, t1), dims["rope_theta"])
    hq = np.asarray(h[seqlen - s_q:seqlen], dtype=np.float64)
    return decode_from_latents(c, kr, hq, W.get("W_DQ"), W["W_UQ"], W["W_UK"],
                               W["W_UV"], dims, seqlen, s_q, tau, heads)


def output_projection(o, W_O):
    """Attention output of the layer for rows of per-head outputs.

    o has shape [R, H, d_head]; W_O is stored [out, in] = [d_model,
    H * d_head] (the practice section's attention_params docstring gives W_O
    as heads*d_head x d).  The heads of a row are concatenated in head order,
    d_head innermost, and projected: y_r = W^O [o_{r,1}; ...; o_{r,H}]
    (shape [R, d_model]).  This is the u_t that the MoE layer of §2.1.2
    takes as input; no residual or norm is printed, so none is added.
    """
    o = np.asarray(o, dtype=np.float64)
    R = o.shape[0]
    cat = o.reshape(R, -1)
    return cat @ np.asarray(W_O, dtype=np.float64).T
