"""FP8 codecs and 1x128 tile quantisation, float64 -- TEST INFRASTRUCTURE ONLY.

Source: "Читаем техотчёт DeepSeek-V3 вместе", §3.3 "Обучение в FP8": the FP8
glossary entry gives the two formats by their largest values (E4M3 up to 448,
E5M2 up to 57 344); item 2 gives one scale per 1x128 activation tile; item 4
says one format, E4M3, serves all tensors.  The 448 maximum fixes the OCP
"E4M3FN" variant: exponent bias 7, no infinities, only S.1111.111 is NaN.

The codec is built from the format definition: every code is decoded by its
bit fields, and encoding is "nearest representable value, ties to the code
with an even mantissa, saturate at +-448" by search over the decoded table.

Block quantisation of weights (item 2: 128 x 128 blocks) applies the same
rule to each block; the block-scaled GEMM (items 2-3) multiplies the
dequantised activations (1 x 128 tiles) and weights.

Tile quantisation (a reading of item 2 for the latent cache): for each token
and each group of 128 consecutive channels, scale s = amax/448 computed in
float32 (s = 1 when amax = 0), code = encode(float32(x) / s) in float32, and the
dequantised value is code * s.  Both sides decide codes in float32.

Power-of-two tile scales (UE8M0): the lesson's continuation of §3.5 notes that
DeepSeek V3.1 moved to FP8 with UE8M0 scales, i.e. scales that are bare powers
of two (an 8-bit exponent, no mantissa).  Reading used here for that cache
format: the scale is the smallest power of two not below amax/448 (the
float32 quotient), and not below 2^-126, so that no code saturates; codes
follow the same rule as above.  Every dequantised value code * scale is then
exactly representable in bfloat16 (and float32) within the normal range.
"""
import numpy as np

E4M3_MAX = 448.0
E5M2_MAX = 57344.0


def e4m3_decode(code):
    """Value of E4M3FN code(s) 0..255 (NaN for 0x7F / 0xFF)."""
    code = np.asarray(code, dtype=np.int64)
    sign = np.where(code & 0x80, -1.0, 1.0)
    e = (code >> 3) & 0xF
    m = code & 0x7
    val = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.power(2.0, e - 7.0))
    val = np.where((e == 0xF) & (m == 0x7), np.nan, val)
    return sign * val


def e5m2_decode(code):
    """Value of E5M2 code(s) 0..255 (IEEE-like: bias 15, inf and NaN at e=31)."""
    code = np.asarray(code, dtype=np.int64)
    sign = np.where(code & 0x80, -1.0, 1.0)
    e = (code >> 2) & 0x1F
    m = code & 0x3
    val = np.where(e == 0, (m / 4.0) * 2.0 ** -14, (1.0 + m / 4.0) * np.power(2.0, e - 15.0))
    val = np.where(e == 0x1F, np.where(m == 0, np.inf, np.nan), val)
    return sign * val


def e4m3_values():
    """Sorted finite non-negative E4M3FN values with their codes."""
    codes = np.arange(0, 0x7F)             # 0x00..0x7E; 0x7F is NaN
    return e4m3_decode(codes), codes


def e4m3_encode(x):
    """Round x to the nearest E4M3FN code, ties to even mantissa, saturating.

    Works on float64 copies of x; NaN is not expected (the inputs are finite).
    """
    x = np.asarray(x, dtype=np.float64)
    vals, codes = e4m3_values()
    a = np.minimum(np.abs(x), E4M3_MAX).ravel()
    idx = np.searchsorted(vals, a)                     # vals[idx-1] < a <= vals[idx]
    idx = np.clip(idx, 1, len(vals) - 1)
    lo, hi = vals[idx - 1], vals[idx]
    dlo, dhi = a - lo, hi - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (codes[idx] % 2 == 0))
    out = np.where(pick_hi, codes[idx], codes[idx - 1])
    out = np.where(a == 0.0, 0, out)
    out = np.where(x.ravel() < 0, out | 0x80, out)
    return out.reshape(x.shape).astype(np.uint8)


def pow2_ceil(s):
    """Smallest power of two >= s for positive float32 s, at least 2^-126."""
    s = np.asarray(s, dtype=np.float32).astype(np.float64)
    m, e = np.frexp(s)                       # s = m 2^e with m in [0.5, 1)
    p = np.where(m == 0.5, np.ldexp(1.0, e - 1), np.ldexp(1.0, e))
    return np.maximum(p, 2.0 ** -126).astype(np.float32)


def quantize_tiles(x, tile=128, scale_rule="amax"):
    """Per-row, per-`tile`-channel E4M3 quantisation of x [n, d] (d % tile == 0).

    scale_rule "amax": s = amax/448; "ue8m0": s = the power of two above (see
    the module docstring).  Returns (codes uint8 [n, d], scales float32
    [n, d // tile]).
    """
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    n, d = x32.shape
    assert d % tile == 0 and scale_rule in ("amax", "ue8m0")
    g = x32.reshape(n, d // tile, tile)
    amax = np.abs(g).max(axis=2)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    if scale_rule == "ue8m0":
        scale = np.where(amax > 0, pow2_ceil(np.where(amax > 0, scale, 1.0)), np.float32(1.0)).astype(np.float32)
    y = (g / scale[:, :, None]).astype(np.float32)
    codes = e4m3_encode(y.astype(np.float64)).reshape(n, d)
    return codes, scale


def dequantize_tiles(codes, scales, tile=128):
    """codes [n, d] uint8, scales [n, d // tile] -> float64 values code * scale."""
    n, d = codes.shape
    v = e4m3_decode(codes).reshape(n, d // tile, tile)
    return (v * np.asarray(scales, dtype=np.float64)[:, :, None]).reshape(n, d)


def quantize_blocks(w, block=128):
    """Per-block E4M3 quantisation of a weight w [n, k] (k % block == 0):
    one scale per block x block block (§3.3 item 2: weights in 128 x 128
    blocks, each group with its own scale), the last row-block cut short when
    n % block != 0.  The rule inside a block is the tile rule above: s =
    amax/448 in float32 (1 for an all-zero block), code = encode(float32(x) /
    s).

    Returns (codes uint8 [n, k], scales float32 [ceil(n / block), k / block]).
    """
    w32 = np.asarray(w, dtype=np.float64).astype(np.float32)
    n, k = w32.shape
    assert k % block == 0
    nb, kb = -(-n // block), k // block
    codes = np.zeros((n, k), dtype=np.uint8)
    scales = np.zeros((nb, kb), dtype=np.float32)
    for i in range(nb):
        for j in range(kb):
            blk = w32[i * block:(i + 1) * block, j * block:(j + 1) * block]
            amax = np.float32(np.abs(blk).max())
            s = amax / np.float32(E4M3_MAX) if amax > 0 else np.float32(1.0)
            scales[i, j] = s
            codes[i * block:(i + 1) * block, j * block:(j + 1) * block] = e4m3_encode(
                (blk / s).astype(np.float32).astype(np.float64))
    return codes, scales


def dequantize_blocks(codes, scales, block=128):
    """codes [n, k] uint8, scales [ceil(n / block), k / block] -> float64 code * scale."""
    n, k = codes.shape
    s = np.repeat(np.repeat(np.asarray(scales, dtype=np.float64), block, 0)[:n], block, 1)
    return e4m3_decode(codes) * s


def gemm_block_scaled(x, w_codes, w_scales, block=128):
    """Y = Q(x) . Q(w)^T of the pages' FP8 GEMM (§3.3 items 2-3): the
    activations x [m, k] quantised in 1 x 128 tiles, the weight given as
    128 x 128-block codes and scales, the product of the dequantised values
    summed exactly (float64).  The per-128 promotion of item 3 is how a
    device keeps this sum accurate; in exact arithmetic it is this sum.

    Returns (y float64 [m, n], x_codes, x_scales)."""
    xc, xs = quantize_tiles(x, block)
    xq = dequantize_tiles(xc, xs, block)
    wq = dequantize_blocks(w_codes, w_scales, block)
    return xq @ wq.T, xc, xs
