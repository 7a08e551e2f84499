"""FP8 codecs and 1x128 tile quantisation, float64 -- TEST INFRASTRUCTURE ONLY.

Source: "Читаем техотчёт DeepSeek-V3 вместе", §3.3 "Обучение в FP8": the FP8
glossary entry gives the two formats by their largest values (E4M3 up to 448,
E5M2 up to 57 344); item 2 gives one scale per 1x128 activation tile; item 4
says one format, E4M3, serves all tensors.  The 448 maximum fixes the OCP
"E4M3FN" variant: exponent bias 7, no infinities, only S.1111.111 is NaN.

The codec is built from the format definition: every code is decoded by its
bit fields, and encoding is "nearest representable value, ties to the code
with an even mantissa, saturate at +-448" by search over the decoded table.

Tile quantisation (a reading of item 2 for the latent cache): for each token
and each group of 128 consecutive channels, scale s = amax/448 computed in
float32 (s = 1 when amax = 0), code = encode(float32(x) / s) in float32, and the
dequantised value is code * s.  Both sides decide codes in float32.
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


def quantize_tiles(x, tile=128):
    """Per-row, per-`tile`-channel E4M3 quantisation of x [n, d] (d % tile == 0).

    Returns (codes uint8 [n, d], scales float32 [n, d // tile]).
    """
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    n, d = x32.shape
    assert d % tile == 0
    g = x32.reshape(n, d // tile, tile)
    amax = np.abs(g).max(axis=2)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    y = (g / scale[:, :, None]).astype(np.float32)
    codes = e4m3_encode(y.astype(np.float64)).reshape(n, d)
    return codes, scale


def dequantize_tiles(codes, scales, tile=128):
    """codes [n, d] uint8, scales [n, d // tile] -> float64 values code * scale."""
    n, d = codes.shape
    v = e4m3_decode(codes).reshape(n, d // tile, tile)
    return (v * np.asarray(scales, dtype=np.float64)[:, :, None]).reshape(n, d)
