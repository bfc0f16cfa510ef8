"""FP8 KV rows (oracle side): OCP E4M3 codes with one power-of-two scale per row.

[tokendh] section "历史太长,会撑爆什么" names KV quantization as the fourth way
to shrink the history: values are kept at lower precision together with the
parameters needed to restore them; [jetabc] notes that the evaluated model
already runs in FP8.  The pages give no format, so the reading taken here is
the plainest one that keeps attention exact over what is stored:

  * element format: OCP 8-bit floating point E4M3 (1 sign, 4 exponent bits with
    bias 7, 3 mantissa bits; no infinities; the all-ones exponent with all-ones
    mantissa is NaN; largest finite magnitude 448; subnormals m * 2^-9);
  * one scale per stored row (one token of one KV head): a power of two 2^e,
    kept as the biased byte e + 127 (the E8M0 scale encoding of the OCP
    microscaling formats), with e the smallest exponent >= -126 for which
    every |x| * 2^-e of the row is at most 448 (e = 0 for an all-zero row; the
    bound keeps every scale a normal float32);
  * a code is x * 2^-e rounded to the nearest E4M3 value, ties to the even
    code; the stored value is code * 2^e, exact in bf16 and fp32;
  * attention, page metadata and selection read the stored values (the
    dequantized rows), so the FP8 path is the bf16 path over those values.
"""
import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(code):
    """Value of one E4M3 code (0..255) as a Python float (NaN for the NaN codes)."""
    code = int(code)
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


DECODE = np.array([e4m3_decode(c) for c in range(256)], np.float64)


def e4m3_encode(y):
    """Nearest E4M3 code of a finite float with |y| <= 448, ties to the even code."""
    y = float(y)
    assert abs(y) <= E4M3_MAX and y == y
    sign = 0x80 if (y < 0 or (y == 0 and np.signbit(y))) else 0
    a = abs(y)
    best = None
    for c in range(0x7F):                       # every non-negative finite code, ascending value
        d = abs(DECODE[c] - a)
        if best is None or d < best[0] or (d == best[0] and (c & 1) == 0 and (best[1] & 1) == 1):
            best = (d, c)
    return sign | best[1]


def e4m3_encode_array(y):
    """Vectorised e4m3_encode: the nearest of the two finite codes around each |y|
    (from the ascending table of non-negative values), ties to the even code."""
    y = np.asarray(y, np.float64)
    assert np.all(np.abs(y) <= E4M3_MAX) and not np.any(np.isnan(y))
    pos = DECODE[:0x7F]                                    # codes 0x00..0x7e, ascending values
    a = np.abs(y)
    hi = np.clip(np.searchsorted(pos, a, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    dlo, dhi = a - pos[lo], pos[hi] - a
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(a == pos[hi], hi, pick)                # exact hits (also a == 0)
    sign = np.where(np.signbit(y), 0x80, 0)
    return (sign | pick).astype(np.uint8)


def row_exponent(amax):
    """Smallest e >= -126 with amax * 2^-e <= 448 (0 when amax is 0)."""
    amax = float(amax)
    if amax == 0.0:
        return 0
    e = int(np.floor(np.log2(amax))) - 9
    while amax * 2.0 ** -e > E4M3_MAX:
        e += 1
    while e > -126 and amax * 2.0 ** -(e - 1) <= E4M3_MAX:
        e -= 1
    return max(e, -126)


def quantize_rows(X):
    """X [..., d] (float values) -> (codes uint8 [..., d], scale bytes uint8 [...] = e + 127)."""
    X = np.asarray(X, np.float64)
    flat = X.reshape(-1, X.shape[-1])
    e = np.array([row_exponent(v) for v in np.abs(flat).max(axis=1)], np.int64)
    codes = e4m3_encode_array(flat * np.exp2(-e.astype(np.float64))[:, None])
    return codes.reshape(X.shape), (e + 127).astype(np.uint8).reshape(X.shape[:-1])


def dequantize_rows(codes, sbytes):
    """Stored values: DECODE[code] * 2^(scale byte - 127), float64 [..., d]."""
    codes = np.asarray(codes, np.uint8)
    e = np.asarray(sbytes, np.int64) - 127
    return DECODE[codes] * np.exp2(e.astype(np.float64))[..., None]
