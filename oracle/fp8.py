"""FP8 storage of the K/V pool (oracle).  TEST INFRASTRUCTURE ONLY.

The v0.2 handbook's release summary lists FP8 among the precisions the
release was measured in; the pool format taken here is the OCP 8-bit
floating-point format E4M3: 1 sign bit, 4 exponent bits with bias 7, 3
mantissa bits; exponent field 0 holds the subnormals m * 2^-9; there is no
infinity, and S.1111.111 is NaN, so the largest finite magnitude is
1.75 * 2^8 = 448.

Reading taken for the stored value of x with a per-pool scale (the pages give
no scale rule): x is multiplied by the float32 reciprocal of the scale in
float32, and the product is rounded to the nearest E4M3 value, ties to the
even mantissa; magnitudes beyond 448 saturate to 448 and NaN stays NaN.  A
stored code reads back as its E4M3 value times the scale.

The quantizer works by enumeration: it decodes all 256 codes from the
format's definition and picks, for each input, the nearest finite one.
"""

import numpy as np


def e4m3_values():
    """Value of every code 0..255 (float64; NaN for the two NaN codes)."""
    out = np.empty(256, dtype=np.float64)
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            v = np.nan
        elif e == 0:
            v = m * 2.0 ** -9
        else:
            v = (1.0 + m / 8.0) * 2.0 ** (e - 7)
        out[c] = -v if s else v
    return out


_VALUES = e4m3_values()
_POS_CODES = np.arange(0, 0x7F)          # finite non-negative codes, increasing values
_POS_VALUES = _VALUES[_POS_CODES]


def quantize_e4m3(x):
    """Nearest E4M3 code of each value (uint8 array of x's shape)."""
    x = np.asarray(x, dtype=np.float64)
    sign = np.where(np.signbit(x), 0x80, 0).astype(np.uint8)
    a = np.abs(x)
    nan = np.isnan(x)
    a_f = np.where(nan, 0.0, a)
    # candidates: the largest finite value <= a and the smallest >= a
    hi = np.clip(np.searchsorted(_POS_VALUES, a_f), 0, len(_POS_VALUES) - 1)
    lo = np.clip(hi - 1, 0, len(_POS_VALUES) - 1)
    d_lo, d_hi = a_f - _POS_VALUES[lo], _POS_VALUES[hi] - a_f
    exact = _POS_VALUES[hi] == a_f
    even_lo = (_POS_CODES[lo] % 2) == 0
    pick_lo = ~exact & ((d_lo < d_hi) | ((d_lo == d_hi) & even_lo))
    code = np.where(pick_lo, _POS_CODES[lo], _POS_CODES[hi])
    code = np.where(a_f >= _POS_VALUES[-1], _POS_CODES[-1], code)   # saturate
    code = np.where(nan, 0x7F, code)
    return (sign | code.astype(np.uint8)).astype(np.uint8)


def store_codes(rows, scale):
    """Codes stored for rows (any float values) with the pool's scale."""
    inv = np.float32(1.0) / np.float32(scale)
    return quantize_e4m3(np.asarray(rows, dtype=np.float32) * inv)


def dequantize(codes, scale):
    """Values that stored codes stand for (float64)."""
    return _VALUES[np.asarray(codes, dtype=np.int64)] * float(scale)


def kv_store_fp8(pool_codes, new_rows, loc, scale):
    """pool_codes: uint8 [N+1, Hkv, D]; new_rows: [T, Hkv, D]; loc: [T].
    Returns the updated copy (later entries win on repeated slots)."""
    out = np.array(pool_codes, copy=True)
    codes = store_codes(new_rows, scale)
    for t, s in enumerate(np.asarray(loc, dtype=np.int64)):
        out[s] = codes[t]
    return out


def stored_values(rows, scale):
    """What a pool in this format returns for rows written into it."""
    return dequantize(store_codes(rows, scale), scale)
