"""Exact widening of stored KV elements to float64, and the OCP E4M3 codec.

Test infrastructure only (see the package docstring).

The pages say only that an fp8 KV cache "halves the cache and the bytes read per
step" ("Serving: vLLM and PagedAttention", section 3.1, the ``kv_cache_dtype``
knob; "PagedAttention" daily term, "Cons": KV quantisation as a bandwidth
lever). The format is not given there; the reading taken is OCP 8-bit
floating point, E4M3 variant ("fn": no infinities, a single NaN mantissa),
written here from that format's definition:

* sign s (bit 7), exponent e (bits 6..3, bias 7), mantissa m (bits 2..0);
* e == 0:            value = (-1)^s * 2^-6 * (m / 8)        (subnormal, incl. +-0)
* e == 15 and m == 7: NaN
* otherwise:         value = (-1)^s * 2^(e - 7) * (1 + m / 8)
* largest finite magnitude 448 (code 0x7E); no infinities.

Encoding (float -> code) is round-to-nearest, ties to the code whose mantissa
LSB is 0, with saturation: any |y| > 448, infinities included, becomes +-448;
NaN becomes 0x7F with the sign bit kept; the sign of zero is kept.

bf16 is the upper half of an IEEE binary32, so widening is exact: place the 16
stored bits in the high half of a 32-bit word, read it as float32, then widen.
"""

import numpy as np


def bf16_bits_to_f64(bits):
    """uint16 bf16 bit patterns -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f32_to_f64(x):
    """float32 -> float64 (exact)."""
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def e4m3_value_table():
    """float64[256]: the value of every E4M3 code, straight from the definition."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = (code >> 7) & 1
        e = (code >> 3) & 0xF
        m = code & 0x7
        sign = -1.0 if s else 1.0
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = sign * (2.0 ** -6) * (m / 8.0)
        else:
            vals[code] = sign * (2.0 ** (e - 7)) * (1.0 + m / 8.0)
    return vals


_TABLE = e4m3_value_table()
# Non-negative finite codes 0x00..0x7E have strictly increasing values.
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = _TABLE[:0x7F]
E4M3_MAX = 448.0


def e4m3_decode(codes):
    """uint8 codes -> float64 values (exact; 0x7F / 0xFF -> NaN)."""
    return _TABLE[np.asarray(codes, dtype=np.uint8).astype(np.int64)]


def e4m3_encode(y):
    """float values -> uint8 E4M3 codes (nearest, ties to even, saturating).

    ``y`` is taken as given (float32 or float64); the comparison is done in
    float64, where every float32 input and every midpoint between adjacent
    E4M3 values is exact, so the rounding decision is exact.
    """
    y = np.asarray(y, dtype=np.float64)
    flat = y.reshape(-1)
    sign = np.signbit(flat)
    mag = np.abs(flat)
    out = np.zeros(flat.shape, dtype=np.int64)

    nan = np.isnan(flat)
    sat = ~nan & (mag > E4M3_MAX)
    reg = ~nan & ~sat

    m = mag[reg]
    hi = np.searchsorted(_POS_VALUES, m, side="left")      # first value >= m
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = m - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - m
    exact = _POS_VALUES[hi] == m
    pick_hi = exact | (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    out[reg] = code
    out[sat] = 0x7E
    out[nan] = 0x7F
    out = out | np.where(sign, 0x80, 0)
    return out.astype(np.uint8).reshape(y.shape)
