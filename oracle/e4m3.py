"""fp8 e4m3 codec written from the format definition (oracle; test only).

The DeepSeek-V2 paper (Chinese translation), section 3.2.3 ("inference
efficiency"), quantises the served KV cache to about 6 bits per element but
does not describe the scheme. The fp8 cache here uses the OCP 8-bit floating
point format E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7,
3 mantissa bits, subnormals when the exponent field is 0, no infinities, and
the single NaN pattern S.1111.111. The largest finite magnitude is
1.75 * 2^8 = 448.
"""

import numpy as np

E4M3_MAX = 448.0


def _value_of(code):
    """Real value of one code (0..255) per the definition."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return np.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3_table():
    """float64 values of all 256 codes (NaN for the two NaN codes)."""
    return np.array([_value_of(c) for c in range(256)], dtype=np.float64)


_TABLE = e4m3_table()
# non-negative finite codes 0x00..0x7E are increasing in value
_POS_VALUES = _TABLE[:0x7F]


def decode_e4m3(codes):
    """Decode an array of uint8 codes to float64."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def encode_e4m3(x):
    """Encode float64 values: round to nearest, ties to even mantissa,
    saturating to +-448 (values beyond the range clamp; NaN stays NaN)."""
    x = np.asarray(x, dtype=np.float64)
    mag = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, mag, side="left")      # first value >= mag
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_hi = _POS_VALUES[hi] - mag
    d_lo = mag - _POS_VALUES[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(mag == _POS_VALUES[hi], hi, code)
    code = code.astype(np.uint8)
    neg = np.signbit(x)
    code = np.where(neg, code | 0x80, code).astype(np.uint8)
    code = np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)
    return code
