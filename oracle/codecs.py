"""Value codecs for the storage formats the path uses.

TEST INFRASTRUCTURE ONLY (see the package docstring).

bf16: the top 16 bits of an IEEE binary32.  Decoding is a shift.
e4m3: the OCP 8-bit floating point "E4M3FN" format: 1 sign bit, 4 exponent
bits with bias 7, 3 mantissa bits, subnormals when the exponent field is 0,
no infinities, and the two codes with all exponent and mantissa bits set
(0x7F, 0xFF) are NaN.  The largest finite magnitude is 448 (code 0x7E).

The indexer-cache dtype follows attention quantisation: an FP8 cache when
attention runs in FP8, else the model dtype (GLM5 TensorCast adaptation
design, section "KV cache dtype and parallel-linear boundary fix"; the FP8
path's "FP8 key cache / scale cache write" in section "DSA Indexer fused
semantic op").  Which FP8 variant is not stated on the pages; OCP e4m3fn is
the reading taken here because it is the FP8 format the target hardware's
conversion instructions implement.

The encoder is written as "nearest representable value" over the full value
table, so that it shares nothing with a bit-manipulation encoder.
"""

import numpy as np

E4M3_MAX = 448.0


def bf16_to_f64(bits):
    """bf16 bit patterns (uint16 / int16 array) -> exact float64 values."""
    u = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def e4m3_value(code):
    """Value of one e4m3fn code (0..255) from the format definition."""
    code = int(code)
    sign = -1.0 if code & 0x80 else 1.0
    exp_field = (code >> 3) & 0xF
    man_field = code & 0x7
    if exp_field == 0xF and man_field == 0x7:
        return float("nan")
    if exp_field == 0:
        mag = (man_field / 8.0) * 2.0 ** (1 - 7)          # subnormal
    else:
        mag = (1.0 + man_field / 8.0) * 2.0 ** (exp_field - 7)
    return sign * mag


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_to_f64(codes):
    """e4m3fn codes (uint8 array) -> float64 values."""
    return E4M3_TABLE[np.asarray(codes).astype(np.uint8)]


# Non-negative finite magnitudes, in code order 0x00..0x7E (monotone).
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = E4M3_TABLE[:0x7F]


def f32_to_e4m3(x):
    """Round float32 values to e4m3fn codes: nearest value, ties to the even
    code (even mantissa), magnitudes at or beyond 448 saturate to 448, the
    sign is kept (so a negative value that rounds to zero gives 0x80).

    NaN inputs are not supported by the path and are rejected here.
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    if np.isnan(x).any():
        raise ValueError("NaN has no e4m3 encoding on this path")
    mag = np.minimum(np.abs(x), E4M3_MAX)
    # index of the first table value >= mag
    hi = np.searchsorted(_POS_VALUES, mag, side="left")
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    code = np.where(mag == _POS_VALUES[hi], _POS_CODES[hi], code)
    neg = np.signbit(x)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)
