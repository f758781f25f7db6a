"""Storage formats used by the codec, written from their definitions.

* FP8 E4M3FN (OCP 8-bit floating point, "fn" = finite, no infinities): 1 sign bit,
  4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes
  subnormals m * 2^-9; S.1111.111 is NaN; the largest finite value is 448.
  References are stored in FP8 (review page, section 2.4 and section 2.5: the
  reference is the value after the storage round trip).
  Encoding is round-to-nearest with ties to the even code, saturating to +-448;
  the sign bit is kept (so -0.0 and negative values that round to zero encode as
  0x80).
* bfloat16: the top 16 bits of an IEEE binary32, round to nearest even.
* fp16: IEEE binary16 (NumPy's float16 cast is round to nearest even).
* Packed codes: INT4 stores two codes per byte, the even coordinate in the low
  nibble; INT2 stores four codes per byte, coordinate 4m + c in bits [2c, 2c+1].
  The pages fix the per-token grouping (section 2.4) but not the bit order; this
  is the order the records use.
"""

from __future__ import annotations

import numpy as np


def _fp8_table() -> np.ndarray:
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = s * m * 2.0 ** -9
        else:
            vals[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


#: value of every FP8 E4M3FN code (index = code byte)
FP8_E4M3FN_VALUES = _fp8_table()
FP8_E4M3FN_MAX = 448.0
# non-negative finite codes 0x00..0x7E in ascending value order
_POS_VALUES = FP8_E4M3FN_VALUES[:0x7F]


def fp8_e4m3fn_decode(codes: np.ndarray) -> np.ndarray:
    """FP8 E4M3FN bytes -> float64 values."""
    return FP8_E4M3FN_VALUES[np.asarray(codes, dtype=np.uint8)]


def fp8_e4m3fn_encode(x: np.ndarray) -> np.ndarray:
    """Round float values to FP8 E4M3FN codes: nearest, ties to even code, saturating."""
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x)
    a = np.abs(x)
    a = np.minimum(a, FP8_E4M3FN_MAX)
    hi = np.searchsorted(_POS_VALUES, a, side="left")  # first value >= a
    hi = np.clip(hi, 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_hi = _POS_VALUES[hi] - a
    d_lo = a - _POS_VALUES[lo]
    pick_hi = d_hi < d_lo
    tie = d_hi == d_lo
    # at an exact tie take the even code
    pick_hi = np.where(tie, (hi % 2) == 0, pick_hi)
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a == 0.0, 0, code).astype(np.uint8)
    code = np.where(sign, code | 0x80, code).astype(np.uint8)
    return code


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest even); returns float32 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def fp16_round(x: np.ndarray) -> np.ndarray:
    """Round to IEEE binary16 (nearest even); returns float64 values."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def pack_codes(q: np.ndarray, bits: int) -> np.ndarray:
    """Pack integer codes [..., d] into bytes [..., d*bits/8]."""
    q = np.asarray(q, dtype=np.uint8)
    if bits == 4:
        lo = q[..., 0::2] & 0xF
        hi = q[..., 1::2] & 0xF
        return (lo | (hi << 4)).astype(np.uint8)
    if bits == 2:
        out = np.zeros(q.shape[:-1] + (q.shape[-1] // 4,), dtype=np.uint8)
        for c in range(4):
            out |= (q[..., c::4] & 0x3) << (2 * c)
        return out
    raise ValueError("bits must be 2 or 4")


def unpack_codes(b: np.ndarray, bits: int) -> np.ndarray:
    """Inverse of pack_codes."""
    b = np.asarray(b, dtype=np.uint8)
    if bits == 4:
        out = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), dtype=np.uint8)
        out[..., 0::2] = b & 0xF
        out[..., 1::2] = b >> 4
        return out
    if bits == 2:
        out = np.empty(b.shape[:-1] + (b.shape[-1] * 4,), dtype=np.uint8)
        for c in range(4):
            out[..., c::4] = (b >> (2 * c)) & 0x3
        return out
    raise ValueError("bits must be 2 or 4")
