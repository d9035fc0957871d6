"""fp8 e4m3 codec for a quantized KV cache -- TEST INFRASTRUCTURE ONLY.

The pages name KV-cache quantization as the way to shrink KV bytes further
("PagedAttention: The vLLM Paper", "Impact and Follow-Ups"; "Limitations":
very long contexts still need quantization).  They fix no format; the reading
here is the OCP 8-bit floating point format E4M3 (the fp8 of gfx950), written
out from its definition:

  * 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
  * exponent field 1..15: normal value (1 + m/8) * 2^(e - 7), except that
    exponent 15 with mantissa 7 is NaN (there are no infinities), so the
    largest finite magnitude is 1.75 * 2^8 = 448;
  * exponent field 0: subnormal value (m/8) * 2^-6 = m * 2^-9.

Encoding (a reading: the pages give none): the fp32 value x / scale is
rounded to the nearest E4M3 value, ties to an even mantissa; magnitudes at or
above 448 saturate to 448; NaN encodes as 0x7F.  Scales are per KV head.
"""
from __future__ import annotations

import math

import numpy as np

MAX_E4M3 = 448.0


def e4m3_to_f64(code: int) -> float:
    """Value of one E4M3 code (NaN for 0x7F / 0xFF)."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


DECODE = np.array([e4m3_to_f64(c) for c in range(256)], dtype=np.float64)


def _round_half_even(v: float) -> int:
    f = math.floor(v)
    r = v - f
    if r > 0.5 or (r == 0.5 and f % 2 == 1):
        return f + 1
    return f


def f32_to_e4m3(y: float) -> int:
    """Nearest E4M3 code of the (fp32-exact) value y: ties to even, saturating."""
    if math.isnan(y):
        return 0x7F
    sign = 0x80 if (y < 0 or (y == 0 and math.copysign(1.0, y) < 0)) else 0
    a = abs(y)
    if a >= MAX_E4M3:
        return sign | 0x7E                       # 448
    if a < 2.0 ** -6:                            # subnormal range: steps of 2^-9
        q = _round_half_even(a / 2.0 ** -9)      # 0..8; 8 is the smallest normal
        return sign | (0x08 if q == 8 else q)
    e = math.floor(math.log2(a))
    while 2.0 ** e > a:                          # guard log2 rounding
        e -= 1
    while 2.0 ** (e + 1) <= a:
        e += 1
    q = _round_half_even((a / 2.0 ** e - 1.0) * 8.0)
    if q == 8:
        e, q = e + 1, 0
    return sign | ((e + 7) << 3) | q


# the non-negative finite codes in increasing order of value
_POS_CODES = np.array(sorted((c for c in range(0x80) if c != 0x7F), key=e4m3_to_f64),
                      dtype=np.uint8)
_POS_VALS = DECODE[_POS_CODES]


def encode(y: np.ndarray) -> np.ndarray:
    """f32_to_e4m3 over an array: the nearest entry of the sorted table of
    finite values (ties to the even code), saturating at 448, NaN to 0x7F."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    hi = np.clip(np.searchsorted(_POS_VALS, a, side="left"), 1, len(_POS_VALS) - 1)
    lo = hi - 1
    dlo, dhi = a - _POS_VALS[lo], _POS_VALS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    code = np.where(a >= MAX_E4M3, np.uint8(0x7E), code)
    neg = np.signbit(y)
    code = np.where(neg, code | np.uint8(0x80), code).astype(np.uint8)
    return np.where(np.isnan(y), np.uint8(0x7F), code).astype(np.uint8)


def quantize(x: np.ndarray, scale: np.ndarray, head_axis: int) -> np.ndarray:
    """uint8 codes of x / scale (fp32 division, correctly rounded) with one
    scale per index along `head_axis`."""
    x32 = np.asarray(x, dtype=np.float32)
    shape = [1] * x32.ndim
    shape[head_axis] = -1
    y = x32 / np.asarray(scale, dtype=np.float32).reshape(shape)
    return encode(y)


def dequantize(codes: np.ndarray, scale: np.ndarray, head_axis: int) -> np.ndarray:
    """fp64 values of the codes times their head's scale (exact in fp64)."""
    shape = [1] * codes.ndim
    shape[head_axis] = -1
    return DECODE[codes] * np.asarray(scale, dtype=np.float64).reshape(shape)
