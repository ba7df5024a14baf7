"""Decoder of OCP fp8 E4M3 ("e4m3fn") codes into fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The codelab "Accelerate attention on GPU with cuDNN and TransformerEngine",
section 10, gives the forward-pass fp8 format as E4M3: 1 sign bit, 4 exponent
bits and 3 mantissa bits. The pages do not say which E4M3 variant; the reading
taken is the OCP "fn" variant (finite only, exponent bias 7, no infinities,
the single NaN pattern S.1111.111, largest finite value 448), the one gfx950's
matrix cores consume.

Decoding, from the format's definition:
  exponent field e == 0: subnormal  (-1)^s * (m / 8) * 2^(1 - 7)
  0 < e and not NaN:      normal     (-1)^s * (1 + m / 8) * 2^(e - 7)
  e == 15 and m == 7:     NaN

The inputs of the fp8 path are codes plus one fp32 descale per tensor (the
codelab's section 10 scales each tensor by a factor derived from its amax):
the real value of a code is its decoded value times the descale, which
``dequantise`` forms in fp64 (exact: a 4-bit significand times a 24-bit one).
"""

from __future__ import annotations

from typing import Optional

import numpy as np

BIAS = 7


def decode_code(code: int) -> float:
    """Value of one 8-bit E4M3fn code."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - BIAS)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - BIAS)


_TABLE = np.array([decode_code(c) for c in range(256)], dtype=np.float64)


def decode(codes: np.ndarray) -> np.ndarray:
    """Decode an array of uint8 codes to fp64 (exact)."""
    codes = np.asarray(codes)
    if codes.dtype != np.uint8:
        raise TypeError("e4m3 codes must be uint8")
    return _TABLE[codes]


def dequantise(codes: np.ndarray, descale: Optional[float]) -> np.ndarray:
    """Real values of uint8 E4M3fn codes under a per-tensor descale, fp64 (exact).

    ``descale=None`` means unscaled codes (a descale of 1)."""
    values = decode(codes)
    if descale is None:
        return values
    return values * float(descale)
