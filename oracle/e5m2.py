"""Decoder of OCP fp8 E5M2 codes into fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The codelab "Accelerate attention on GPU with cuDNN and TransformerEngine",
section 10, keeps the backward pass's gradients in E5M2: 1 sign bit, 5 exponent
bits and 2 mantissa bits (the wider range of the two fp8 formats, for
gradients; E4M3 carries the forward tensors). E5M2 follows the IEEE pattern:
exponent bias 15, infinities and NaNs in the all-ones exponent, largest finite
value 1.75 * 2^15 = 57344.

Decoding, from the format's definition:
  exponent field e == 0:        subnormal  (-1)^s * (m / 4) * 2^(1 - 15)
  0 < e < 31:                   normal     (-1)^s * (1 + m / 4) * 2^(e - 15)
  e == 31 and m == 0:           (-1)^s * infinity
  e == 31 and m != 0:           NaN

Gradients enter the fp8 backward pass as codes plus one fp32 descale per
tensor (the per-tensor scaling of section 10): the real value of a code is
its decoded value times the descale, which ``dequantise`` forms in fp64
(exact: a 3-bit significand times a 24-bit one).
"""

from __future__ import annotations

from typing import Optional

import numpy as np

BIAS = 15
MAX_FINITE = 57344.0


def decode_code(code: int) -> float:
    """Value of one 8-bit E5M2 code."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 2) & 0x1F
    m = code & 0x3
    if e == 0x1F:
        return sign * float("inf") if m == 0 else float("nan")
    if e == 0:
        return sign * (m / 4.0) * 2.0 ** (1 - BIAS)
    return sign * (1.0 + m / 4.0) * 2.0 ** (e - BIAS)


_TABLE = np.array([decode_code(c) for c in range(256)], dtype=np.float64)


def decode(codes: np.ndarray) -> np.ndarray:
    """Decode an array of uint8 codes to fp64 (exact)."""
    codes = np.asarray(codes)
    if codes.dtype != np.uint8:
        raise TypeError("e5m2 codes must be uint8")
    return _TABLE[codes]


def dequantise(codes: np.ndarray, descale: Optional[float]) -> np.ndarray:
    """Real values of uint8 E5M2 codes under a per-tensor descale, fp64 (exact).

    ``descale=None`` means unscaled codes (a descale of 1)."""
    values = decode(codes)
    if descale is None:
        return values
    return values * float(descale)
