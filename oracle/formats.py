"""Small floating-point formats used by the quantized attention path, written
out from their definitions (test infrastructure: see ``oracle/__init__.py``).

Every format here is a binary floating-point format described by three
numbers: the count of stored mantissa bits, the exponent of its smallest
normal binade, and its largest finite magnitude.  Rounding is to nearest,
ties to even; the sign of the input is kept (a negative value that rounds to
zero becomes -0), and the two 8/4-bit formats saturate at their largest
finite magnitude instead of overflowing.

* FP8 E4M3 ("e4m3fn", the OCP 8-bit format with no infinities): 3 mantissa
  bits, smallest normal 2**-6, subnormal step 2**-9, largest finite 448.
  The pages name FP8 as the attention precision (NVIDIA RTX AI optimiert
  FLUX.1 fuer Bilddaten mit niedriger Genauigkeit, hyper.ai/de; and the
  Korean copy of that article, hyper.ai/kr).
* FP4 E2M1: 1 mantissa bit, smallest normal 1, magnitudes
  {0, 0.5, 1, 1.5, 2, 3, 4, 6}.  The pages name FP4 as the Q/K precision of
  the 4-bit variant (same articles).
* bfloat16: 7 mantissa bits, smallest normal 2**-126 (the precision of the
  inputs and the output of the attention).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class FloatFormat:
    name: str
    mant_bits: int      # stored mantissa bits
    emin: int           # exponent of the smallest normal binade
    max_finite: float   # largest finite magnitude
    exp_bits: int       # width of the exponent field (for codes)


E4M3 = FloatFormat("e4m3fn", mant_bits=3, emin=-6, max_finite=448.0, exp_bits=4)
E2M1 = FloatFormat("e2m1", mant_bits=1, emin=0, max_finite=6.0, exp_bits=2)
BF16 = FloatFormat("bf16", mant_bits=7, emin=-126,
                   max_finite=float((2.0 - 2.0 ** -7) * 2.0 ** 127), exp_bits=8)


def round_to(x, fmt: FloatFormat, saturate: bool = True) -> np.ndarray:
    """Round float64 values to ``fmt`` (nearest, ties to even), as float64.

    The rounding step of a value is 2**(e - mant_bits), where e is the
    exponent of the value's binade, floored at ``fmt.emin`` so that the
    subnormal range shares the step of the smallest normal binade.  Dividing
    by a power of two is exact, so ``rint`` (ties to even) decides the
    rounding on an exact quotient.  A value that rounds up across a binade
    edge lands on the first value of the next binade, which is representable.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("round_to: non-finite input")
    a = np.abs(x)
    if saturate:
        a = np.minimum(a, fmt.max_finite)
    _, e = np.frexp(a)              # a = f * 2**e with f in [0.5, 1)
    e = np.maximum(e - 1, fmt.emin)  # a in [2**e, 2**(e+1))
    step = np.ldexp(1.0, e - fmt.mant_bits)
    r = np.rint(a / step) * step
    return np.copysign(r, x)


def encode(values, fmt: FloatFormat) -> np.ndarray:
    """Bit pattern (sign | exponent field | mantissa field) of values that are
    already representable in ``fmt`` (E4M3 or E2M1).  Exponent bias is
    1 - emin; exponent field 0 holds the subnormals and zero."""
    v = np.asarray(values, dtype=np.float64)
    a = np.abs(v)
    sign = np.signbit(v).astype(np.int64)
    normal = a >= 2.0 ** fmt.emin
    _, e = np.frexp(np.where(normal, a, 1.0))
    e = e - 1
    exp_field = np.where(normal, e - fmt.emin + 1, 0)
    frac = np.where(normal, a / np.ldexp(1.0, e) - 1.0, a / 2.0 ** fmt.emin)
    mant = frac * (1 << fmt.mant_bits)
    if not np.all(mant == np.floor(mant)):
        raise ValueError("encode: value not representable")
    total = 1 + fmt.exp_bits + fmt.mant_bits
    code = (sign << (total - 1)) | (exp_field.astype(np.int64) << fmt.mant_bits) | mant.astype(np.int64)
    return code.astype(np.uint8)


def decode(codes, fmt: FloatFormat) -> np.ndarray:
    """Value of each bit pattern of ``fmt`` (E4M3 or E2M1) as float64.  The
    E4M3 patterns S.1111.111 are NaN."""
    c = np.asarray(codes).astype(np.int64)
    total = 1 + fmt.exp_bits + fmt.mant_bits
    sign = np.where((c >> (total - 1)) & 1, -1.0, 1.0)
    exp_field = (c >> fmt.mant_bits) & ((1 << fmt.exp_bits) - 1)
    mant = c & ((1 << fmt.mant_bits) - 1)
    sub = mant / (1 << fmt.mant_bits) * 2.0 ** fmt.emin
    nor = (1.0 + mant / (1 << fmt.mant_bits)) * np.ldexp(1.0, (exp_field + fmt.emin - 1).astype(np.int64))
    val = sign * np.where(exp_field == 0, sub, nor)
    if fmt is E4M3:
        val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return val


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) to their exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round float64 values to bfloat16 (nearest, ties to even, no saturation)
    and return the uint16 bit patterns."""
    r = round_to(x, BF16, saturate=False).astype(np.float32)   # exact: bf16 values are fp32 values
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def f32(x) -> np.ndarray:
    """One correctly rounded conversion to IEEE binary32 (kept as float32)."""
    return np.asarray(x).astype(np.float32)
