"""Independent vectorised NumPy E4M3 codec -- TEST INFRASTRUCTURE ONLY.

A second implementation of the OCP E4M3 ("e4m3fn") codec, written
differently from the C oracle so that the two can check each other:

* decode follows the gguf-py ``F8_E4M3.dequantize_blocks`` formulation on
  page [P2] (git.wylab.me compare view, branch osimons/ocp_fp8_kv, gguf-py
  quants): sign * ldexp(mantissa, -9) for exponent field 0, else
  sign * ldexp(1 + mantissa/8, exponent - 7); magnitude 0x7F is NaN.
* encode rounds |x| on the E4M3 grid of its binade (spacing 2^(e-3), with
  the binade clamped at the smallest normal exponent -6 so that the
  subnormal grid is 2^-9) using NumPy's round-half-even ``rint``, then
  rebuilds the code bits from the rounded value.  Saturation and NaN follow
  page [P2] ggml_fp32_to_f8_e4m3: NaN -> sign|0x7F, Inf and |x| >= 448 ->
  sign|0x7E, zero keeps its sign.
"""
from __future__ import annotations

import numpy as np


def decode(codes) -> np.ndarray:
    bits = np.asarray(codes).astype(np.uint8)
    sign = np.where(bits & 0x80, np.float32(-1.0), np.float32(1.0))
    mag = bits & 0x7F
    exponent = (mag >> 3).astype(np.int32)
    mantissa = (mag & 0x07).astype(np.float32)
    values = np.where(exponent == 0,
                      np.ldexp(mantissa, -9),
                      np.ldexp(np.float32(1.0) + mantissa / np.float32(8.0), exponent - 7))
    values = np.where(mag == 0x7F, np.float32(np.nan), values).astype(np.float32)
    return (sign * values).astype(np.float32)


def encode(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    sign = np.where(np.signbit(x), np.uint8(0x80), np.uint8(0)).astype(np.uint8)
    a = np.abs(x).astype(np.float64)          # exact widening
    finite = np.isfinite(a)
    safe = np.where(finite & (a > 0), a, 1.0)
    _, ex = np.frexp(safe)                     # safe = f * 2^ex, f in [0.5, 1)
    binade = np.maximum(ex - 1, -6)            # floor(log2 a), clamped to the normal minimum
    step = np.ldexp(1.0, binade - 3)           # grid spacing inside the binade
    q = np.rint(safe / step) * step            # round half even on that grid (exact in fp64)
    # rebuild the code from the rounded magnitude q
    small = q < 2.0 ** -6
    sub_code = np.rint(q / 2.0 ** -9)
    _, qe = np.frexp(np.where(small, 1.0, q))
    qb = qe - 1
    mant = np.rint((np.where(small, 1.0, q) / np.ldexp(1.0, qb) - 1.0) * 8.0)
    norm_code = (qb + 7) * 8 + mant
    code = np.where(small, sub_code, norm_code)
    code = np.where(a >= 448.0, 0x7E, code)    # saturation (also Inf)
    code = np.where(a == 0.0, 0, code)
    code = np.where(np.isnan(a), 0x7F, code)
    code = np.where(np.isinf(a), 0x7E, code)
    return (code.astype(np.int64).astype(np.uint8) | sign).astype(np.uint8)
