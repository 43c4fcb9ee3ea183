"""Number formats used by the layer, written from their definitions.

bf16: 1 sign bit, 8 exponent bits (bias 127), 7 stored mantissa bits; the top
half of an IEEE binary32. Upcasting is exact.

E2M1 (the element of MXFP4): 1 sign bit, 2 exponent bits (bias 1), 1 mantissa
bit, no infinities or NaN. The pages name the format (WASTE "Kimi K3, as
released", section "Gate 3 repeated on real K3 experts"; SlimServe quants.md,
MXFP4 variant: "4-bit E2M1 floating-point values") but print no value table.
Reading taken: the OCP Microscaling v1.0 definition, codes 0..7 =
0, 0.5, 1, 1.5, 2, 3, 4, 6 and codes 8..15 their negatives (code 8 = -0).
Code 1 is subnormal and is kept (never flushed).

E8M0 (the MXFP4 block scale): an unsigned biased exponent; the pages state the
value is exactly 2^(e-127). Code 255 is NaN in the OCP definition (never
produced by the synthetic inputs).

This module is part of the oracle (test infrastructure only).
"""
from __future__ import annotations

import numpy as np

# E2M1 magnitudes for the 3-bit (exponent, mantissa) field, OCP MX v1.0.
_E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_TABLE = np.concatenate([_E2M1_MAG, -_E2M1_MAG])  # index = 4-bit code


def e2m1_value(code):
    """Value of 4-bit E2M1 codes (array or int)."""
    return E2M1_TABLE[np.asarray(code, dtype=np.int64) & 0xF]


def e8m0_value(code):
    """Value of E8M0 scale codes: 2^(code-127); NaN for code 255."""
    c = np.asarray(code, dtype=np.int64)
    v = np.ldexp(1.0, c - 127)
    return np.where(c == 255, np.nan, v)


def bf16_to_f64(bits) -> np.ndarray:
    """Exact upcast of bf16 bit patterns (uint16) to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):          # NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)


def f64_to_bf16(x) -> np.ndarray:
    """Round float64 values to bf16 (round to nearest, ties to even).

    One rounding from the float64 value: the significand is scaled to 8
    significant bits and rounded half-to-even; subnormals keep their fixed
    quantum 2^-133; magnitudes that round to >= 2^128 become infinity.
    Returns uint16 bit patterns."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    finite = np.isfinite(x)
    xf = np.where(finite, x, 0.0)
    m, e = np.frexp(xf)                       # xf = m * 2^e, 0.5 <= |m| < 1
    # bf16 normal: 8 significant bits -> quantum 2^(e-8); subnormal quantum 2^-133
    q_exp = np.maximum(e - 8, -133)
    r = np.rint(np.ldexp(xf, -q_exp))         # rint rounds half to even
    val = np.ldexp(r, q_exp)
    val = np.where(np.abs(val) >= 2.0 ** 128, np.copysign(np.inf, xf), val)
    out[...] = np.where(finite, val, x)
    f32 = out.astype(np.float32)              # exact: val is a bf16 value
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
