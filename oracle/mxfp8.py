"""MXFP8 activations (oracle; test infrastructure only).

The K3 report review (section on quantization-aware training, and the section
comparing the public configuration with the report) says that from SFT on the
routed experts run with MXFP4 weights and MXFP8 input activations, while the
shared experts, the latent projections and the router stay at higher
precision. The pages name the format only; this module takes the OCP
Microscaling v1.0 definitions:

  element  E4M3: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; no
           infinities; exponent field 15 with mantissa 7 is NaN, so the
           largest magnitude is 1.75 * 2^8 = 448; exponent field 0 holds the
           subnormals m/8 * 2^-6 (smallest 2^-9).
  block    32 consecutive values of a row share one E8M0 scale X = 2^s.
  scale    s = floor(log2(amax)) - 8, where 8 is the exponent of E4M3's
           largest normal; X stays a normal float (s >= -126: an all-zero or
           tiny block uses 2^-126) and s <= 127.
  element  each value v becomes the E4M3 value nearest to v / X (ties to the
           even mantissa), magnitudes past 448 saturating to 448.

Reading taken: the quantizer reads the activation the
expert receives, the latent row rounded to bf16 for the gate/up projections and
the GLU output (not rounded) for the down projection; the bf16 path of the
layer is the graded reference and this mode is reported beside it.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_value(code) -> np.ndarray:
    """Value of 8-bit E4M3 codes from the bit fields (NaN for S.1111.111)."""
    c = np.asarray(code, dtype=np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def e4m3_round(y) -> np.ndarray:
    """Nearest E4M3 value to y (float64 array; ties to even mantissa; |y| > 448 -> 448)."""
    y = np.asarray(y, dtype=np.float64)
    a = np.minimum(np.abs(y), E4M3_MAX)
    # quantum of the binade of a: 2^(e - 3) for normals (a >= 2^-6), 2^-9 below
    _, ex = np.frexp(np.where(a > 0, a, 1.0))          # a = f * 2^ex, 0.5 <= f < 1
    q_exp = np.maximum(ex - 1 - 3, -9)
    r = np.ldexp(np.rint(np.ldexp(a, -q_exp)), q_exp)   # rint: half to even
    r = np.minimum(r, E4M3_MAX)
    return np.copysign(r, y)


def scale_exponent(amax) -> np.ndarray:
    """Shared exponent s of a block with max magnitude amax: floor(log2 amax) - 8, in [-126, 127]."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(np.where(amax > 0, amax, 0.0))     # amax = f * 2^ex -> floor(log2) = ex - 1
    s = np.where(amax > 0, ex - 1 - 8, -126)
    return np.clip(s, -126, 127)


def quantize(v: np.ndarray) -> np.ndarray:
    """MXFP8 quantize-dequantize along the last axis in blocks of 32 (float64 in, float64 out)."""
    v = np.asarray(v, dtype=np.float64)
    n = v.shape[-1]
    if n % 32:
        raise ValueError("the last axis must be a multiple of 32")
    blocks = v.reshape(v.shape[:-1] + (n // 32, 32))
    s = scale_exponent(np.max(np.abs(blocks), axis=-1))[..., None]
    return np.ldexp(e4m3_round(np.ldexp(blocks, -s)), s).reshape(v.shape)
