"""MXFP4 decoding (oracle; test infrastructure only).

Storage as on the WASTE "Kimi K3, as released" page (shard-header listing
under "The headline correction", and section "Gate 3 repeated on real K3
experts"): a matrix [rows, cols] is kept as weight_packed U8 [rows, cols/2]
holding two E2M1 nibbles per byte, LOW nibble first (element 2j is the low
nibble of byte j, element 2j+1 the high nibble), plus weight_scale U8
[rows, cols/32] holding one E8M0 exponent per 32 consecutive weights of a row,
whose value is exactly 2^(e-127).
"""
from __future__ import annotations

import numpy as np

from .numerics import E2M1_TABLE, e8m0_value


def decode(packed: np.ndarray, scales: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Decode one MXFP4 matrix to float64 [rows, cols] (exact)."""
    if cols % 32:
        raise ValueError("cols must be a multiple of 32")
    p = np.asarray(packed, dtype=np.uint8).reshape(rows, cols // 2)
    s = np.asarray(scales, dtype=np.uint8).reshape(rows, cols // 32)
    # element 2j (low nibble of byte j) then element 2j+1 (high nibble): stacked on a last
    # axis of 2, so that row-major order of [rows, cols/2, 2] is the element order
    vals = np.stack([E2M1_TABLE[p & 0x0F], E2M1_TABLE[p >> 4]], axis=-1)
    # one scale per 32 consecutive elements of a row
    vals = vals.reshape(rows, cols // 32, 32) * e8m0_value(s)[:, :, None]
    return vals.reshape(rows, cols)


def split_glu_record(packed: np.ndarray, scales: np.ndarray, inp: int, inter: int):
    """Split a GLU record [gate | up | down] into its three (packed, scales) pairs.

    gate and up are [inter, inp]; down is [inp, inter] (the routed experts'
    w1 | w3 | w2, or the shared experts' gate | up | down)."""
    n_gu = inter * inp // 2
    s_gu = inter * inp // 32
    p = np.asarray(packed).reshape(-1)
    s = np.asarray(scales).reshape(-1)
    if p.size != 3 * n_gu or s.size != 3 * s_gu:
        raise ValueError("record size does not match [gate | up | down]")
    return ((p[:n_gu], s[:s_gu]),
            (p[n_gu:2 * n_gu], s[s_gu:2 * s_gu]),
            (p[2 * n_gu:], s[2 * s_gu:]))


def decode_glu_record(packed, scales, inp: int, inter: int):
    """Decode a GLU record to float64 (gate [inter, inp], up [inter, inp], down [inp, inter])."""
    (pg, sg), (pu, su), (pd, sd) = split_glu_record(packed, scales, inp, inter)
    return (decode(pg, sg, inter, inp), decode(pu, su, inter, inp), decode(pd, sd, inp, inter))
