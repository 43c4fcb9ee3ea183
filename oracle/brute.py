"""Pure-Python scalar twin of the layer for tiny sizes (oracle; test infrastructure only).

Written independently of `oracle.layer` and `oracle.mxfp4`: E2M1 values come
from the bit fields (sign, 2-bit exponent with bias 1, 1 mantissa bit), bf16
from the IEEE bit layout via `struct`, and every contraction is an explicit
loop. It exists to cross-check the numpy oracle on inputs small enough for
scalar loops. The dataflow is the one described on the WASTE "Kimi K3, as
released" page ("Port status", row "latent MoE"; "Against the technical
report" for the router) and the K3 report review ("Stable LatentMoE").
"""
from __future__ import annotations

import math
import struct


def e2m1(code: int) -> float:
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    mag = 0.5 * m if e == 0 else (2.0 ** (e - 1)) * (1.0 + 0.5 * m)
    return -mag if s else mag


def bf16(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def decode(packed, scales, rows, cols):
    """MXFP4 [rows, cols] from bytes (low nibble = even element) and E8M0 scales."""
    out = [[0.0] * cols for _ in range(rows)]
    for r in range(rows):
        for c in range(cols):
            byte = int(packed[r * (cols // 2) + c // 2])
            nib = (byte & 0xF) if c % 2 == 0 else (byte >> 4)
            sc = int(scales[r * (cols // 32) + c // 32])
            out[r][c] = e2m1(nib) * (2.0 ** (sc - 127))
    return out


def matvec(W, v):
    return [sum(W[i][j] * v[j] for j in range(len(v))) for i in range(len(W))]


def silu(g):
    return g / (1.0 + math.exp(-g)) if g > -700 else 0.0


def glu_record(packed, scales, inp, inter):
    n = inter * inp // 2
    s = inter * inp // 32
    gate = decode(packed[:n], scales[:s], inter, inp)
    up = decode(packed[n:2 * n], scales[s:2 * s], inter, inp)
    down = decode(packed[2 * n:], scales[2 * s:], inp, inter)
    return gate, up, down


def situ(g, u, beta, linear_beta):
    """SiTU by the same reading as oracle.layer.situ (the sigmoid branch and the linear
    branch each limited by beta * tanh(z / beta)), written with math.tanh."""
    return beta * math.tanh(silu(g) / beta) * linear_beta * math.tanh(u / linear_beta)


def glu_ffn(rec, v, situ_betas=None):
    gate, up, down = rec
    g = matvec(gate, v)
    u = matvec(up, v)
    if situ_betas is None:
        h = [silu(a) * b for a, b in zip(g, u)]
    else:
        h = [situ(a, b, *situ_betas) for a, b in zip(g, u)]
    return matvec(down, h)


def forward(x_bits, down_bits, norm_bits, router_w, select_bias, exp_packed, exp_scales,
            up_bits, shared, k, inter, shared_inter, rms_eps, rsf, situ_betas=None):
    """Returns dict(ids, weights, y64) with nested Python lists. situ_betas = (beta,
    linear_beta) selects SiTU as the GLU activation of every expert, else SiLU(g) * u."""
    T = len(x_bits)
    H = len(x_bits[0])
    L = len(down_bits)
    E = len(router_w)
    Wd = [[bf16(b) for b in row] for row in down_bits]
    Wu = [[bf16(b) for b in row] for row in up_bits]
    g = None if norm_bits is None else [bf16(b) for b in norm_bits]
    recs = [glu_record(exp_packed[e], exp_scales[e], L, inter) for e in range(E)]
    shrec = None if shared is None else glu_record(shared[0], shared[1], H, shared_inter)
    all_ids, all_w, ys = [], [], []
    for t in range(T):
        x = [bf16(b) for b in x_bits[t]]
        logits = [sum(x[h] * float(router_w[e][h]) for h in range(H)) for e in range(E)]
        s = [1.0 / (1.0 + math.exp(-a)) for a in logits]
        key = [s[e] + (0.0 if select_bias is None else float(select_bias[e])) for e in range(E)]
        chosen = sorted(sorted(range(E), key=lambda e: (-key[e], e))[:k])
        tot = sum(s[e] for e in chosen)
        w = [s[e] / tot * rsf for e in chosen]
        z = matvec(Wd, x)
        c = [0.0] * L
        for wj, e in zip(w, chosen):
            o = glu_ffn(recs[e], z, situ_betas)
            for i in range(L):
                c[i] += wj * o[i]
        if g is not None:
            ms = sum(v * v for v in c) / L
            inv = 1.0 / math.sqrt(ms + rms_eps)
            c = [c[i] * inv * g[i] for i in range(L)]
        y = matvec(Wu, c)
        if shrec is not None:
            ysh = glu_ffn(shrec, x, situ_betas)
            y = [a + b for a, b in zip(y, ysh)]
        all_ids.append(chosen)
        all_w.append(w)
        ys.append(y)
    return {"ids": all_ids, "weights": all_w, "y64": ys}


def align(ids, E, B):
    """moe_align_block_size by plain list manipulation."""
    T = len(ids)
    k = len(ids[0]) if T else 0
    pairs = T * k
    flat = [ids[t][j] for t in range(T) for j in range(k)]
    sorted_ids, expert_ids = [], []
    for e in range(E):
        members = [p for p in range(pairs) if flat[p] == e]
        if not members:
            continue
        nb = (len(members) + B - 1) // B
        sorted_ids += members + [pairs] * (nb * B - len(members))
        expert_ids += [e] * nb
    return sorted_ids, expert_ids
