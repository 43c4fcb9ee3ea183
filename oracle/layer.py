"""One Stable LatentMoE layer, evaluated directly (oracle; test infrastructure only).

Dataflow, from the pages:
  * WASTE "Kimi K3, as released", section "What is new since Kimi-Linear",
    item 1, and the "Port status" table, row "latent MoE": the 7168-wide
    hidden state is projected down to the 3584-wide latent
    (routed_expert_down_proj), the routed experts run on the latent, an
    optional RMSNorm (routed_expert_norm) follows, and routed_expert_up_proj
    maps back to 7168; the shared experts stay on the full hidden state.
  * Same page, section "Against the technical report": the router is a
    sigmoid with e_score_correction_bias used for selection only, the weights
    are renormalised over the selected top-k and then multiplied by
    routed_scaling_factor; the RMSNorm sits before the up-projection.
  * K3 report review, section "Stable LatentMoE": 896 experts, 16 selected
    per token (1/56), two full-width shared experts; the routed chain is
    down-projection -> gated experts -> aggregation -> normalisation ->
    up-projection. Section "parameter count", first step: each routed expert
    is a GLU MLP, gate and up 3584->3072, down 3072->3584; second step: the
    two shared experts are merged into one 2x3072 = 6144 wide GLU.
  * SlimServe quants.md, note on moe_align_block_size: one padded
    expert-sorted layout whose row alignment is the LCM of the consumers' tile
    widths, with expert ids per tile; expert ids above 255 must work.

Readings taken where the pages are silent:
  R1  the RMSNorm acts on the aggregated latent, after the combine.
  R2  RMSNorm(c) = c / sqrt(mean(c^2) + eps) * g (eps inside the root).
  R4  the GLU activation is SiLU(gate) * up by default; SiTU's formula is not printed.
  R17 SiTU, selectable (activation="situ"): beta * tanh(SiLU(gate) / beta) *
      linear_beta * tanh(up / linear_beta), beta 4, linear_beta 25 -- a reading built from
      the properties the pages state; parity unpinned against K3's own SituAndMul.
  R5  w1 is the gate, w3 the up projection, w2 the down projection.
  R8  ties in the selection key go to the lower expert id; the selected ids
      are stored in ascending id order (a function of the selected set only).
  R10 the router weight scales each expert's output after w2.
  R11 the layer output is y = routed + shared (no residual inside the layer).
  R12 align: flat slot index t*k+j in ascending order inside each expert's
      segment, segments padded to a multiple of B with the sentinel T*k,
      experts in ascending id order, empty experts get no block; capacity is
      B*floor((T*k + min(E, T*k)*(B-1)) / B) entries, the tail past
      num_tokens_post_padded holds the sentinel and expert id -1.

Arithmetic: float64 throughout, on exactly upcast inputs; the final output is
rounded once to bf16 (round to nearest even).
"""
from __future__ import annotations

from typing import Callable, Optional, Sequence

import numpy as np

from . import mxfp8
from .mxfp4 import decode_glu_record
from .numerics import bf16_to_f64, f64_to_bf16

NEAR_TIE = 1e-6


def sigmoid(x):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def silu(g):
    """SiLU(g) = g * sigmoid(g)."""
    return g * sigmoid(g)


def glu(gate, up):
    """GLU activation of the experts: SiLU(gate) * up (reading R4)."""
    return silu(gate) * up


# SiTU parameters of the K3 configuration (WASTE "Kimi K3, as released", "What is new since
# Kimi-Linear", item 3: activation_situ_beta and activation_situ_linear_beta)
SITU_BETA = 4.0
SITU_LINEAR_BETA = 25.0


def situ(gate, up, beta: float = SITU_BETA, linear_beta: float = SITU_LINEAR_BETA):
    """SiTU ("Sigmoid Tanh Unit") GLU activation -- reading R17, PARITY UNPINNED against K3's
    own SituAndMul, whose formula the pages do not print.

    What the pages fix: SiTU replaces SiLU in the GLU of both FFN paths (WASTE page, "Port
    status"); the sigmoid branch and the tanh branch of the GLU are each soft-limited, by
    beta_1 = 4 and beta_2 = 25, so that one output coordinate stays below beta_1 * beta_2 =
    100 in magnitude, and the limit has the form beta * tanh(z / beta) = z + O(z^3 / beta^2),
    so that SiTU is close to SwiGLU near the origin (K3 report review, "SiTU-GLU").
    Reading: the sigmoid branch is SiLU(gate) and the linear branch is up, each passed
    through that limit with its own beta:
        SiTU(gate, up) = beta * tanh(SiLU(gate) / beta) * linear_beta * tanh(up / linear_beta).
    (An alternative that also meets every stated fact, SiLU(beta * tanh(gate / beta)) for
    the first factor, is not used.)"""
    return beta * np.tanh(silu(gate) / beta) * (linear_beta * np.tanh(up / linear_beta))


def glu_activation(name: str, beta: float = SITU_BETA, linear_beta: float = SITU_LINEAR_BETA):
    """The experts' GLU activation by name: "silu" (default) or "situ"."""
    if name == "silu":
        return glu
    if name == "situ":
        return lambda g, u: situ(g, u, beta, linear_beta)
    raise ValueError("activation must be 'silu' or 'situ'")


def rmsnorm(c, g, eps: float):
    """RMSNorm over the last axis: c / sqrt(mean(c^2) + eps) * g (reading R2)."""
    c = np.asarray(c, dtype=np.float64)
    ms = np.mean(c * c, axis=-1, keepdims=True)
    out = c / np.sqrt(ms + eps)
    return out if g is None else out * np.asarray(g, dtype=np.float64)


def chain_input(y_bits: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """The next layer's input in a stack of layers: the weightless RMSNorm of this layer's
    bf16 output, rounded to bf16 (reading R16). The pages put an RMSNorm in front of each
    decoder block's input (K3 report review, section on Block AttnRes: standard PreNorm
    residuals); without it the chained outputs grow by the shared experts' gain at every
    layer. Harness glue between layers, not part of the layer."""
    return f64_to_bf16(rmsnorm(bf16_to_f64(y_bits), None, eps))


# --------------------------------------------------------------------------- router

def route(x64: np.ndarray, router_w: np.ndarray, select_bias: Optional[np.ndarray], k: int,
          rsf: float = 1.0, near_tie: float = NEAR_TIE) -> dict:
    """Sigmoid router with selection-only bias and top-k.

    logits = x . W_r^T (float64); s = sigmoid(logits); key = s + bias.
    The k experts with the largest key are selected (ties to the lower id),
    stored in ascending id order; weights w_j = s_j / sum(s_sel) * rsf use the
    unbiased scores. A token is flagged as a near tie when the k-th and
    (k+1)-th keys differ by at most `near_tie`."""
    x64 = np.asarray(x64, dtype=np.float64)
    W = np.asarray(router_w, dtype=np.float64)
    T, E = x64.shape[0], W.shape[0]
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    logits = x64 @ W.T
    scores = sigmoid(logits)
    keys = scores + (0.0 if select_bias is None else np.asarray(select_bias, dtype=np.float64)[None, :])
    ids = np.empty((T, k), dtype=np.int32)
    flags = np.zeros(T, dtype=bool)
    margin = np.full(T, np.inf)
    expert_index = np.arange(E)
    for t in range(T):
        order = np.lexsort((expert_index, -keys[t]))   # key descending, then id ascending
        sel = order[:k]
        if k < E:
            margin[t] = keys[t, order[k - 1]] - keys[t, order[k]]
            flags[t] = margin[t] <= near_tie
        ids[t] = np.sort(sel)
    s_sel = np.take_along_axis(scores, ids.astype(np.int64), axis=1)
    weights = s_sel / s_sel.sum(axis=1, keepdims=True) * rsf
    return {"logits": logits, "scores": scores, "keys": keys, "ids": ids,
            "weights": weights, "near_tie": flags, "margin": margin}


# --------------------------------------------------------------------------- align

def align_capacity(T: int, k: int, E: int, B: int) -> int:
    """Entries of the padded layout that always suffice (reading R12)."""
    pairs = T * k
    return B * ((pairs + min(E, pairs) * (B - 1)) // B)


def align(ids: np.ndarray, E: int, B: int) -> dict:
    """moe_align_block_size on ids [T, k] (reading R12).

    Returns counts [E], sorted_ids [cap], expert_ids [cap/B], num_post,
    inv_pos [T*k] (position of each flat slot index in sorted_ids)."""
    ids = np.asarray(ids)
    T, k = ids.shape
    pairs = T * k
    cap = align_capacity(T, k, E, B)
    flat = ids.reshape(-1).astype(np.int64)
    if pairs and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert id out of range")
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    sorted_ids = np.full(cap, pairs, dtype=np.int32)
    expert_ids = np.full(cap // B, -1, dtype=np.int32)
    inv_pos = np.empty(pairs, dtype=np.int32)
    off = 0
    for e in range(E):
        c = int(counts[e])
        if c == 0:
            continue
        members = np.nonzero(flat == e)[0]          # ascending flat index
        sorted_ids[off:off + c] = members
        inv_pos[members] = off + np.arange(c)
        padded = -(-c // B) * B
        expert_ids[off // B: (off + padded) // B] = e
        off += padded
    return {"counts": counts, "sorted_ids": sorted_ids, "expert_ids": expert_ids,
            "num_post": off, "inv_pos": inv_pos, "cap": cap, "B": B}


# --------------------------------------------------------------------------- layer

def _expert_source(experts) -> Callable[[int], tuple]:
    """Accept (packed [E, rec], scales [E, srec]) arrays or a callable e -> (packed, scales)."""
    if callable(experts):
        return experts
    packed, scales = experts
    return lambda e: (packed[e], scales[e])


def expert_ffn(z_rows: np.ndarray, w1: np.ndarray, w3: np.ndarray, w2: np.ndarray, act: str = "bf16",
               glu_fn=glu) -> np.ndarray:
    """One routed expert on latent rows: (act(z W1^T, z W3^T)) W2^T with the GLU activation
    glu_fn (default SiLU(gate) * up).

    act="mxfp8": the expert's inputs are MXFP8 (mxfp8.py): z_rows are expected already
    quantized, and the GLU output is quantized before w2."""
    h = glu_fn(z_rows @ w1.T, z_rows @ w3.T)
    if act == "mxfp8":
        h = mxfp8.quantize(h)
    return h @ w2.T


def forward(x_bits: np.ndarray, down_bits: np.ndarray, norm_bits: Optional[np.ndarray],
            router_w: np.ndarray, select_bias: Optional[np.ndarray], experts,
            up_bits: np.ndarray, shared: Optional[tuple], k: int, *,
            inter: int, shared_inter: int = 0, rms_eps: float = 1e-6, rsf: float = 1.0,
            align_block: int = 16, tokens: Optional[Sequence[int]] = None, act: str = "bf16",
            activation: str = "silu", situ_beta: float = SITU_BETA,
            situ_linear_beta: float = SITU_LINEAR_BETA) -> dict:
    """Evaluate the layer.

    x_bits bf16 [T, H]; down_bits bf16 [L, H]; norm_bits bf16 [L] or None;
    router_w fp32 [E, H]; select_bias fp32 [E] or None; experts = (packed
    [E, rec], scales [E, srec]) or callable e -> (packed, scales), records
    w1 | w3 | w2; up_bits bf16 [H, L]; shared = (packed, scales) gate | up |
    down or None.

    Routing and align cover all T tokens. Per-token results (z, O, c, c_norm,
    y_routed, y_shared, y) are computed for `tokens` (default: all), in that
    order.

    act="bf16" (default): the routed experts read the latent and the GLU output as
    they are. act="mxfp8": they read MXFP8 activations (mxfp8.py), the latent
    rounded to bf16 and then quantized, the GLU output quantized before w2; the
    shared experts, projections and router are unchanged.

    activation="situ": the GLU activation of the routed and the shared experts is SiTU
    (situ, reading R17) with the given betas instead of SiLU(gate) * up."""
    glu_fn = glu_activation(activation, situ_beta, situ_linear_beta)
    if act not in ("bf16", "mxfp8"):
        raise ValueError("act must be 'bf16' or 'mxfp8'")
    X = bf16_to_f64(x_bits)
    T, H = X.shape
    Wd = bf16_to_f64(down_bits)
    L = Wd.shape[0]
    Wr = np.asarray(router_w, dtype=np.float64)
    E = Wr.shape[0]
    toks = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)

    r = route(X, Wr, select_bias, k, rsf)
    al = align(r["ids"], E, align_block)

    Xs = X[toks]
    z = Xs @ Wd.T                                          # [n, L]

    # routed experts: each expert decoded once, applied to its rows
    get = _expert_source(experts)
    ids_s = r["ids"][toks]
    z_in = mxfp8.quantize(bf16_to_f64(f64_to_bf16(z))) if act == "mxfp8" else z
    O = np.zeros((len(toks), k, L))
    for e in np.unique(ids_s):
        rows, slots = np.nonzero(ids_s == e)
        p, s = get(int(e))
        w1, w3, w2 = decode_glu_record(p, s, L, inter)
        O[rows, slots] = expert_ffn(z_in[rows], w1, w3, w2, act, glu_fn)

    w_s = r["weights"][toks]
    c = np.einsum("tj,tjl->tl", w_s, O)                    # weighted combine over slots
    c_norm = rmsnorm(c, bf16_to_f64(norm_bits), rms_eps) if norm_bits is not None else c
    y_r = c_norm @ bf16_to_f64(up_bits).T                  # [n, H]

    if shared is not None:
        gs, us, ds = decode_glu_record(shared[0], shared[1], H, shared_inter)
        y_s = glu_fn(Xs @ gs.T, Xs @ us.T) @ ds.T
    else:
        y_s = np.zeros_like(y_r)

    y64 = y_r + y_s
    return {"route": r, "align": al, "tokens": toks, "z": z, "O": O, "c": c,
            "c_norm": c_norm, "y_routed": y_r, "y_shared": y_s, "y64": y64,
            "y": f64_to_bf16(y64)}
