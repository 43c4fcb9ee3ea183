"""Seeded synthetic inputs for one Stable LatentMoE layer.

Shapes follow the Kimi K3 layer as described on the WASTE "Kimi K3, as
released" page (section "Shape" and the shard-header listing under "The
headline correction"): hidden 7168, latent 3584, 896 routed experts with top-16
routing, expert intermediate 3072, two shared experts merged to a 6144-wide
GLU (SlimServe quants.md, K3 GGUF tensor inventory, where the shared experts
are MXFP4).

Value distributions (one reading per item, stated once here):
  * activations x: N(0, 1) drawn in fp32, rounded to bf16 (round to nearest
    even), returned as raw uint16 bit patterns;
  * down / up projections: N(0, std = 1/sqrt(fan_in)) rounded to bf16;
  * router weight: fp32 N(0, std = 1/sqrt(hidden)), or, for the "uniform"
    router, U(-sqrt(3/hidden), +sqrt(3/hidden)) which has the same variance;
  * RMSNorm weight: 1 + 0.1 N(0, 1) rounded to bf16 (so that a dropped
    multiply by the weight is visible);
  * MXFP4 packed bytes: uniform over 0..255 (both nibbles uniform over the 16
    E2M1 codes); E8M0 scale codes uniform over 119..123, i.e. scales
    2^-8 .. 2^-4;
  * optional selection-only router bias: a Zipf(s) profile over a seeded
    permutation of expert ranks, b_e = c * rank_e^(-s).

Every tensor, and every expert inside a tensor, has its own PCG64 stream
seeded by SeedSequence(seed, spawn_key=(layer, tensor_id, index)), so any one
expert can be regenerated alone and the activations for T tokens are the first
T rows of one stream (prefix-consistent across token counts).

Nothing here computes any part of the layer.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

# tensor ids inside the spawn key
_X, _DOWN, _NORM, _ROUTER, _BIAS, _EXP_PACKED, _EXP_SCALES, _UP, _SH_PACKED, _SH_SCALES = range(10)

SCALE_CODE_LO = 119  # 2^-8
SCALE_CODE_HI = 123  # 2^-4


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    """Dimensions and input recipe of one latent-MoE layer workload."""
    name: str
    T: int                      # tokens
    hidden: int = 7168
    latent: int = 3584
    n_experts: int = 896
    topk: int = 16
    inter: int = 3072           # routed expert intermediate width
    shared_inter: int = 6144    # merged shared GLU width; 0 = no shared experts
    norm: bool = True           # RMSNorm on the aggregated latent
    rms_eps: float = 1e-6
    routed_scaling_factor: float = 1.0
    router_dist: str = "normal"  # "normal" | "uniform"
    zipf_s: Optional[float] = None   # selection-bias Zipf exponent, None = no bias
    zipf_c: float = 0.0              # selection-bias amplitude
    n_layers: int = 1
    seed: int = 0

    def with_(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)

    @property
    def pairs(self) -> int:
        return self.T * self.topk


def expert_record_bytes(c: LayerConfig) -> int:
    """Packed MXFP4 bytes of one routed expert: w1 | w3 | w2."""
    return 2 * c.inter * c.latent // 2 + c.latent * c.inter // 2


def expert_scale_bytes(c: LayerConfig) -> int:
    """E8M0 scale bytes of one routed expert: w1 | w3 | w2."""
    return 2 * c.inter * c.latent // 32 + c.latent * c.inter // 32


def shared_record_bytes(c: LayerConfig) -> int:
    return 2 * c.shared_inter * c.hidden // 2 + c.hidden * c.shared_inter // 2


def shared_scale_bytes(c: LayerConfig) -> int:
    return 2 * c.shared_inter * c.hidden // 32 + c.hidden * c.shared_inter // 32


# Named workloads: the shapes and recipes of the layer studied on the pages.
NAMED_CONFIGS = {
    # T=4, 16 experts, top-4, no norm, no shared experts.
    "tiny": LayerConfig("tiny", T=4, n_experts=16, topk=4, shared_inter=0, norm=False),
    # One K3 layer at decode batch 16.
    "decode16": LayerConfig("decode16", T=16),
    # Large decode batch with a uniform-random router.
    "decode256": LayerConfig("decode256", T=256, router_dist="uniform"),
    # Prefill of 8192 tokens.
    "prefill8192": LayerConfig("prefill8192", T=8192),
    # Eight chained layers, 4096 tokens, Zipf(1.1) selection bias. The amplitude puts the
    # hottest expert of layer 0 at about 10x the mean load (731 of 65,536 pairs); it was
    # found by bisection over the oracle's router (tests/golden/zipf_amplitude.py, which
    # records it in tests/golden/zipf_amplitude.json).
    "stack8x4096": LayerConfig("stack8x4096", T=4096, n_layers=8, zipf_s=1.1, zipf_c=0.1754),
}


def named_config(name: str, **overrides) -> LayerConfig:
    return NAMED_CONFIGS[name].with_(**overrides)


def _rng(c: LayerConfig, layer: int, tensor: int, index: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(c.seed, spawn_key=(layer, tensor, index))
    return np.random.Generator(np.random.PCG64(ss))


def _to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 draws -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def make_x(c: LayerConfig, layer: int = 0, T: Optional[int] = None) -> np.ndarray:
    """Activations x, bf16 bits uint16 [T, hidden]."""
    T = c.T if T is None else T
    g = _rng(c, layer, _X)
    return _to_bf16_bits(g.standard_normal((T, c.hidden), dtype=np.float32))


def make_dense(c: LayerConfig, layer: int = 0) -> dict:
    """Down / up projections, norm weight, router weight and selection bias."""
    H, L, E = c.hidden, c.latent, c.n_experts
    out = {}
    out["down"] = _to_bf16_bits(
        _rng(c, layer, _DOWN).standard_normal((L, H), dtype=np.float32) * np.float32(1.0 / np.sqrt(H)))
    out["up"] = _to_bf16_bits(
        _rng(c, layer, _UP).standard_normal((H, L), dtype=np.float32) * np.float32(1.0 / np.sqrt(L)))
    if c.norm:
        out["norm"] = _to_bf16_bits(
            np.float32(1.0) + np.float32(0.1) * _rng(c, layer, _NORM).standard_normal(L, dtype=np.float32))
    else:
        out["norm"] = None
    gr = _rng(c, layer, _ROUTER)
    if c.router_dist == "normal":
        out["router"] = gr.standard_normal((E, H), dtype=np.float32) * np.float32(1.0 / np.sqrt(H))
    elif c.router_dist == "uniform":
        a = np.sqrt(3.0 / H)
        out["router"] = gr.uniform(-a, a, size=(E, H)).astype(np.float32)
    else:
        raise ValueError(c.router_dist)
    if c.zipf_s is not None:
        ranks = _rng(c, layer, _BIAS).permutation(E).astype(np.float64) + 1.0
        out["select_bias"] = (c.zipf_c * ranks ** (-c.zipf_s)).astype(np.float32)
    else:
        out["select_bias"] = None
    return out


def make_expert(c: LayerConfig, layer: int, e: int):
    """One routed expert: (packed uint8 [record bytes], scales uint8 [scale bytes]).

    Record order is w1 | w3 | w2, each row-major [out, in/2] (nibbles) and
    [out, in/32] (scales)."""
    g = _rng(c, layer, _EXP_PACKED, e)
    packed = g.integers(0, 256, size=expert_record_bytes(c), dtype=np.uint8)
    g = _rng(c, layer, _EXP_SCALES, e)
    scales = g.integers(SCALE_CODE_LO, SCALE_CODE_HI + 1, size=expert_scale_bytes(c), dtype=np.uint8)
    return packed, scales


def make_shared(c: LayerConfig, layer: int = 0):
    """Merged shared GLU: (packed, scales) in gate | up | down order, or None."""
    if c.shared_inter == 0:
        return None
    packed = _rng(c, layer, _SH_PACKED).integers(0, 256, size=shared_record_bytes(c), dtype=np.uint8)
    scales = _rng(c, layer, _SH_SCALES).integers(
        SCALE_CODE_LO, SCALE_CODE_HI + 1, size=shared_scale_bytes(c), dtype=np.uint8)
    return packed, scales


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def fill_experts(c: LayerConfig, layer: int, packed_out: np.ndarray, scales_out: np.ndarray,
                 experts=None, threads: Optional[int] = None) -> None:
    """Write experts (default: all) into caller arrays [n, record] / [n, scales].

    Row i of the outputs receives expert experts[i]."""
    experts = list(range(c.n_experts)) if experts is None else list(experts)
    assert packed_out.shape == (len(experts), expert_record_bytes(c))
    assert scales_out.shape == (len(experts), expert_scale_bytes(c))

    def one(i):
        p, s = make_expert(c, layer, experts[i])
        packed_out[i] = p
        scales_out[i] = s

    with ThreadPoolExecutor(threads or _workers()) as ex:
        list(ex.map(one, range(len(experts))))


def make_router_scores(m: int, n: int, seed: int = 0, dyadic: bool = False, logit_std: float = 1.0) -> np.ndarray:
    """Router scores fp32 [m, n] in (0, 1), as a sigmoid router emits them: logits drawn
    N(0, logit_std) -- the configs' router gives logits of standard deviation about 1 --
    then sigmoid, rounded once to fp32. dyadic=True instead draws multiples of 2^-12 in
    (0, 1), so that many keys tie exactly. Own stream: SeedSequence(seed, (99, m, n))."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(99, m, n))))
    if dyadic:
        return (g.integers(1, 4096, size=(m, n)) / 4096.0).astype(np.float32)
    z = g.standard_normal((m, n)) * logit_std
    return (1.0 / (1.0 + np.exp(-z))).astype(np.float32)


def make_selection_bias(n: int, seed: int = 0, std: float = 0.05) -> np.ndarray:
    """A selection bias fp32 [n] ~ N(0, std). Own stream: SeedSequence(seed, (98, n))."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(98, n))))
    return (g.standard_normal(n) * std).astype(np.float32)
