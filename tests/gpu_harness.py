"""GPU-side helpers for the parity tests, the smoke check and the benchmark.

Uploads seeded inputs from `workload`, runs the library through its binding
and returns host arrays. Holds no layer arithmetic (comparisons only).
"""
from __future__ import annotations

import numpy as np
import torch

from latent_moe_expert_amd import layer as L
from workload import gen

MAX_REL = 2e-2     # max |gpu - ref| / max |ref|, per tensor
MIN_COS = 0.9995   # cosine similarity, per tensor (float64)
W_ABS = 1e-6       # routing weights


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_dev_bf16(bits: np.ndarray, dev="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def dev_bf16_to_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


class DeviceLayer:
    """One layer's weights resident on the GPU."""

    def __init__(self, c: gen.LayerConfig, layer: int = 0, dense: dict = None, experts=None, chunk: int = 64,
                 dev: str = "cuda"):
        self.c = c
        self.layer = layer
        d = gen.make_dense(c, layer) if dense is None else dense
        self.host_dense = d
        self.down = to_dev_bf16(d["down"], dev)
        self.up = to_dev_bf16(d["up"], dev)
        self.norm = None if d["norm"] is None else to_dev_bf16(d["norm"], dev)
        self.router = torch.from_numpy(np.ascontiguousarray(d["router"])).to(dev)
        self.bias = None if d["select_bias"] is None else torch.from_numpy(d["select_bias"]).to(dev)
        rec, srec = gen.expert_record_bytes(c), gen.expert_scale_bytes(c)
        self.packed = torch.empty((c.n_experts, rec), dtype=torch.uint8, device=dev)
        self.scales = torch.empty((c.n_experts, srec), dtype=torch.uint8, device=dev)
        if experts is not None:   # host arrays given (tests that hand-build experts)
            self.packed.copy_(torch.from_numpy(experts[0]))
            self.scales.copy_(torch.from_numpy(experts[1]))
        else:
            hp = np.empty((min(chunk, c.n_experts), rec), np.uint8)
            hs = np.empty((min(chunk, c.n_experts), srec), np.uint8)
            for e0 in range(0, c.n_experts, chunk):
                ids = list(range(e0, min(c.n_experts, e0 + chunk)))
                gen.fill_experts(c, layer, hp[:len(ids)], hs[:len(ids)], experts=ids)
                self.packed[e0:e0 + len(ids)].copy_(torch.from_numpy(hp[:len(ids)]))
                self.scales[e0:e0 + len(ids)].copy_(torch.from_numpy(hs[:len(ids)]))
        sh = gen.make_shared(c, layer)
        if sh is None:
            self.sh_packed = self.sh_scales = None
        else:
            self.sh_packed = torch.from_numpy(sh[0]).to(dev)
            self.sh_scales = torch.from_numpy(sh[1]).to(dev)

    def dims(self, T: int, align_block: int = 0, expert_path: int = 0, act_format: int = 0, glu_act: int = 0,
             situ_betas=(4.0, 25.0)):
        c = self.c
        return L.make_dims(T, c.hidden, c.latent, c.n_experts, c.inter, c.shared_inter, align_block, c.rms_eps,
                           c.routed_scaling_factor, expert_path, act_format, glu_act, *situ_betas)

    def run(self, x_bits: np.ndarray = None, x_dev: torch.Tensor = None, taps: bool = True, align_block: int = 0,
            expert_path: int = 0, act_format: int = 0, with_O: bool = False, keep_y_dev: bool = False,
            glu_act: int = 0, situ_betas=(4.0, 25.0)):
        c = self.c
        x = to_dev_bf16(x_bits) if x_dev is None else x_dev
        T = x.shape[0]
        dims = self.dims(T, align_block, expert_path, act_format, glu_act, situ_betas)
        ws = torch.empty(max(L.moe_latent_workspace_size(dims, c.topk), 256), dtype=torch.uint8, device=x.device)
        y = torch.empty((T, c.hidden), dtype=torch.bfloat16, device=x.device)
        out = {}
        tp = None
        if taps:
            cap, blk = L.moe_latent_align_layout(dims, c.topk)
            dv = x.device
            tp = {
                "z": torch.empty((T, c.latent), dtype=torch.int16, device=dv),
                "logits": torch.empty((T, c.n_experts), dtype=torch.float32, device=dv),
                "topk_ids": torch.empty((T, c.topk), dtype=torch.int32, device=dv),
                "topk_w": torch.empty((T, c.topk), dtype=torch.float32, device=dv),
                "counts": torch.empty(c.n_experts, dtype=torch.int32, device=dv),
                "sorted_ids": torch.empty(cap, dtype=torch.int32, device=dv),
                "expert_ids": torch.empty(cap // blk, dtype=torch.int32, device=dv),
                "num_post": torch.empty(1, dtype=torch.int32, device=dv),
                "inv_pos": torch.empty(T * c.topk, dtype=torch.int32, device=dv),
                "c": torch.empty((T, c.latent), dtype=torch.float32, device=dv),
                "c_norm": torch.empty((T, c.latent), dtype=torch.int16, device=dv),
                "y_routed": torch.empty((T, c.hidden), dtype=torch.float32, device=dv),
                "y_shared": torch.empty((T, c.hidden), dtype=torch.float32, device=dv),
            }
            if with_O:   # expert outputs by flat slot index t*k+j: T*k x latent fp32
                tp["O"] = torch.empty((T * c.topk, c.latent), dtype=torch.float32, device=dv)
            out["B"] = blk
        L.moe_latent_forward_ex(dims, x, self.down, self.norm, self.router, self.bias, self.packed, self.scales,
                                self.up, self.sh_packed, self.sh_scales, c.topk, y, ws, taps=tp)
        torch.cuda.synchronize()
        out["y"] = dev_bf16_to_bits(y)
        if keep_y_dev:
            out["y_dev"] = y
        if tp is not None:
            for k, v in tp.items():
                a = v.cpu().numpy()
                out[k] = a.view(np.uint16) if v.dtype == torch.int16 else a
        return out

    def oracle_experts(self):
        """Expert source for the oracle: regenerate expert e from its seeded stream."""
        return lambda e: gen.make_expert(self.c, self.layer, e)


_K3 = {}


def k3_layer() -> DeviceLayer:
    """Layer 0 of the K3 workloads (shared by the decode and prefill configs): 896 experts
    on the GPU (15.7 GB), uploaded once per test session."""
    if "layer" not in _K3:
        _K3["layer"] = DeviceLayer(gen.named_config("decode16"))
    return _K3["layer"]


def maxrel(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.abs(b).max()
    return float(np.abs(a - b).max() / den) if den > 0 else float(np.abs(a - b).max())


def cosine(a, b) -> float:
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 and nb == 0:
        return 1.0
    return float(a @ b / (na * nb))


def assert_close(name, gpu, ref, max_rel=MAX_REL, min_cos=MIN_COS):
    mr, cs = maxrel(gpu, ref), cosine(gpu, ref)
    print(f"  {name}: max_rel={mr:.3e} cos={cs:.7f}")
    assert mr <= max_rel and cs >= min_cos, f"{name}: max_rel={mr:.3e} cos={cs:.7f}"
    return mr, cs


def compare_layer(out: dict, ref: dict, T: int, k: int, E: int, tokens=None, w_tol=None):
    """The comparison protocol: near-tie tokens excluded and counted; ids bit-exact;
    per-expert token lists bit-exact; weights 1e-6 abs (or within w_tol [T, k], the bound
    for a chained layer whose input differs from the oracle's); z, c, c_norm, y_routed,
    y_shared, y each within MAX_REL and MIN_COS. `ref` is an oracle evaluation
    whose per-token results cover `tokens` (default: all)."""
    flags = ref["route"]["near_tie"]
    keep = ~flags
    n_flag = int(flags.sum())
    print(f"  near-tie tokens excluded: {n_flag} of {T}")
    ids_ref = ref["route"]["ids"]
    assert np.array_equal(out["topk_ids"][keep], ids_ref[keep]), "topk_ids differ"
    dw = np.abs(out["topk_w"][keep] - ref["route"]["weights"][keep])
    assert (dw <= (W_ABS if w_tol is None else w_tol[keep])).all(), f"topk_w differ by up to {dw.max():.3e}"
    # per-expert token lists (unflagged tokens), from the GPU's align output
    pairs = T * k
    s, ex, n = out["sorted_ids"], out["expert_ids"], int(out["num_post"][0])
    B = out["B"]
    flat_keep = np.repeat(keep, k)
    al = ref["align"]
    for e in np.unique(ids_ref[keep]):
        blocks = np.nonzero(ex[: n // B] == e)[0]
        seg = np.concatenate([s[b * B:(b + 1) * B] for b in blocks]) if len(blocks) else np.array([], np.int32)
        seg = seg[seg < pairs]
        seg = seg[flat_keep[seg]]
        refseg = np.nonzero(ids_ref.reshape(-1) == e)[0]
        refseg = refseg[flat_keep[refseg]]
        assert np.array_equal(seg, refseg), f"token list of expert {e} differs"
    if n_flag == 0:
        for key in ("sorted_ids", "expert_ids", "counts", "inv_pos"):
            assert np.array_equal(out[key], al[key]), f"{key} differs"
        assert n == al["num_post"]
    toks = ref["tokens"]
    sel = keep[toks]
    rows = toks[sel]
    assert_close("z", bf16_bits_to_f64(out["z"][rows]), ref["z"][sel])
    assert_close("c", out["c"][rows], ref["c"][sel])
    assert_close("c_norm", bf16_bits_to_f64(out["c_norm"][rows]), ref["c_norm"][sel])
    assert_close("y_routed", out["y_routed"][rows], ref["y_routed"][sel])
    if np.abs(ref["y_shared"]).max() > 0:
        assert_close("y_shared", out["y_shared"][rows], ref["y_shared"][sel])
    else:
        assert np.all(out["y_shared"][rows] == 0)
    assert_close("y", bf16_bits_to_f64(out["y"][rows]), ref["y64"][sel])
    return n_flag


def expert_outputs_check(out: dict, c, x_bits: np.ndarray, down_bits: np.ndarray, experts_src, experts, k: int,
                         act: str = "bf16", activation: str = "silu", situ_betas=(4.0, 25.0)):
    """Every slot of each expert in `experts`: the GPU's expert output O (tap, by flat slot
    index t*k+j, before the routing weight) against the oracle's expert FFN applied to the
    oracle's latent of the slot's token, within MAX_REL / MIN_COS per expert. Slots are
    those of the GPU's align output (itself checked bit-exact against the oracle)."""
    from oracle.layer import expert_ffn, glu_activation
    from oracle.mxfp4 import decode_glu_record
    glu_fn = glu_activation(activation, *situ_betas)
    from oracle.numerics import bf16_to_f64
    sorted_ids, B = out["sorted_ids"], out["B"]
    ex = out["expert_ids"]
    n_post = int(out["num_post"][0])
    Wd = bf16_to_f64(down_bits)
    pairs = x_bits.shape[0] * k
    for e in experts:
        blocks = np.nonzero(ex[: n_post // B] == e)[0]
        pos = np.concatenate([np.arange(b * B, (b + 1) * B) for b in blocks])
        pos = pos[sorted_ids[pos] < pairs]
        flat = sorted_ids[pos]
        toks = flat // k
        z = bf16_to_f64(x_bits[toks]) @ Wd.T
        p, sc = experts_src(int(e))
        w1, w3, w2 = decode_glu_record(p, sc, c.latent, c.inter)
        ref = expert_ffn(z, w1, w3, w2, act, glu_fn)
        assert_close(f"O[expert {int(e)}: {len(pos)} slots]", out["O"][flat], ref)
