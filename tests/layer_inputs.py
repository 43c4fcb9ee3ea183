"""Builds one layer's seeded inputs (from `workload`) in the form the oracle takes.

Helper for the tests only: no layer arithmetic lives here beyond MXFP4 *encoding*
of hand-constructed matrices, which the closed-form tests use to build inputs.
"""
import numpy as np

from workload import gen

# E2M1 codes by value (OCP MX v1.0); used only to encode hand-built test matrices
_E2M1_VALUES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def small_config(**kw):
    base = dict(name="small", T=7, hidden=256, latent=128, n_experts=12, topk=3, inter=96,
                shared_inter=64, norm=True)
    base.update(kw)
    return gen.LayerConfig(**base)


def build(c, layer=0, experts=True):
    """Host inputs of config c: dict with x, down, norm, router, select_bias, up,
    exp_packed [E, rec], exp_scales [E, srec], shared (packed, scales) or None."""
    d = gen.make_dense(c, layer)
    d["x"] = gen.make_x(c, layer)
    if experts:
        P = np.empty((c.n_experts, gen.expert_record_bytes(c)), dtype=np.uint8)
        S = np.empty((c.n_experts, gen.expert_scale_bytes(c)), dtype=np.uint8)
        gen.fill_experts(c, layer, P, S)
        d["exp_packed"], d["exp_scales"] = P, S
    d["shared"] = gen.make_shared(c, layer)
    return d


def oracle_forward(c, d, tokens=None, align_block=16, experts=None, act="bf16", activation="silu",
                   situ_betas=(4.0, 25.0)):
    from oracle import layer
    ex = (d["exp_packed"], d["exp_scales"]) if experts is None else experts
    return layer.forward(d["x"], d["down"], d["norm"], d["router"], d["select_bias"], ex,
                         d["up"], d["shared"], c.topk, inter=c.inter, shared_inter=c.shared_inter,
                         rms_eps=c.rms_eps, rsf=c.routed_scaling_factor, align_block=align_block,
                         tokens=tokens, act=act, activation=activation, situ_beta=situ_betas[0],
                         situ_linear_beta=situ_betas[1])


def encode_mxfp4(values, scale_codes):
    """Encode a dense matrix whose entries are E2M1 values times their group scale.

    values [R, C] float, scale_codes [R, C/32] uint8 -> (packed [R, C/2], scales)."""
    values = np.asarray(values, dtype=np.float64)
    R, C = values.shape
    sc = np.asarray(scale_codes, dtype=np.int64).reshape(R, C // 32)
    unit = values / np.repeat(np.ldexp(1.0, sc - 127), 32, axis=1)
    codes = np.empty((R, C), dtype=np.uint8)
    for code in range(15, -1, -1):
        codes[unit == _E2M1_VALUES[code]] = code   # +0 wins over -0 (lower code last)
    ok = np.zeros((R, C), dtype=bool)
    for code, v in enumerate(_E2M1_VALUES):
        ok |= unit == v
    if not ok.all():
        raise ValueError("matrix not representable")
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, sc.astype(np.uint8)
