"""Pins for the oracle's MXFP8 activations (CPU only).

E4M3 values against the OCP constants (tests/golden/e4m3_ocp.json) and, for every
code, against torch's float8_e4m3fn (an independent implementation of the same
format); rounding against torch's conversion; the MX block-scale rule (largest
magnitude lands in [256, 448]); saturation; idempotence; the element error bound;
and an exact scaling invariance of the layer's mxfp8 mode.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import mxfp8
from oracle.layer import forward
from tests import layer_inputs as li

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    with open(os.path.join(GOLD, "e4m3_ocp.json")) as f:
        return json.load(f)


def test_e4m3_golden_constants():
    g = _golden()
    for code, val in g["values"].items():
        assert mxfp8.e4m3_value(int(code, 16)) == val
    for code in g["nan_codes"]:
        assert np.isnan(mxfp8.e4m3_value(int(code, 16)))
    v = mxfp8.e4m3_value(np.arange(256))
    assert np.nanmax(v) == g["max_normal"] and mxfp8.E4M3_MAX == g["max_normal"]
    pos = v[(v > 0) & np.isfinite(v)]
    assert pos.min() == g["min_subnormal"]
    assert pos[pos >= g["min_normal"]].min() == g["min_normal"]


def test_e4m3_every_code_matches_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = mxfp8.e4m3_value(np.arange(256))
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    assert np.all((ref == got) | both_nan)


def test_e4m3_round_matches_torch_in_range():
    rng = np.random.default_rng(0)
    vals = mxfp8.e4m3_value(np.arange(256))
    fin = np.unique(vals[np.isfinite(vals)])
    mids = (fin[1:] + fin[:-1]) / 2                       # every tie between neighbours
    y = np.concatenate([fin, mids, rng.uniform(-448, 448, 20000), rng.normal(0, 1, 20000),
                        rng.normal(0, 0.01, 20000)])
    y32 = y.astype(np.float32).astype(np.float64)          # torch converts from fp32
    ref = torch.from_numpy(y32.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(mxfp8.e4m3_round(y32), ref)


def test_e4m3_round_saturates_and_ties_to_even():
    assert mxfp8.e4m3_round(np.array([1000.0, -1e9, 449.0]))[0] == 448.0
    assert mxfp8.e4m3_round(np.array([-1e9]))[0] == -448.0
    # 1 + 1/16 lies halfway between 1.0 (mantissa 000) and 1.125 (001): even is 1.0
    assert mxfp8.e4m3_round(np.array([1.0625]))[0] == 1.0
    # 1.1875 lies between 1.125 (001) and 1.25 (010): even is 1.25
    assert mxfp8.e4m3_round(np.array([1.1875]))[0] == 1.25


def test_block_scale_rule_and_bounds():
    rng = np.random.default_rng(1)
    v = rng.normal(0, 1, (64, 256)) * np.exp(rng.uniform(-20, 20, (64, 1)))
    q = mxfp8.quantize(v)
    blocks = v.reshape(64, 8, 32)
    qb = q.reshape(64, 8, 32)
    amax = np.abs(blocks).max(-1)
    s = np.floor(np.log2(amax)) - 8                       # emax of E4M3 is 8
    scaled_max = np.abs(qb).max(-1) / np.exp2(s)
    assert np.all((scaled_max >= 256) & (scaled_max <= 448))
    # every element is an E4M3 value times 2^s
    codes = qb / np.exp2(s)[..., None]
    fin = mxfp8.e4m3_value(np.arange(256))
    assert np.all(np.isin(codes, fin[np.isfinite(fin)]))
    # error bound: half a quantum of the element's binade (3 mantissa bits), 2^-10 * X below
    err = np.abs(qb - blocks)
    xs = np.exp2(s)[..., None]
    a = np.abs(blocks) / xs
    bound = np.where(a >= 2.0 ** -6, np.exp2(np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 4), 2.0 ** -10) * xs
    sat = a > 448
    assert np.all(err[~sat] <= bound[~sat] * (1 + 1e-12))
    assert np.array_equal(mxfp8.quantize(q), q)            # idempotent


def test_power_of_two_equivariance():
    rng = np.random.default_rng(2)
    v = rng.normal(0, 1, (8, 64))
    for k in (-40, -3, 5, 30):
        assert np.array_equal(mxfp8.quantize(v * 2.0 ** k), mxfp8.quantize(v) * 2.0 ** k)


def test_zero_block_and_tiny_scale():
    q = mxfp8.quantize(np.zeros((2, 32)))
    assert np.all(q == 0)
    assert mxfp8.scale_exponent(np.array([0.0, 2.0 ** -140]))[0] == -126
    assert mxfp8.scale_exponent(np.array([2.0 ** -140]))[0] == -126


def test_layer_mxfp8_mode_down_scale_shift_doubles_output():
    """Adding 1 to every w2 scale code doubles each routed expert's output exactly in the
    mxfp8 mode too (the GLU output is quantized before w2, so it is unchanged)."""
    c = li.small_config(T=6, hidden=256, latent=256, n_experts=6, topk=2, inter=256, shared_inter=0, norm=False)
    d = li.build(c)
    a = li.oracle_forward(c, d, act="mxfp8")
    p, s = d["exp_packed"], d["exp_scales"].copy()
    gu = 2 * c.inter * c.latent // 32
    s[:, gu:] = s[:, gu:] + 1
    b = li.oracle_forward(c, {**d, "exp_scales": s}, act="mxfp8")
    assert np.array_equal(b["O"], 2 * a["O"])
    # and the mode differs from the bf16 reference by the quantization error only
    r = li.oracle_forward(c, d)
    rel = np.linalg.norm(a["y_routed"] - r["y_routed"]) / np.linalg.norm(r["y_routed"])
    assert 1e-3 < rel < 0.1
