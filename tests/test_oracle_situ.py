"""Pins for the oracle's SiTU activation (reading R17; CPU only).

The pages do not print SiTU's formula, so its parity against K3's own SituAndMul is
unpinned. What the pages fix is pinned here (WASTE "Kimi K3, as released", "What is new
since Kimi-Linear" item 3 and "Port status"; K3 report review, "SiTU-GLU"):
  * one output coordinate is bounded by beta * linear_beta = 4 * 25 = 100, and each branch
    is limited by its own beta;
  * each limit is beta * tanh(z / beta) = z + O(z^3 / beta^2), so SiTU is SwiGLU near the
    origin: the difference's leading term is -(s^3 u / beta^2 + s u^3 / linear_beta^2) / 3
    with s = SiLU(gate), which also fixes which beta belongs to which branch;
  * with both betas large SiTU is SiLU(gate) * up;
  * it is used by both FFN paths (routed and shared experts): the whole layer against the
    independent scalar twin with SiTU, and the layer with huge betas against the SiLU layer.
"""
import numpy as np
import pytest

from oracle import brute, layer
from tests import layer_inputs as li
from workload import gen

B1, B2 = layer.SITU_BETA, layer.SITU_LINEAR_BETA


def test_situ_constants_are_the_k3_configuration():
    assert (B1, B2) == (4.0, 25.0)


def test_bound_is_beta_times_linear_beta():
    rng = np.random.default_rng(0)
    g = rng.standard_normal(100000) * 10.0 ** rng.uniform(-3, 6, 100000)
    u = rng.standard_normal(100000) * 10.0 ** rng.uniform(-3, 6, 100000)
    v = layer.situ(g, u)
    assert np.all(np.abs(v) <= B1 * B2)
    # the supremum is reached: both branches saturate at their betas
    assert layer.situ(1e4, 1e4) == B1 * B2
    assert layer.situ(1e4, -1e4) == -B1 * B2
    # the sigmoid branch stays above SiLU's minimum (about -0.2785) for negative gates
    assert np.all(layer.situ(-np.logspace(-3, 6, 50), 1e4) > -0.2785 * B2)


def test_each_branch_is_limited_by_its_own_beta():
    big = 1e6
    assert layer.situ(big, 1.0) == pytest.approx(B1 * np.tanh(1.0 / B2) * B2, rel=1e-15)
    assert layer.situ(1.0, big) == pytest.approx(B1 * np.tanh(layer.silu(1.0) / B1) * B2, rel=1e-15)


def test_close_to_swiglu_near_the_origin():
    """|SiTU - SiLU(g) u| <= |s| |u|^3 / (3 b2^2) + |u| |s|^3 / (3 b1^2) everywhere (tanh x lies
    between x - x^3/3 and x), and that bound's terms are the leading terms near 0."""
    rng = np.random.default_rng(1)
    g = rng.standard_normal(20000) * 3
    u = rng.standard_normal(20000) * 30
    s = layer.silu(g)
    d = np.abs(layer.situ(g, u) - s * u)
    bound = np.abs(s) * np.abs(u) ** 3 / (3 * B2 ** 2) + np.abs(u) * np.abs(s) ** 3 / (3 * B1 ** 2)
    assert np.all(d <= bound * (1 + 1e-12) + 1e-300)
    # the leading term, branch by branch: a gate-branch term with beta_1, an up-branch term
    # with beta_2 (swapping the betas breaks both)
    for gg, uu in ((0.05, 1.0), (1.0, 0.05), (0.02, 0.03)):
        for scale in (1e-1, 1e-2):
            gs, us = gg * scale, uu * scale
            ss = layer.silu(gs)
            lead = -(ss ** 3 * us / B1 ** 2 + ss * us ** 3 / B2 ** 2) / 3
            diff = layer.situ(gs, us) - ss * us
            assert diff == pytest.approx(lead, rel=2e-2)
    # the gate branch alone: up tiny, so only the beta_1 term counts
    gs, us = 2.0, 1e-6
    ss = layer.silu(gs)
    assert (layer.situ(gs, us) - ss * us) / (ss * us) == pytest.approx(np.tanh(ss / B1) * B1 / ss - 1, rel=1e-6)


def test_large_betas_give_swiglu():
    rng = np.random.default_rng(2)
    g = rng.standard_normal(1000) * 5
    u = rng.standard_normal(1000) * 5
    np.testing.assert_allclose(layer.situ(g, u, 1e9, 1e9), layer.silu(g) * u, rtol=1e-14, atol=1e-300)


def test_symmetries_and_zeros():
    rng = np.random.default_rng(3)
    g = rng.standard_normal(1000) * 5
    u = rng.standard_normal(1000) * 50
    assert np.array_equal(layer.situ(g, -u), -layer.situ(g, u))
    assert np.all(layer.situ(0.0, u) == 0.0) and np.all(layer.situ(g, 0.0) == 0.0)
    # monotone in the up branch
    uu = np.linspace(-200, 200, 4001)
    assert np.all(np.diff(layer.situ(1.5, uu)) > 0)


@pytest.mark.parametrize("shared", [True, False])
def test_layer_with_situ_against_the_scalar_twin(shared):
    """SiTU in both FFN paths, through the whole layer: the numpy oracle against the pure-Python
    twin (own decoding, loops, math.tanh); small betas so that both limits act."""
    c = gen.LayerConfig("brute_situ", T=4, hidden=64, latent=32, n_experts=6, topk=2, inter=32,
                        shared_inter=32 if shared else 0, norm=True)
    d = li.build(c)
    d["x"] = (d["x"].astype(np.uint32) + np.uint32(0x0100)).astype(np.uint16)   # x times ~4: saturating inputs
    betas = (0.75, 1.5)
    out = li.oracle_forward(c, d, activation="situ", situ_betas=betas)
    b = brute.forward(d["x"].tolist(), d["down"].tolist(), d["norm"].tolist(), d["router"].tolist(), None,
                      [list(r) for r in d["exp_packed"]], [list(r) for r in d["exp_scales"]], d["up"].tolist(),
                      None if d["shared"] is None else (list(d["shared"][0]), list(d["shared"][1])),
                      c.topk, c.inter, c.shared_inter, c.rms_eps, c.routed_scaling_factor, situ_betas=betas)
    assert out["route"]["ids"].tolist() == b["ids"]
    ref = np.array(b["y64"])
    np.testing.assert_allclose(out["y64"], ref, rtol=1e-9, atol=1e-11 * np.abs(ref).max())
    silu_out = li.oracle_forward(c, d)
    assert np.abs(silu_out["y64"] - out["y64"]).max() > 1e-3 * np.abs(ref).max()   # SiTU does act here


def test_layer_with_huge_betas_is_the_silu_layer():
    c = li.small_config(T=6, n_experts=10, topk=3, shared_inter=64)
    d = li.build(c)
    a = li.oracle_forward(c, d)
    b = li.oracle_forward(c, d, activation="situ", situ_betas=(1e9, 1e9))
    np.testing.assert_allclose(b["y64"], a["y64"], rtol=1e-12, atol=1e-14 * np.abs(a["y64"]).max())
