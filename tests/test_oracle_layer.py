"""Whole-layer pins for the oracle (CPU only).

T7  dense equivalence at k = E (no top-k, align or gather needed);
T8  E = 1, k = 1 reduces to a plain dense FFN chain;
T9  brute force against the independent pure-Python twin (with forced exact ties);
T10 E8M0 shift invariance (power-of-two scaling) and what it tells about the
    norm placement and the gate/up roles;
T13 determinism; T14 prefix consistency across token counts;
and a closed form: experts, projections and shared experts built from signed
permutation matrices, so every output is a gather that the test computes by
indexing alone.
"""
import numpy as np
import pytest

from oracle import brute, layer
from oracle.mxfp4 import decode_glu_record
from oracle.numerics import bf16_to_f64
from tests import layer_inputs as li
from workload import gen


def _dense_equivalent_routed(c, d):
    """c_t = sum_e w_e(t) f_e(z_t) as ONE dense GLU of width E*I with per-token unit scaling."""
    X = bf16_to_f64(d["x"])
    z = X @ bf16_to_f64(d["down"]).T
    logits = X @ d["router"].astype(np.float64).T
    s = 1.0 / (1.0 + np.exp(-logits))
    w = s / s.sum(axis=1, keepdims=True) * c.routed_scaling_factor      # [T, E]
    W1, W3, W2 = [], [], []
    for e in range(c.n_experts):
        a, b, cc = decode_glu_record(d["exp_packed"][e], d["exp_scales"][e], c.latent, c.inter)
        W1.append(a), W3.append(b), W2.append(cc)
    W1, W3, W2 = np.concatenate(W1), np.concatenate(W3), np.concatenate(W2, axis=1)
    G, U = z @ W1.T, z @ W3.T
    h = G / (1 + np.exp(-G)) * U * np.repeat(w, c.inter, axis=1)
    return h @ W2.T


def test_t7_dense_equivalence_when_k_equals_E():
    c = li.small_config(n_experts=5, topk=5, T=6, norm=False, shared_inter=0)
    d = li.build(c)
    out = li.oracle_forward(c, d)
    ref = _dense_equivalent_routed(c, d)
    np.testing.assert_allclose(out["c"], ref, rtol=1e-9, atol=1e-12 * np.abs(ref).max())


def test_t8_single_expert_is_a_plain_ffn_chain():
    c = li.small_config(n_experts=1, topk=1, T=4)
    d = li.build(c)
    out = li.oracle_forward(c, d)
    X = bf16_to_f64(d["x"])
    z = X @ bf16_to_f64(d["down"]).T
    w1, w3, w2 = decode_glu_record(d["exp_packed"][0], d["exp_scales"][0], c.latent, c.inter)
    g = z @ w1.T
    ffn = (g / (1 + np.exp(-g)) * (z @ w3.T)) @ w2.T
    nrm = ffn / np.sqrt((ffn ** 2).mean(axis=1, keepdims=True) + c.rms_eps) * bf16_to_f64(d["norm"])
    gs, us, ds = decode_glu_record(d["shared"][0], d["shared"][1], c.hidden, c.shared_inter)
    a = X @ gs.T
    shared = (a / (1 + np.exp(-a)) * (X @ us.T)) @ ds.T
    ref = nrm @ bf16_to_f64(d["up"]).T + shared
    assert np.all(out["route"]["weights"] == 1.0)
    np.testing.assert_allclose(out["y64"], ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max())


@pytest.mark.parametrize("with_bias,norm,shared", [(False, True, True), (True, False, False)])
def test_t9_brute_force_twin(with_bias, norm, shared):
    c = gen.LayerConfig("brute", T=5, hidden=64, latent=32, n_experts=8, topk=2, inter=32,
                        shared_inter=32 if shared else 0, norm=norm)
    d = li.build(c)
    d["router"][5] = d["router"][1]          # experts 1 and 5 always tie exactly
    d["router"][6] = d["router"][2]
    if with_bias:
        d["select_bias"] = np.linspace(-0.05, 0.05, 8).astype(np.float32)
        d["select_bias"][3] = 2.0            # expert 3 is always first
        d["select_bias"][[1, 5]] = 1.5       # 1 and 5 tie exactly for the k-th (last) place
    out = li.oracle_forward(c, d)
    b = brute.forward(d["x"].tolist(), d["down"].tolist(),
                      None if d["norm"] is None else d["norm"].tolist(),
                      d["router"].tolist(), None if d["select_bias"] is None else d["select_bias"].tolist(),
                      [list(r) for r in d["exp_packed"]], [list(r) for r in d["exp_scales"]],
                      d["up"].tolist(), None if d["shared"] is None else (list(d["shared"][0]), list(d["shared"][1])),
                      c.topk, c.inter, c.shared_inter, c.rms_eps, c.routed_scaling_factor)
    assert out["route"]["ids"].tolist() == b["ids"]
    if with_bias:
        assert all(1 in row and 5 not in row for row in b["ids"])   # tie broken to the lower id
    np.testing.assert_allclose(out["route"]["weights"], np.array(b["weights"]), rtol=1e-12)
    ref = np.array(b["y64"])
    np.testing.assert_allclose(out["y64"], ref, rtol=1e-9, atol=1e-11 * np.abs(ref).max())


def _shift_scales(d, c, which, delta):
    """Add delta to every E8M0 code of one matrix (w1, w3 or w2) of every expert."""
    n_gu = c.inter * c.latent // 32
    sl = {"w1": slice(0, n_gu), "w3": slice(n_gu, 2 * n_gu), "w2": slice(2 * n_gu, 3 * n_gu)}[which]
    d2 = dict(d)
    s = d["exp_scales"].copy()
    s[:, sl] += np.uint8(delta)
    d2["exp_scales"] = s
    return d2


def test_t10_e8m0_shift_invariance():
    c = li.small_config(T=5, shared_inter=0, norm=False)
    d = li.build(c)
    base = li.oracle_forward(c, d)
    for which in ("w2", "w3"):          # linear in w2 and in the up branch: output doubles exactly
        out = li.oracle_forward(c, _shift_scales(d, c, which, 1))
        assert np.array_equal(out["O"], 2 * base["O"])
        assert np.array_equal(out["y_routed"], 2 * base["y_routed"])
    out = li.oracle_forward(c, _shift_scales(d, c, "w1", 1))   # the gate is nonlinear
    assert not np.allclose(out["O"], 2 * base["O"], rtol=1e-3)
    # with the norm after the aggregate (and eps = 0) the doubled aggregate cancels exactly
    cn = c.with_(norm=True, rms_eps=0.0)
    dn = li.build(cn)
    b0 = li.oracle_forward(cn, dn)
    b1 = li.oracle_forward(cn, _shift_scales(dn, cn, "w2", 1))
    assert np.array_equal(b1["c"], 2 * b0["c"])
    assert np.array_equal(b1["y_routed"], b0["y_routed"])


def test_t13_determinism():
    c = li.small_config()
    d1, d2 = li.build(c), li.build(c)
    for k in ("x", "down", "up", "norm", "router", "exp_packed", "exp_scales"):
        assert np.array_equal(d1[k], d2[k])
    a, b = li.oracle_forward(c, d1), li.oracle_forward(c, d2)
    assert np.array_equal(a["y64"], b["y64"]) and np.array_equal(a["y"], b["y"])


def test_t14_prefix_consistency_across_T():
    c5, c9 = li.small_config(T=5), li.small_config(T=9)
    d5, d9 = li.build(c5), li.build(c9)
    assert np.array_equal(d5["x"], d9["x"][:5])
    a, b = li.oracle_forward(c5, d5), li.oracle_forward(c9, d9)
    assert np.array_equal(a["route"]["ids"], b["route"]["ids"][:5])
    # BLAS may block a 5-row and a 9-row product differently: equal up to summation order
    np.testing.assert_allclose(a["y64"], b["y64"][:5], rtol=1e-12, atol=1e-13)
    # a token subset gives the same per-token results as the full evaluation
    s = li.oracle_forward(c9, d9, tokens=[7, 2])
    np.testing.assert_allclose(s["y64"], b["y64"][[7, 2]], rtol=1e-12, atol=1e-13)


def _signed_perm(rows, cols, rng, scale_code=127, value=1.0):
    """A [rows, cols] matrix with one +-value per row at a random column (distinct columns
    while they last). Returns (dense, col_index, sign)."""
    colidx = rng.permutation(max(rows, cols))[:rows] % cols
    sign = rng.choice([-1.0, 1.0], size=rows)
    M = np.zeros((rows, cols))
    M[np.arange(rows), colidx] = sign * value * 2.0 ** (scale_code - 127)
    return M, colidx, sign


def test_closed_form_with_signed_permutation_weights():
    rng = np.random.default_rng(11)
    c = li.small_config(T=6, n_experts=5, topk=2, shared_inter=64)
    H, L, I, Is, E = c.hidden, c.latent, c.inter, c.shared_inter, c.n_experts
    d = li.build(c, experts=False)
    # down: z[l] = x[pd[l]] * sd[l];  up: y_r[h] = c'[pu[h] ] * su[h]
    Dn, pd, sd = _signed_perm(L, H, rng)
    Up, pu, su = _signed_perm(H, L, rng)
    d["down"] = (np.ascontiguousarray(Dn, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    d["up"] = (np.ascontiguousarray(Up, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    recs_p, recs_s, perms = [], [], []
    for e in range(E):
        parts, meta = [], []
        for rows, cols, code, val in ((I, L, 126 + e % 3, 1.5), (I, L, 128, -2.0), (L, I, 125, 6.0)):
            M, idx, sg = _signed_perm(rows, cols, rng, code, val)
            parts.append(li.encode_mxfp4(M, np.full((rows, cols // 32), code)))
            meta.append((idx, sg * val * 2.0 ** (code - 127)))
        recs_p.append(np.concatenate([p.reshape(-1) for p, _ in parts]))
        recs_s.append(np.concatenate([s.reshape(-1) for _, s in parts]))
        perms.append(meta)
    d["exp_packed"], d["exp_scales"] = np.stack(recs_p), np.stack(recs_s)
    sh_parts, sh_meta = [], []
    for rows, cols, code, val in ((Is, H, 127, 1.0), (Is, H, 126, 3.0), (H, Is, 127, -0.5)):
        M, idx, sg = _signed_perm(rows, cols, rng, code, val)
        sh_parts.append(li.encode_mxfp4(M, np.full((rows, cols // 32), code)))
        sh_meta.append((idx, sg * val * 2.0 ** (code - 127)))
    d["shared"] = (np.concatenate([p.reshape(-1) for p, _ in sh_parts]),
                   np.concatenate([s.reshape(-1) for _, s in sh_parts]))
    out = li.oracle_forward(c, d)

    x = bf16_to_f64(d["x"])
    ids, w = out["route"]["ids"], out["route"]["weights"]
    silu = lambda v: v / (1 + np.exp(-v))
    for t in range(c.T):
        z = x[t, pd] * sd
        acc = np.zeros(L)
        for j in range(c.topk):
            (i1, a1), (i3, a3), (i2, a2) = perms[ids[t, j]]
            h = silu(z[i1] * a1) * (z[i3] * a3)
            acc += w[t, j] * h[i2] * a2
        np.testing.assert_allclose(out["c"][t], acc, rtol=1e-13, atol=1e-300)
        cn = acc / np.sqrt(np.mean(acc ** 2) + c.rms_eps) * bf16_to_f64(d["norm"])
        yr = cn[pu] * su
        (g1, b1), (g3, b3), (g2, b2) = sh_meta
        hs = silu(x[t, g1] * b1) * (x[t, g3] * b3)
        ys = hs[g2] * b2
        np.testing.assert_allclose(out["y_routed"][t], yr, rtol=1e-12, atol=1e-300)
        np.testing.assert_allclose(out["y_shared"][t], ys, rtol=1e-12, atol=1e-300)


def test_chain_input_closed_forms():
    """The stack's chaining step (weightless RMSNorm of a layer's bf16 output, rounded to
    bf16): a hand-computed row, constant rows, exact scale invariance with eps = 0, and
    unit RMS up to bf16 rounding."""
    f = lambda v: np.asarray(v, np.float32).view(np.uint32).__rshift__(16).astype(np.uint16)
    # [3, 4, 0, 0]: mean square 6.25, RMS 2.5 -> [1.2, 1.6, 0, 0], rounded to bf16 by hand:
    # 1.2 = 1.0011001|1001..b -> 1.0011010b = 0x3f9a; 1.6 = 1.1001100|1100..b -> 0x3fcd
    out = layer.chain_input(f([[3.0, 4.0, 0.0, 0.0]]), eps=0.0)
    assert out.tolist() == [[0x3F9A, 0x3FCD, 0, 0]]
    # constant rows normalise to +-1 exactly
    out = layer.chain_input(f([[7.5] * 8, [-0.25] * 8]), eps=0.0)
    assert (out[0] == 0x3F80).all() and (out[1] == 0xBF80).all()
    rng = np.random.default_rng(5)
    y = f(rng.standard_normal((6, 256)) * 300.0)
    y2 = f(bf16_to_f64(y) * 2.0)                       # exact: doubling a bf16 value
    assert np.array_equal(layer.chain_input(y, eps=0.0), layer.chain_input(y2, eps=0.0))
    rms = np.sqrt(np.mean(bf16_to_f64(layer.chain_input(y)) ** 2, axis=1))
    assert np.all(np.abs(rms - 1.0) <= 2.0 ** -8)
