"""GPU parity of stacked layers (marked gpu): the chaining step, chained layers against the
oracle's own chain, and the align entry point on ids a token repeats.

A stack feeds layer l+1 the weightless RMSNorm of layer l's bf16 output (reading R16,
oracle.layer.chain_input; on the GPU moe_rmsnorm). The oracle evaluates the chain from
its own outputs, never from the GPU's, so a chained layer's input on the GPU differs from
the oracle's by the previous layer's tolerance (measured: about 3e-3 relative RMS). The
router logits are linear in the input, so the logit difference that input difference
causes is exactly dl = (x_gpu - x_ref) . W_r^T; the sigmoid moves a key by at most
sigma'(xi) * |dl|, where xi is the point of [l - |dl|, l + |dl|] nearest 0 (sigma' peaks at
0). A token's selection is determined when the smallest selected key minus its bound still
exceeds the largest unselected key plus its bound; the other tokens are excluded from the
comparison and counted, like the 1e-6 near ties at the first layer. Only the oracle's own
logits and keys enter the rule, and nothing from the GPU becomes an oracle input.
"""
import numpy as np
import pytest

from tests import layer_inputs as li
from workload import gen

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

KEY_EPS = 1e-6   # fp32 routing on the GPU against fp64 in the oracle


def chained_bounds(ref, x_gpu_bits, x_ref_bits, router_w, rsf=1.0):
    """For a chained layer: (flags, w_tol). flags[t] = True when the input difference could
    change token t's selection (excluded); w_tol [T, k] bounds how far the routing weights
    w = s / sum(s_selected) * rsf can move, from the same per-score bounds |ds_e| <= b_e:
    |dw_j| <= (b_j S + s_j B) / (S (S - B)) * rsf with S = sum s, B = sum b over the selection."""
    from oracle.numerics import bf16_to_f64
    r = ref["route"]
    dl = np.abs((bf16_to_f64(x_gpu_bits) - bf16_to_f64(x_ref_bits)) @ np.asarray(router_w, np.float64).T)
    xi = np.maximum(0.0, np.abs(r["logits"]) - dl)
    sx = 1.0 / (1.0 + np.exp(-xi))
    bound = sx * (1.0 - sx) * dl + KEY_EPS
    T, E = r["keys"].shape
    ids = r["ids"].astype(np.int64)
    sel = np.zeros((T, E), dtype=bool)
    np.put_along_axis(sel, ids, True, axis=1)
    low = np.where(sel, r["keys"] - bound, np.inf).min(axis=1)
    high = np.where(sel, -np.inf, r["keys"] + bound).max(axis=1)
    s_sel = np.take_along_axis(r["scores"], ids, axis=1)
    b_sel = np.take_along_axis(bound, ids, axis=1)
    S, B = s_sel.sum(axis=1, keepdims=True), b_sel.sum(axis=1, keepdims=True)
    w_tol = (b_sel * S + s_sel * B) / (S * (S - B)) * abs(rsf) + 1e-6
    return ~(low > high), w_tol


@pytest.fixture(scope="module", autouse=True)
def _gpu_available():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from latent_moe_expert_amd import _lib
    _lib.load()


def _H():
    from tests import gpu_harness
    return gpu_harness


def _bits_ulp_diff(a, b):
    """|a - b| in bf16 units in the last place, for finite values of one sign."""
    return np.abs(a.astype(np.int32) - b.astype(np.int32))


@pytest.mark.parametrize("rows,cols,weighted,inplace", [(37, 7168, False, False), (5, 3584, True, False),
                                                        (1, 4, False, True), (64, 4100, True, True),
                                                        (300, 512, False, False)])
def test_rmsnorm_entry_point(rows, cols, weighted, inplace):
    """moe_rmsnorm against the oracle's RMSNorm rounded to bf16: equal bits, except values whose
    exact result lies within fp32 rounding of a bf16 rounding midpoint (one ulp apart)."""
    from latent_moe_expert_amd import layer as L
    from oracle.layer import rmsnorm
    from oracle.numerics import bf16_to_f64, f64_to_bf16
    H = _H()
    rng = np.random.default_rng(rows * 7 + cols)
    x = f64_to_bf16(rng.standard_normal((rows, cols)) * 300.0)
    g = f64_to_bf16(1.0 + 0.1 * rng.standard_normal(cols)) if weighted else None
    xd = H.to_dev_bf16(x)
    yd = xd if inplace else torch.empty_like(xd)
    L.moe_rmsnorm(xd, yd, None if g is None else H.to_dev_bf16(g), eps=1e-6)
    torch.cuda.synchronize()
    got = H.dev_bf16_to_bits(yd)
    ref = f64_to_bf16(rmsnorm(bf16_to_f64(x), None if g is None else bf16_to_f64(g), 1e-6))
    d = _bits_ulp_diff(got, ref)
    assert d.max() <= 1
    assert (d > 0).mean() <= 1e-3


@pytest.mark.parametrize("E,scale,reps", [(6, 1, 1), (5000, 800, 1),  # 5000: the hash-table align
                                          (6, 1, 40),    # 200 tokens: one block over 4 chunks
                                          (6, 1, 120)])  # 600 tokens: count, scan and scatter kernels
def test_align_repeated_ids_keep_first_slot(E, scale, reps):
    """A token that lists an expert twice: the first slot is placed, later ones are dropped
    (inv_pos -1), like ids out of range. Expected arrays by brute force on a small case (five
    tokens, repeated reps times)."""
    from latent_moe_expert_amd import layer as L
    k, B = 3, 4
    ids = np.array([[0, 2, 2], [5, 5, 5], [1, 3, 9], [3, 0, 3], [4, -1, 4]], np.int32)
    ids = np.tile(np.where(ids >= 0, ids * scale, ids).astype(np.int32), (reps, 1))
    T = ids.shape[0]
    keep = np.zeros_like(ids, dtype=bool)
    for t in range(T):
        seen = set()
        for j in range(k):
            e = int(ids[t, j])
            if 0 <= e < E and e not in seen:
                keep[t, j] = True
                seen.add(e)
    flat = ids.reshape(-1)
    kf = keep.reshape(-1)
    counts = np.array([int(((flat == e) & kf).sum()) for e in range(E)], np.int32)
    cap = B * ((T * k + min(E, T * k) * (B - 1)) // B)
    sorted_ref = np.full(cap, T * k, np.int32)
    eids_ref = np.full(cap // B, -1, np.int32)
    inv_ref = np.full(T * k, -1, np.int32)
    off = 0
    for e in range(E):
        members = [i for i in range(T * k) if kf[i] and flat[i] == e]
        for r, i in enumerate(members):
            sorted_ref[off + r] = i
            inv_ref[i] = off + r
        padded = -(-len(members) // B) * B
        eids_ref[off // B:(off + padded) // B] = e
        off += padded
    dev = "cuda"
    out = {n: torch.full((m,), -7, dtype=torch.int32, device=dev)
           for n, m in (("sorted", cap), ("eids", cap // B), ("num", 1), ("inv", T * k), ("counts", E))}
    scratch = torch.empty(max(1, L.moe_align_workspace_size(T, k, E)), dtype=torch.uint8, device=dev)
    for _ in range(2):   # deterministic from run to run
        L.moe_align_block_size(torch.from_numpy(ids).to(dev), T, k, E, B, out["sorted"], out["eids"], out["num"],
                               out["inv"], out["counts"], scratch)
        torch.cuda.synchronize()
        assert np.array_equal(out["sorted"].cpu().numpy(), sorted_ref)
        assert np.array_equal(out["eids"].cpu().numpy(), eids_ref)
        assert int(out["num"].item()) == off
        assert np.array_equal(out["inv"].cpu().numpy(), inv_ref)
        assert np.array_equal(out["counts"].cpu().numpy(), counts)


@pytest.mark.parametrize("path,kw", [
    (1, dict(T=48, hidden=512, latent=256, n_experts=24, topk=4, inter=256, shared_inter=256,
             zipf_s=1.1, zipf_c=0.05)),
    (2, dict(T=96, hidden=512, latent=512, n_experts=16, topk=4, inter=512, shared_inter=512)),
], ids=["stream", "mfma"])
def test_small_stack_chain_three_layers(path, kw):
    """Three layers with distinct seeded weights chained through moe_rmsnorm; every token of
    every layer against the oracle's own chain (oracle.layer.chain_input)."""
    from latent_moe_expert_amd import layer as L
    from oracle.layer import chain_input
    H = _H()
    c = li.small_config(**kw)
    x_host = gen.make_x(c, 0)
    x_dev = H.to_dev_bf16(x_host)
    x_ref = x_host
    diverged = np.zeros(c.T, dtype=bool)   # tokens whose routing differed within the bound at an earlier layer
    for layer in range(3):
        d = li.build(c, layer=layer)
        d["x"] = x_ref
        dl = H.DeviceLayer(c, layer=layer, dense={k: d[k] for k in ("down", "up", "norm", "router", "select_bias")},
                           experts=(d["exp_packed"], d["exp_scales"]))
        out = dl.run(x_dev=x_dev, expert_path=path, keep_y_dev=True)
        ref = li.oracle_forward(c, {**d, **dl.host_dense}, align_block=out["B"])
        if layer:
            x_gpu = H.dev_bf16_to_bits(x_dev)
            ok = ~diverged
            H.assert_close(f"layer {layer} input", H.bf16_bits_to_f64(x_gpu[ok]), H.bf16_bits_to_f64(x_ref[ok]))
            flags, w_tol = chained_bounds(ref, x_gpu, x_ref, d["router"], c.routed_scaling_factor)
            # a flagged token is excluded only when its selection did change; an unflagged one
            # must match exactly (compare_layer)
            changed = ~(out["topk_ids"] == ref["route"]["ids"]).all(axis=1)
            diverged |= flags & changed
            ref["route"]["near_tie"] = diverged.copy()
        else:
            w_tol = None
            changed = ~(out["topk_ids"] == ref["route"]["ids"]).all(axis=1)
            diverged |= ref["route"]["near_tie"] & changed
        print(f" layer {layer}:")
        H.compare_layer(out, ref, c.T, c.topk, c.n_experts, w_tol=w_tol)
        assert np.isfinite(H.bf16_bits_to_f64(out["y"])).all()
        nxt = torch.empty_like(out["y_dev"])
        L.moe_rmsnorm(out["y_dev"], nxt, None, eps=1e-6)
        x_dev = nxt
        x_ref = chain_input(ref["y"])


@pytest.mark.fullsize
@pytest.mark.timeout(900)
def test_full_stack_layer1_on_normalised_layer0_output():
    """Layers 0 and 1 of the 8-layer stack at full K3 size (T=4096, Zipf selection bias):
    layer 1 runs on moe_rmsnorm of layer 0's output. The oracle runs layer 0 for the sampled
    tokens, chains them (chain_input) and runs layer 1 on them; routing, the latent, the
    aggregate, the routed and shared outputs and y of layer 1 are compared per token."""
    from latent_moe_expert_amd import layer as L
    from oracle.layer import chain_input
    H = _H()
    c = gen.named_config("stack8x4096")
    l0 = H.k3_layer()
    dense0 = {**l0.host_dense, "select_bias": gen.make_dense(c, 0)["select_bias"]}
    saved = l0.bias
    l0.bias = torch.from_numpy(dense0["select_bias"]).cuda()
    x = gen.make_x(c)
    try:
        out0 = l0.run(x, taps=False, keep_y_dev=True)
    finally:
        l0.bias = saved
    x1_dev = torch.empty_like(out0["y_dev"])
    L.moe_rmsnorm(out0["y_dev"], x1_dev, None, eps=c.rms_eps)
    l1 = H.DeviceLayer(c, layer=1)
    l1_dense = l1.host_dense
    try:
        out1 = l1.run(x_dev=x1_dev)
    finally:
        del l1
        torch.cuda.empty_cache()
    counts = out1["counts"]
    hot = int(np.argmax(counts))
    print(f"  layer 1: hottest expert {hot} with {int(counts[hot])} pairs "
          f"({counts[hot] * c.n_experts / (c.T * c.topk):.1f}x the mean)")
    rng = np.random.default_rng(3)
    hot_tokens = np.nonzero((out1["topk_ids"] == hot).any(axis=1))[0]
    S = sorted({0, c.T - 1, int(hot_tokens[0]), int(hot_tokens[-1])} |
               set(rng.choice(c.T, size=12, replace=False).tolist()))
    ref0 = li.oracle_forward(c, {"x": x, **dense0, "shared": gen.make_shared(c, 0)}, experts=l0.oracle_experts(),
                             tokens=S)
    x1_ref = chain_input(ref0["y"])                                     # [|S|, H], the oracle's own chain
    H.assert_close("layer 1 input", H.bf16_bits_to_f64(H.dev_bf16_to_bits(x1_dev)[S]),
                   H.bf16_bits_to_f64(x1_ref))
    c1 = c.with_(T=len(S))
    ref1 = li.oracle_forward(c1, {"x": x1_ref, **l1_dense, "shared": gen.make_shared(c, 1)},
                             experts=lambda e: gen.make_expert(c, 1, e))
    x1_gpu = H.dev_bf16_to_bits(x1_dev)[S]
    flags, w_tol = chained_bounds(ref1, x1_gpu, x1_ref, l1_dense["router"], c.routed_scaling_factor)
    changed = ~(out1["topk_ids"][S] == ref1["route"]["ids"]).all(axis=1)
    keep = ~(flags & changed)      # unflagged tokens must match exactly
    print(f"  layer 1: {int(flags.sum())} of {len(S)} tokens within the input-difference bound, "
          f"{int((~keep).sum())} of them routed differently (excluded)")
    assert keep.sum() >= 4
    rows = np.asarray(S)[keep]
    assert np.array_equal(out1["topk_ids"][rows], ref1["route"]["ids"][keep])
    assert (np.abs(out1["topk_w"][rows] - ref1["route"]["weights"][keep]) <= w_tol[keep]).all()
    H.assert_close("z", H.bf16_bits_to_f64(out1["z"][rows]), ref1["z"][keep])
    H.assert_close("c", out1["c"][rows], ref1["c"][keep])
    H.assert_close("c_norm", H.bf16_bits_to_f64(out1["c_norm"][rows]), ref1["c_norm"][keep])
    H.assert_close("y_routed", out1["y_routed"][rows], ref1["y_routed"][keep])
    H.assert_close("y_shared", out1["y_shared"][rows], ref1["y_shared"][keep])
    H.assert_close("y", H.bf16_bits_to_f64(out1["y"][rows]), ref1["y64"][keep])
