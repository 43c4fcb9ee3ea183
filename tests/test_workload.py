"""The seeded input generator: determinism, stream independence, recipes (CPU only)."""
import numpy as np

from workload import gen


def test_same_seed_same_bytes_and_independent_streams():
    c = gen.named_config("tiny")
    p0, s0 = gen.make_expert(c, 0, 3)
    p1, s1 = gen.make_expert(c, 0, 3)
    assert np.array_equal(p0, p1) and np.array_equal(s0, s1)
    q, _ = gen.make_expert(c, 0, 4)
    assert not np.array_equal(p0[:4096], q[:4096])
    r, _ = gen.make_expert(c, 1, 3)            # another layer
    assert not np.array_equal(p0[:4096], r[:4096])
    assert s0.min() >= 119 and s0.max() <= 123


def test_fill_experts_matches_single_generation():
    c = gen.LayerConfig("f", T=2, hidden=256, latent=128, n_experts=6, topk=2, inter=64, shared_inter=0)
    P = np.empty((3, gen.expert_record_bytes(c)), np.uint8)
    S = np.empty((3, gen.expert_scale_bytes(c)), np.uint8)
    gen.fill_experts(c, 0, P, S, experts=[5, 0, 2], threads=2)
    for i, e in enumerate([5, 0, 2]):
        p, s = gen.make_expert(c, 0, e)
        assert np.array_equal(P[i], p) and np.array_equal(S[i], s)


def test_x_is_prefix_consistent_and_bf16_of_normal():
    c = gen.named_config("decode16")
    a = gen.make_x(c, 0, T=16)
    b = gen.make_x(c, 0, T=40)
    assert np.array_equal(a, b[:16])
    v = (b.astype(np.uint32) << 16).view(np.float32)
    assert abs(v.mean()) < 0.02 and abs(v.std() - 1) < 0.02


def test_dense_recipe_shapes_and_scales():
    c = gen.LayerConfig("d", T=2, hidden=512, latent=256, n_experts=8, topk=2, inter=128, shared_inter=0)
    d = gen.make_dense(c)
    dn = (d["down"].astype(np.uint32) << 16).view(np.float32)
    assert d["down"].shape == (256, 512) and d["up"].shape == (512, 256)
    assert abs(dn.std() * np.sqrt(512) - 1) < 0.05
    assert d["router"].dtype == np.float32 and abs(d["router"].std() * np.sqrt(512) - 1) < 0.05
    u = gen.make_dense(c.with_(router_dist="uniform"))["router"]
    assert np.abs(u).max() <= np.sqrt(3 / 512) and abs(u.std() * np.sqrt(512) - 1) < 0.05
    z = gen.make_dense(c.with_(zipf_s=1.1, zipf_c=0.5))["select_bias"]
    assert np.isclose(z.max(), 0.5) and np.isclose(np.sort(z)[-2], 0.5 * 2 ** -1.1, rtol=1e-6)


def test_router_scores_and_bias_streams():
    """Seeded, reproducible, of the stated ranges, and independent of other streams."""
    from workload import gen
    a = gen.make_router_scores(64, 96, seed=3)
    b = gen.make_router_scores(64, 96, seed=3)
    assert a.dtype == np.float32 and a.shape == (64, 96) and np.array_equal(a, b)
    assert np.all((a > 0) & (a < 1))
    assert not np.array_equal(a, gen.make_router_scores(64, 96, seed=4))
    d = gen.make_router_scores(32, 40, seed=1, dyadic=True)
    assert np.all(d * 4096 == np.round(d * 4096)) and np.all((d > 0) & (d < 1))
    assert len(np.unique(d)) < d.size                      # exact ties occur
    s = gen.make_selection_bias(896, seed=0)
    assert s.dtype == np.float32 and abs(float(s.std()) - 0.05) < 0.01
    assert np.array_equal(s, gen.make_selection_bias(896, seed=0))


def test_stack_zipf_amplitude_matches_its_calibration():
    """The stacked workload's bias amplitude is the one tests/golden/zipf_amplitude.py found
    (hottest expert of layer 0 at about 10x the mean load, reading R13)."""
    import json
    import os
    rec = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "zipf_amplitude.json")))
    c = gen.named_config("stack8x4096")
    assert rec["workload"] == c.name and rec["zipf_s"] == c.zipf_s and rec["zipf_c"] == c.zipf_c
    assert abs(rec["ratio"] - 10.0) < 0.5
