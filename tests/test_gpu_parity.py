"""GPU parity: the HIP library against the CPU oracle (marked gpu).

Comparison protocol (per tensor): routing ids and per-expert token lists
bit-exact, near-tie tokens (k-th and (k+1)-th keys within 1e-6) excluded and
counted; routing weights within 1e-6; z, c, c_norm, y_routed, y_shared and y
each within max |gpu - ref| / max |ref| <= 2e-2 and cosine >= 0.9995 (bf16
activations with fp32 accumulation against a float64 evaluation).
"""
import numpy as np
import pytest

from tests import layer_inputs as li
from workload import gen

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_available():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from latent_moe_expert_amd import _lib
    _lib.load()  # raises when the library is not built: there is no fallback


def _harness():
    from tests import gpu_harness
    return gpu_harness


PATH_STREAM, PATH_MFMA = 1, 2


def _run_small(c, align_block=0, dense=None, experts=None, expert_path=0):
    H = _harness()
    d = li.build(c) if experts is None else experts
    dl = H.DeviceLayer(c, dense=dense if dense is not None else {k: d[k] for k in
                                                                  ("down", "up", "norm", "router", "select_bias")},
                       experts=(d["exp_packed"], d["exp_scales"]))
    out = dl.run(d["x"], align_block=align_block, expert_path=expert_path)
    ref = li.oracle_forward(c, {**d, **dl.host_dense}, align_block=out["B"])
    return out, ref, d


SMALL = [
    # (name, config kwargs): several row tiles, ragged token tails, norm on/off, shared on/off
    ("ragged37", dict(T=37, hidden=512, latent=512, n_experts=40, topk=6, inter=256, shared_inter=256)),
    ("multi_tile_experts", dict(T=64, hidden=256, latent=256, n_experts=8, topk=4, inter=512, shared_inter=256)),
    ("no_norm_no_shared", dict(T=19, hidden=512, latent=256, n_experts=12, topk=3, inter=256, shared_inter=0,
                               norm=False)),
    ("single_token", dict(T=1, hidden=256, latent=256, n_experts=10, topk=2, inter=256, shared_inter=256)),
    ("rsf_and_bias", dict(T=23, hidden=256, latent=256, n_experts=24, topk=5, inter=256, shared_inter=256,
                          routed_scaling_factor=2.446, zipf_s=1.1, zipf_c=0.05)),
    # decode batches outside the one-launch routing (E > 1024, k > 16): separate split-K sums,
    # the sorting router and align, then the column-spread combine
    ("experts_over_1024", dict(T=12, hidden=256, latent=512, n_experts=1100, topk=8, inter=256, shared_inter=0)),
    ("topk_over_16", dict(T=9, hidden=256, latent=256, n_experts=64, topk=24, inter=256, shared_inter=256)),
    # the widest latent the boundary takes: 32 column blocks per token in the combine
    ("latent_8192", dict(T=5, hidden=256, latent=8192, n_experts=6, topk=2, inter=256, shared_inter=0)),
    # above 4096 experts: the radix-select router and the hash-table align (one chunk, then several)
    ("experts_over_4096", dict(T=20, hidden=256, latent=256, n_experts=5000, topk=16, inter=256, shared_inter=0)),
    ("experts_over_4096_chunks", dict(T=100, hidden=256, latent=256, n_experts=5000, topk=8, inter=256,
                                      shared_inter=256)),
]


@pytest.mark.parametrize("name,kw", SMALL, ids=[s[0] for s in SMALL])
def test_small_layer_parity(name, kw):
    H = _harness()
    c = li.small_config(**kw)
    out, ref, _ = _run_small(c)
    H.compare_layer(out, ref, c.T, c.topk, c.n_experts)


# The scaled-MFMA expert path: sizes multiples of 512, several K windows, experts split
# into several jobs of at most 192 slots, ragged tails, dense shared rows over two jobs.
MFMA_SMALL = [
    ("two_windows", dict(T=96, hidden=1024, latent=1024, n_experts=8, topk=4, inter=1024, shared_inter=512)),
    ("experts_over_160_slots_k_eq_E", dict(T=256, hidden=512, latent=512, n_experts=4, topk=4, inter=512,
                                           shared_inter=512, norm=False)),
    ("ragged_no_shared", dict(T=37, hidden=512, latent=512, n_experts=40, topk=6, inter=512, shared_inter=0)),
    ("bias_rsf_three_windows", dict(T=200, hidden=512, latent=1536, n_experts=24, topk=5, inter=512,
                                    shared_inter=1024, routed_scaling_factor=2.446, zipf_s=1.1, zipf_c=0.05)),
    # about 128 slots per expert: jobs of 5 to 12 row tiles (every row-count bucket)
    ("jobs_of_5_to_12_tiles", dict(T=512, hidden=512, latent=512, n_experts=8, topk=2, inter=512,
                                   shared_inter=512)),
    # a Zipf-skewed router: jobs of 1, 2, 3, 4, 5, 7 and 12 row tiles, so the 2-, 4-, 6-, 8- and
    # 12-tile kernels each run jobs with fewer valid tiles than they cover
    ("jobs_of_1_to_12_tiles_zipf", dict(T=224, hidden=512, latent=512, n_experts=20, topk=4, inter=512,
                                        shared_inter=512, zipf_s=1.1, zipf_c=0.5)),
    # a latent above 4096: the bf16-O combine's threads take four 8-column vectors of the row
    ("latent_4608", dict(T=96, hidden=512, latent=4608, n_experts=8, topk=4, inter=512, shared_inter=512)),
    # 128 x 128 dense tiles with more tiles than compute units (9 x 32 for the up-projection), so
    # the up-projection is not split over K and adds the shared output in bf16
    ("mid_rows_unsplit_up_projection", dict(T=1100, hidden=4096, latent=512, n_experts=16, topk=4, inter=512,
                                            shared_inter=512)),
]


# The MFMA path at intermediate widths of the K3 family (1536 and 3072 GLU columns, multiples
# of 3 x 512): 9..12-tile jobs, two-job experts next to two dense shared jobs, three windows.
MFMA_WIDE = [
    # jobs of 9..11 row tiles (3 row tiles per row-wave, the last wave partly or wholly past the
    # valid rows), ragged tails
    ("wide_buckets", dict(T=430, hidden=512, latent=512, n_experts=8, topk=3, inter=1536, shared_inter=0)),
    # k = E: each expert gets every token (280 slots, two jobs), shared experts over two dense jobs
    ("wide_split_jobs_shared", dict(T=280, hidden=1536, latent=1024, n_experts=4, topk=4, inter=1536,
                                    shared_inter=1536, norm=False)),
    # small jobs and three K windows of the latent
    ("wide_three_windows", dict(T=61, hidden=512, latent=1536, n_experts=12, topk=3, inter=3072,
                                shared_inter=1536, routed_scaling_factor=2.446, zipf_s=1.1, zipf_c=0.05)),
]


@pytest.mark.parametrize("name,kw", MFMA_WIDE, ids=[s[0] for s in MFMA_WIDE])
def test_mfma_path_k3_widths_parity(name, kw):
    H = _harness()
    c = li.small_config(**kw)
    out, ref, d = _run_small(c, expert_path=PATH_MFMA)
    H.compare_layer(out, ref, c.T, c.topk, c.n_experts)


@pytest.mark.parametrize("name,kw", MFMA_SMALL, ids=[s[0] for s in MFMA_SMALL])
def test_mfma_path_parity(name, kw):
    H = _harness()
    c = li.small_config(**kw)
    out, ref, _ = _run_small(c, expert_path=PATH_MFMA)
    H.compare_layer(out, ref, c.T, c.topk, c.n_experts)


def test_both_paths_on_one_input():
    """The same layer through the streaming and the MFMA expert kernels: each within
    the tolerance of the oracle."""
    H = _harness()
    c = li.small_config(T=64, hidden=512, latent=1024, n_experts=16, topk=4, inter=512, shared_inter=512)
    d = li.build(c)
    dl = H.DeviceLayer(c, dense={k: d[k] for k in ("down", "up", "norm", "router", "select_bias")},
                       experts=(d["exp_packed"], d["exp_scales"]))
    a = dl.run(d["x"], expert_path=PATH_STREAM)
    b = dl.run(d["x"], expert_path=PATH_MFMA)
    ref = li.oracle_forward(c, {**d, **dl.host_dense}, align_block=a["B"])
    H.compare_layer(a, ref, c.T, c.topk, c.n_experts)
    H.compare_layer(b, ref, c.T, c.topk, c.n_experts)


def test_mfma_path_align_block_48():
    """Jobs follow the expert segments of a B = 48 layout."""
    H = _harness()
    c = li.small_config(T=70, n_experts=9, topk=3, hidden=512, latent=512, inter=512, shared_inter=0)
    out, ref, _ = _run_small(c, align_block=48, expert_path=PATH_MFMA)
    assert out["B"] == 48
    H.compare_layer(out, ref, c.T, c.topk, c.n_experts)


@pytest.mark.parametrize("B", [32, 48])
def test_align_block_multiple_of_16(B):
    """Layout blocks of B = 32 or 48 slots read by the 16-slot kernel tiles (ids expanded B/16 times)."""
    H = _harness()
    c = li.small_config(T=29, n_experts=9, topk=3, hidden=256, latent=256, inter=256, shared_inter=0)
    out, ref, _ = _run_small(c, align_block=B)
    assert out["B"] == B
    H.compare_layer(out, ref, c.T, c.topk, c.n_experts)


@pytest.mark.parametrize("n_experts", [40, 37])
def test_dense_projections_256_tiles_all_rows(n_experts):
    """T = 2100 tokens take the 256 x 224 dense-projection tiles (M >= 2048): a ragged last
    M tile (52 rows), partial N tiles (z: 768 = 3 x 224 + 96 columns; the router's 40 or 37 of
    224 rows, K = 3 x hidden; the up-projection's 1024 = 4 x 224 + 128 with the shared addend);
    every token compared. With 37 experts the router's output rows are 37 floats apart, so its
    tiles take the element-by-element epilogue instead of the 16-byte stores."""
    H = _harness()
    c = li.small_config(T=2100, hidden=1024, latent=768, n_experts=n_experts, topk=3, inter=256, shared_inter=256)
    out, ref, _ = _run_small(c)
    H.compare_layer(out, ref, c.T, c.topk, c.n_experts)


def test_k_equals_E_dense_equivalence():
    H = _harness()
    c = li.small_config(T=9, n_experts=6, topk=6, hidden=256, latent=256, inter=256, shared_inter=0, norm=False)
    out, ref, _ = _run_small(c)
    H.compare_layer(out, ref, c.T, c.topk, c.n_experts)
    assert np.all(out["topk_ids"] == np.arange(6))


def test_expert_ids_above_255():
    """Experts 255, 256 and 299 forced through the selection bias must all run."""
    H = _harness()
    c = li.small_config(T=12, n_experts=300, topk=4, hidden=256, latent=256, inter=256, shared_inter=0)
    d = li.build(c)
    bias = np.zeros(c.n_experts, np.float32)
    bias[[255, 256, 299]] = 3.0
    d["select_bias"] = bias
    dl = H.DeviceLayer(c, dense={k: d[k] for k in ("down", "up", "norm", "router", "select_bias")},
                       experts=(d["exp_packed"], d["exp_scales"]))
    out = dl.run(d["x"])
    ref = li.oracle_forward(c, d, align_block=out["B"])
    assert np.all(np.isin([255, 256, 299], out["topk_ids"]).all())
    assert all({255, 256, 299} <= set(r) for r in out["topk_ids"].tolist())
    H.compare_layer(out, ref, c.T, c.topk, c.n_experts)
    assert np.abs(out["y_routed"]).max() > 0


def test_empty_batch_enqueues_nothing():
    H = _harness()
    from latent_moe_expert_amd import layer as L
    c = li.small_config(T=3, hidden=256, latent=256, n_experts=6, topk=2, inter=256, shared_inter=256)
    d = li.build(c)
    dl = H.DeviceLayer(c, dense={k: d[k] for k in ("down", "up", "norm", "router", "select_bias")},
                       experts=(d["exp_packed"], d["exp_scales"]))
    dims = dl.dims(0)
    x = torch.empty((0, c.hidden), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((0, c.hidden), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    L.moe_latent_forward(dims, x, dl.down, dl.norm, dl.router, dl.bias, dl.packed, dl.scales, dl.up, dl.sh_packed,
                         dl.sh_scales, c.topk, y, ws)
    torch.cuda.synchronize()


def test_determinism_bitwise():
    H = _harness()
    c = li.small_config(T=33, n_experts=20, topk=4, hidden=512, latent=256, inter=256, shared_inter=256)
    d = li.build(c)
    dl = H.DeviceLayer(c, dense={k: d[k] for k in ("down", "up", "norm", "router", "select_bias")},
                       experts=(d["exp_packed"], d["exp_scales"]))
    a, b = dl.run(d["x"]), dl.run(d["x"])
    for k in ("y", "z", "c", "y_routed", "y_shared", "sorted_ids", "topk_w"):
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("T,k,E,B,seed", [(5, 2, 8, 16, 0), (300, 16, 896, 16, 1), (1000, 4, 37, 32, 2),
                                          (8192, 16, 896, 16, 3), (64, 8, 4096, 16, 4), (1, 1, 1, 1, 5),
                                          (130, 3, 3, 64, 6),
                                          # above 4096 experts the chunk masks live in an LDS hash table
                                          (48, 16, 65535, 16, 7), (300, 64, 20000, 16, 8), (1000, 8, 4097, 32, 9),
                                          (70, 2, 65535, 1, 10),
                                          # one block for up to 8 chunks of 64 tokens (masks in LDS)
                                          (512, 16, 896, 16, 11), (190, 8, 1500, 48, 13),
                                          # past the one-block limits: 9 chunks, or masks above 64 KB
                                          (520, 16, 896, 16, 14), (200, 8, 2000, 16, 12)])
def test_moe_align_block_size_bit_exact_on_oracle_ids(T, k, E, B, seed):
    """The align entry point on ids the oracle routed (here: random distinct ids),
    bit-exact on every array including the padded tail."""
    from latent_moe_expert_amd import layer as L
    from oracle.layer import align
    rng = np.random.default_rng(seed)
    ids = np.stack([np.sort(rng.choice(E, size=k, replace=False)) for _ in range(T)]).astype(np.int32)
    ref = align(ids, E, B)
    cap = ref["cap"]
    dev = "cuda"
    t_ids = torch.from_numpy(ids).to(dev)
    sorted_ids = torch.full((cap,), -7, dtype=torch.int32, device=dev)
    expert_ids = torch.full((cap // B,), -7, dtype=torch.int32, device=dev)
    num_post = torch.zeros(1, dtype=torch.int32, device=dev)
    inv_pos = torch.zeros(T * k, dtype=torch.int32, device=dev)
    counts = torch.zeros(E, dtype=torch.int32, device=dev)
    scratch = torch.empty(max(1, L.moe_align_workspace_size(T, k, E)), dtype=torch.uint8, device=dev)
    L.moe_align_block_size(t_ids, T, k, E, B, sorted_ids, expert_ids, num_post, inv_pos, counts, scratch)
    torch.cuda.synchronize()
    assert np.array_equal(sorted_ids.cpu().numpy(), ref["sorted_ids"])
    assert np.array_equal(expert_ids.cpu().numpy(), ref["expert_ids"])
    assert int(num_post.item()) == ref["num_post"]
    assert np.array_equal(inv_pos.cpu().numpy(), ref["inv_pos"])
    assert np.array_equal(counts.cpu().numpy(), ref["counts"])


@pytest.mark.parametrize("T,E,k", [(50, 64, 8),
                                   # one wave per token, 2 / 4 / 8 / 16 keys per lane
                                   (37, 100, 6), (200, 256, 16), (130, 500, 16), (300, 896, 16),
                                   (65, 1024, 16),
                                   # 17 to 4096 experts or k above 16: the LDS bitonic sort
                                   (40, 300, 24),
                                   # above 4096 experts: the radix-select router
                                   (20, 5000, 16), (6, 65535, 64)])
def test_moe_route_entry_point(T, E, k):
    from latent_moe_expert_amd import layer as L
    from oracle.layer import route
    H = _harness()
    c = li.small_config(T=T, n_experts=E, topk=k, hidden=512, latent=256, inter=256, shared_inter=256)
    d = li.build(c, experts=False)
    dims = L.make_dims(c.T, c.hidden, c.latent, c.n_experts, c.inter, c.shared_inter)
    x = H.to_dev_bf16(d["x"])
    ids = torch.empty((c.T, c.topk), dtype=torch.int32, device="cuda")
    w = torch.empty((c.T, c.topk), dtype=torch.float32, device="cuda")
    lg = torch.empty((c.T, c.n_experts), dtype=torch.float32, device="cuda")
    L.moe_route(dims, x, torch.from_numpy(d["router"]).cuda(), None, c.topk, ids, w, lg)
    torch.cuda.synchronize()
    r = route(H.bf16_bits_to_f64(d["x"]), d["router"], None, c.topk)
    keep = ~r["near_tie"]
    assert np.array_equal(ids.cpu().numpy()[keep], r["ids"][keep])
    assert np.abs(w.cpu().numpy()[keep] - r["weights"][keep]).max() <= 1e-6
    assert np.abs(lg.cpu().numpy() - r["logits"]).max() <= 1e-5 * np.abs(r["logits"]).max()


@pytest.mark.parametrize("E,n_top", [(128, 70), (128, 40), (896, 0), (1024, 17)])
def test_decode_route_exact_ties(E, n_top):
    """Keys tied exactly at the top (zero router: every score 0.5; bias 1 on n_top experts, 0
    elsewhere): the 16 lowest ids among the top keys win (all 16 lowest ids when nothing is
    biased), each with weight rsf / 16, and the layout is the oracle's align of those ids. The
    near-tie rule of the other parity tests excludes exactly these tokens, so here the expected
    ids follow from the tie rule itself."""
    from oracle.layer import align
    H = _harness()
    c = li.small_config(T=5, n_experts=E, topk=16, hidden=256, latent=256, inter=256, shared_inter=0)
    d = li.build(c)
    rng = np.random.default_rng(E + n_top)
    top = np.sort(rng.choice(E, size=n_top, replace=False)) if n_top else np.arange(0)
    bias = np.zeros(E, np.float32)
    bias[top] = 1.0
    dense = {"down": d["down"], "up": d["up"], "norm": d["norm"], "router": np.zeros_like(d["router"]),
             "select_bias": bias}
    dl = H.DeviceLayer(c, dense=dense, experts=(d["exp_packed"], d["exp_scales"]))
    out = dl.run(d["x"])
    want = top[:16] if n_top >= 16 else np.arange(16)
    assert (out["topk_ids"] == want[None, :].astype(np.int32)).all()
    assert (out["topk_w"] == np.float32(c.routed_scaling_factor / 16)).all()
    ref = align(out["topk_ids"].astype(np.int64), E, out["B"])
    n = ref["num_post"]
    assert int(out["num_post"][0]) == n
    assert np.array_equal(out["sorted_ids"][:n], ref["sorted_ids"][:n])
    assert np.array_equal(out["inv_pos"], ref["inv_pos"])


@pytest.mark.parametrize("E,case", [(128, "tied"), (896, "tied"), (896, "biased"), (1024, "biased"),
                                    (1024, "over_64_candidates"), (300, "over_64_candidates")])
def test_route_entry_exact_ties(E, case):
    """moe_route with a zero router (every score 0.5) and a selection bias that ties keys
    exactly: the 16 lowest ids among the largest keys win, each with weight 1/16.
    "over_64_candidates": the 16 lanes holding experts e % 64 < 16 get biases 2 + 0.01 * (e % 64),
    equal within a lane, so the keys at or above the 16th-largest lane maximum number more than
    64 and the one-wave router takes its successive-maxima path; the winners are all the experts
    with e % 64 == 15 (the largest key), lowest ids first."""
    from latent_moe_expert_amd import layer as L
    H = _harness()
    T, k = 70, 16
    c = li.small_config(T=T, n_experts=E, topk=k, hidden=256, latent=256, inter=256, shared_inter=0)
    d = li.build(c, experts=False)
    bias = np.zeros(E, np.float32)
    if case == "biased":
        top = np.sort(np.random.default_rng(E).choice(E, size=40, replace=False))
        bias[top] = 1.0
        want = top[:k]
    elif case == "over_64_candidates":
        e = np.arange(E)
        lanes = e % 64
        bias[lanes < 16] = (2.0 + 0.01 * lanes[lanes < 16]).astype(np.float32)
        want = e[lanes == 15][:k]
        assert len(want) == k or E < 64 * k
    else:
        want = np.arange(k)
    dims = L.make_dims(c.T, c.hidden, c.latent, c.n_experts, c.inter, c.shared_inter)
    x = H.to_dev_bf16(d["x"])
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    router = torch.zeros((E, c.hidden), dtype=torch.float32, device="cuda")
    L.moe_route(dims, x, router, torch.from_numpy(bias).cuda(), k, ids, w, lg)
    torch.cuda.synchronize()
    if len(want) < k:  # fewer experts with the largest key than k: the next lane's follow
        order = sorted(range(E), key=lambda i: (-float(np.float32(0.5) + bias[i]), i))
        want = np.sort(np.array(order[:k]))
    assert (ids.cpu().numpy() == np.asarray(want, np.int32)[None, :]).all()
    assert (w.cpu().numpy() == np.float32(1.0 / k)).all()


def test_route_dump_appends_each_forward(tmp_path, monkeypatch):
    """MOE_DUMP_ROUTE=path: every forward appends its top-k ids and weights, equal to the taps."""
    from latent_moe_expert_amd import layer as L
    H = _harness()
    c = li.small_config(T=21, n_experts=40, topk=6, hidden=512, latent=256, inter=256, shared_inter=256)
    d = li.build(c)
    dl = H.DeviceLayer(c, dense={k: d[k] for k in ("down", "up", "norm", "router", "select_bias")},
                       experts=(d["exp_packed"], d["exp_scales"]))
    path = tmp_path / "route.bin"
    monkeypatch.setenv("MOE_DUMP_ROUTE", str(path))
    outs = [dl.run(d["x"]), dl.run(d["x"][:9])]
    monkeypatch.delenv("MOE_DUMP_ROUTE")
    dl.run(d["x"])  # unset: nothing appended
    recs = L.read_route_dump(str(path))
    assert len(recs) == 2
    for rec, out in zip(recs, outs):
        assert rec["n_experts"] == c.n_experts
        assert np.array_equal(rec["topk_ids"], out["topk_ids"])
        assert np.array_equal(rec["topk_w"], out["topk_w"])


def test_tiny_named_config_full_width():
    """T=4, hidden 7168, latent 3584, 16 experts, top-4, intermediate 3072, no norm, no shared."""
    H = _harness()
    c = gen.named_config("tiny")
    dl = H.DeviceLayer(c)
    x = gen.make_x(c)
    out = dl.run(x)
    ref = li.oracle_forward(c, {"x": x, **dl.host_dense, "shared": None}, experts=dl.oracle_experts(),
                            align_block=out["B"])
    H.compare_layer(out, ref, c.T, c.topk, c.n_experts)


# ------------------------------------------------------------------ full K3 layer sizes

SLOTS_PER_JOB = 192      # the MFMA path's job size (12 row tiles of 16)


def _job_table(counts, spj=SLOTS_PER_JOB):
    """(expert, first slot within the expert, valid slots) per job, in the order the MFMA
    path numbers its jobs: experts ascending, each split into chunks of spj slots."""
    jobs = []
    for e, n in enumerate(counts.tolist()):
        for f in range(0, n, spj):
            jobs.append((e, f, min(spj, n - f)))
    return jobs


def _tile_bucket(nvalid):
    tiles = -(-nvalid // 16)
    return 4 if tiles <= 4 else 8 if tiles <= 8 else 10 if tiles <= 10 else 12


def _pick_mfma_cases(out, k, n_random, seed):
    """Experts whose every slot is compared (tap O) and tokens whose outputs are compared,
    chosen from the job table so that they cover: every row-tile bucket (4/8/10/12), all 8
    XCD classes (job index mod 8), the last job, an expert split over several jobs, the
    last valid row of a full 192-slot job, a row of a later job and a partial 16-row tile."""
    counts = out["counts"]
    jobs = _job_table(counts)
    experts, tokens = [], set()
    want_bucket = {4, 8, 10, 12}
    want_xcd = set(range(8))
    for j, (e, f, n) in enumerate(jobs):
        b, x = _tile_bucket(n), j % 8
        if b in want_bucket or x in want_xcd:
            if e not in experts:
                experts.append(e)
            want_bucket.discard(b)
            want_xcd.discard(x)
        if not want_bucket and not want_xcd:
            break
    last_e = jobs[-1][0]
    if last_e not in experts:
        experts.append(last_e)
    hot = int(np.argmax(counts))
    if hot not in experts:
        experts.append(hot)
    # tokens at chosen slots of chosen jobs, read from the GPU's expert-sorted layout
    s, ex, B = out["sorted_ids"], out["expert_ids"], out["B"]
    n_post = int(out["num_post"][0])

    def token_at(e, slot):
        blocks = np.nonzero(ex[: n_post // B] == e)[0]
        return int(s[blocks[0] * B + slot]) // k

    if counts[hot] > SLOTS_PER_JOB:
        tokens.add(token_at(hot, SLOTS_PER_JOB - 1))         # last valid row of a full job
        tokens.add(token_at(hot, int(counts[hot]) - 1))      # a row of the last (later) job
    for e in experts:
        n = int(counts[e])
        tokens.add(token_at(e, n - 1))                       # last valid row (a partial tile if n % 16)
    rng = np.random.default_rng(seed)
    T = out["topk_ids"].shape[0]
    tokens |= set(rng.choice(T, size=n_random, replace=False).tolist()) | {0, T - 1}
    return experts, sorted(tokens)


def _full_case(name, sample=None, n_random=12, o_experts=None, seed=0):
    """One K3 layer at full size: routing and align for every token, numeric outputs on the
    sampled tokens, and every slot of selected experts (tap O) on either expert path."""
    H = _harness()
    c = gen.named_config(name)
    dl = H.k3_layer()
    dense = dl.host_dense
    if c.router_dist != "normal":   # decode256: uniform router, same experts
        dense = {**dense, "router": gen.make_dense(c)["router"]}
        dl.router = torch.from_numpy(dense["router"]).cuda()
    x = gen.make_x(c)
    try:
        out = dl.run(x, with_O=True)
    finally:
        if c.router_dist != "normal":
            dl.router = torch.from_numpy(dl.host_dense["router"]).cuda()
    if o_experts is None:
        experts, tokens = _pick_mfma_cases(out, c.topk, n_random, seed)
    else:
        experts, tokens = o_experts(out), []
    if sample is not None:
        tokens = sorted(set(tokens) | set(sample))
    print(f"  {name}: {len(tokens)} tokens, every slot of experts {experts}")
    ref = li.oracle_forward(c, {"x": x, **dense, "shared": gen.make_shared(c)}, experts=dl.oracle_experts(),
                            align_block=out["B"], tokens=tokens)
    H.compare_layer(out, ref, c.T, c.topk, c.n_experts)
    H.expert_outputs_check(out, c, x, dense["down"], dl.oracle_experts(), experts, c.topk)


def _busiest(n):
    return lambda out: [int(e) for e in np.argsort(-out["counts"], kind="stable")[:n]]


@pytest.mark.fullsize
@pytest.mark.timeout(900)
def test_full_decode16():
    """Every one of the 16 tokens, and every slot of the 4 busiest experts."""
    _full_case("decode16", sample=list(range(16)), o_experts=_busiest(4))


@pytest.mark.fullsize
@pytest.mark.timeout(900)
def test_full_decode256():
    """24 tokens spread over the batch, and every slot of the 6 busiest experts."""
    _full_case("decode256", sample=list(range(3, 256, 11)), o_experts=_busiest(6))


@pytest.mark.fullsize
@pytest.mark.timeout(900)
def test_full_prefill8192():
    """The MFMA path at 8192 tokens: every slot of experts chosen to cover each row-tile
    bucket, all 8 XCD classes, the last job and the busiest expert; tokens at job
    boundaries and partial tiles plus random ones."""
    _full_case("prefill8192", n_random=14, seed=1)


@pytest.mark.fullsize
@pytest.mark.timeout(900)
def test_full_stack_layer_zipf_hot_experts():
    """Layer 0 of the 8-layer stack workload: T=4096 with the Zipf(1.1) selection bias, where
    the hottest expert takes ~731 of the 65536 pairs (about 10x the mean) and is split over
    four MFMA jobs. Same weights as the decode workloads (layer 0), plus the bias."""
    H = _harness()
    c = gen.named_config("stack8x4096")
    dl = H.k3_layer()
    dense = {**dl.host_dense, "select_bias": gen.make_dense(c)["select_bias"]}
    x = gen.make_x(c)
    saved = dl.bias
    dl.bias = torch.from_numpy(dense["select_bias"]).cuda()
    try:
        out = dl.run(x, with_O=True)
    finally:
        dl.bias = saved
    counts = out["counts"]
    hot = int(np.argmax(counts))
    assert counts[hot] > 3 * SLOTS_PER_JOB  # four jobs
    experts, tokens = _pick_mfma_cases(out, c.topk, n_random=8, seed=2)
    print(f"  hottest expert {hot}: {int(counts[hot])} pairs; {len(tokens)} tokens; experts {experts}")
    ref = li.oracle_forward(c, {"x": x, **dense, "shared": gen.make_shared(c)}, experts=dl.oracle_experts(),
                            align_block=out["B"], tokens=tokens)
    H.compare_layer(out, ref, c.T, c.topk, c.n_experts)
    H.expert_outputs_check(out, c, x, dense["down"], dl.oracle_experts(), experts, c.topk)
