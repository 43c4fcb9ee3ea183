"""GPU parity of the MXFP8 activation mode (MOE_ACT_MXFP8) against the oracle's
act="mxfp8" evaluation (marked gpu).

- moe_mxfp8_round bit-exact against oracle.mxfp8.quantize on bf16 inputs whose
  blocks span scales from 2^-90 to 2^92, with values down to 2^-20 of their
  block's largest (E4M3 subnormals and underflow to zero), exact E4M3 midpoints
  (ties to even), saturation past 448 * 2^s and all-zero blocks.
- The whole layer in MXFP8 mode on both expert paths, with the comparison
  protocol of the bf16 mode (ids and token lists bit-exact, tensors within
  max-rel 2e-2 and cosine 0.9995).
- The mode is not vacuous: the GPU's MXFP8 output is several times closer to
  the oracle's MXFP8 evaluation than the oracle's bf16 evaluation is.
"""
import numpy as np
import pytest

from tests import layer_inputs as li
from workload import gen

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

PATH_STREAM, PATH_MFMA = 1, 2
ACT_MXFP8 = 1


@pytest.fixture(scope="module", autouse=True)
def _gpu_available():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from latent_moe_expert_amd import _lib
    _lib.load()  # raises when the library is not built: there is no fallback


def _harness():
    from tests import gpu_harness
    return gpu_harness


def _round_inputs(rows=96, K=1024, seed=11):
    """bf16 bit patterns: per 32-block a random exponent in [-80, 100]; random signs and
    mantissas; some blocks hold values on E4M3 midpoints of their scale, some a value
    past the saturation point, some are all zero."""
    rng = np.random.default_rng(seed)
    G = K // 32
    e = rng.integers(-80, 101, size=(rows, G))
    mant = rng.uniform(1.0, 2.0, size=(rows, K))
    v = np.sign(rng.uniform(-1, 1, size=(rows, K))) * mant * np.ldexp(1.0, np.repeat(e, 32, axis=1)
                                                                     - rng.integers(0, 20, size=(rows, K)))
    # midpoints: unit values (m + 1/2) * 2^(k - 3) of the E4M3 grid, the block amax at 2^8 exactly
    for r in range(0, rows, 3):
        g = int(rng.integers(G))
        k = rng.integers(-6, 9, size=32)
        m = rng.integers(8, 16, size=32)
        unit = (m + 0.5) * np.ldexp(1.0, k - 3)
        unit[0] = 256.0
        unit = np.minimum(unit, 448.0)
        v[r, 32 * g:32 * g + 32] = np.ldexp(unit, int(e[r, g]) - 8) * np.sign(rng.uniform(-1, 1, 32))
    # saturation: 1.875 * 2^p (exact in bf16) as the block's largest value gives s = p - 8
    # and a unit value of 480 > 448
    for r in range(1, rows, 5):
        g = int(rng.integers(G))
        v[r, 32 * g] = np.ldexp(480.0, int(e[r, g]) - 8)
    for r in range(2, rows, 7):
        g = int(rng.integers(G))
        v[r, 32 * g:32 * g + 32] = 0.0
    from oracle.numerics import f64_to_bf16
    return f64_to_bf16(v)


def test_mxfp8_round_bit_exact():
    from latent_moe_expert_amd import layer as L
    from oracle import mxfp8
    from oracle.numerics import bf16_to_f64, f64_to_bf16
    H = _harness()
    xb = _round_inputs()
    ref = mxfp8.quantize(bf16_to_f64(xb))
    assert np.abs(ref[ref != 0]).min() >= 2.0 ** -126  # exact in bf16
    ref_bits = f64_to_bf16(ref)
    assert np.array_equal(bf16_to_f64(ref_bits), ref)
    x = H.to_dev_bf16(xb)
    y = torch.empty_like(x)
    L.moe_mxfp8_round(x, y)
    torch.cuda.synchronize()
    got = H.dev_bf16_to_bits(y)
    assert np.array_equal(got, ref_bits), f"{int((got != ref_bits).sum())} elements differ"
    # in place, and a row count that is not a multiple of the kernel's block
    x2 = H.to_dev_bf16(xb[:37])
    L.moe_mxfp8_round(x2, x2)
    torch.cuda.synchronize()
    assert np.array_equal(H.dev_bf16_to_bits(x2), ref_bits[:37])


def _run(c, expert_path, align_block=0):
    H = _harness()
    d = li.build(c)
    dl = H.DeviceLayer(c, dense={k: d[k] for k in ("down", "up", "norm", "router", "select_bias")},
                       experts=(d["exp_packed"], d["exp_scales"]))
    out = dl.run(d["x"], align_block=align_block, expert_path=expert_path, act_format=ACT_MXFP8)
    host = {**d, **dl.host_dense}
    ref = li.oracle_forward(c, host, align_block=out["B"], act="mxfp8")
    return out, ref, host


STREAM_CASES = [
    ("ragged37", dict(T=37, hidden=512, latent=512, n_experts=40, topk=6, inter=256, shared_inter=256)),
    ("multi_tile_experts", dict(T=64, hidden=256, latent=256, n_experts=8, topk=4, inter=512, shared_inter=256)),
    ("no_norm_no_shared", dict(T=19, hidden=512, latent=256, n_experts=12, topk=3, inter=256, shared_inter=0,
                               norm=False)),
    ("single_token", dict(T=1, hidden=256, latent=256, n_experts=10, topk=2, inter=256, shared_inter=256)),
]

MFMA_CASES = [
    ("two_windows", dict(T=96, hidden=1024, latent=1024, n_experts=8, topk=4, inter=1024, shared_inter=512)),
    ("ragged_no_shared", dict(T=37, hidden=512, latent=512, n_experts=40, topk=6, inter=512, shared_inter=0)),
    ("bias_rsf_three_windows", dict(T=200, hidden=512, latent=1536, n_experts=24, topk=5, inter=512,
                                    shared_inter=1024, routed_scaling_factor=2.446, zipf_s=1.1, zipf_c=0.05)),
    ("jobs_of_5_to_12_tiles", dict(T=512, hidden=512, latent=512, n_experts=8, topk=2, inter=512,
                                   shared_inter=512)),
    # a Zipf-skewed router: jobs of 1, 2, 3, 4, 5, 7 and 12 row tiles (every row-tile kernel)
    ("jobs_of_1_to_12_tiles_zipf", dict(T=224, hidden=512, latent=512, n_experts=20, topk=4, inter=512,
                                        shared_inter=512, zipf_s=1.1, zipf_c=0.5)),
]


@pytest.mark.parametrize("name,kw", STREAM_CASES, ids=[s[0] for s in STREAM_CASES])
def test_stream_path_mxfp8(name, kw):
    H = _harness()
    c = li.small_config(**kw)
    out, ref, _ = _run(c, PATH_STREAM)
    H.compare_layer(out, ref, c.T, c.topk, c.n_experts)


@pytest.mark.parametrize("name,kw", MFMA_CASES, ids=[s[0] for s in MFMA_CASES])
def test_mfma_path_mxfp8(name, kw):
    H = _harness()
    c = li.small_config(**kw)
    out, ref, _ = _run(c, PATH_MFMA)
    H.compare_layer(out, ref, c.T, c.topk, c.n_experts)


def test_mfma_path_mxfp8_align_block_48():
    H = _harness()
    c = li.small_config(T=70, n_experts=9, topk=3, hidden=512, latent=512, inter=512, shared_inter=0)
    out, ref, _ = _run(c, PATH_MFMA, align_block=48)
    assert out["B"] == 48
    H.compare_layer(out, ref, c.T, c.topk, c.n_experts)


@pytest.mark.parametrize("path", [PATH_STREAM, PATH_MFMA])
def test_mxfp8_mode_follows_mxfp8_numerics(path):
    """The routed output in MXFP8 mode sits far closer to the oracle's MXFP8 evaluation
    than to its bf16 one, so the mode does round the expert inputs."""
    H = _harness()
    c = li.small_config(T=64, hidden=512, latent=1024, n_experts=16, topk=4, inter=512, shared_inter=512)
    out, ref8, host = _run(c, path)
    ref16 = li.oracle_forward(c, host, align_block=out["B"], act="bf16")
    keep = ~ref8["route"]["near_tie"]
    gap_mode = H.maxrel(ref16["y_routed"][keep], ref8["y_routed"][keep])
    err = H.maxrel(out["y_routed"][keep], ref8["y_routed"][keep])
    print(f"  bf16 vs mxfp8 oracle: {gap_mode:.3e}; gpu mxfp8 vs mxfp8 oracle: {err:.3e}")
    assert gap_mode > 1e-2
    assert err < 0.25 * gap_mode


# ------------------------------------------------------------------ full K3 layer sizes

def _full_case(name, sample):
    H = _harness()
    c = gen.named_config(name)
    dl = H.k3_layer()
    x = gen.make_x(c)
    out = dl.run(x, act_format=ACT_MXFP8)
    ref = li.oracle_forward(c, {"x": x, **dl.host_dense, "shared": gen.make_shared(c)}, experts=dl.oracle_experts(),
                            align_block=out["B"], tokens=sample, act="mxfp8")
    H.compare_layer(out, ref, c.T, c.topk, c.n_experts)


@pytest.mark.fullsize
@pytest.mark.timeout(900)
def test_full_decode16_mxfp8():
    _full_case("decode16", sample=[0, 9, 15])


@pytest.mark.fullsize
@pytest.mark.timeout(900)
def test_full_prefill8192_mxfp8():
    _full_case("prefill8192", sample=[0, 4097, 8191])
