"""GPU parity of the Quantile Balancing kernels (moe_qb_histogram, moe_qb_bias)
against oracle/qb.py (marked gpu).

Everything here is integer or an fp32 decision, so the bar is bit-exact:
- alpha, each token's (k+1)-th largest biased key, equal as fp32 bit patterns;
- the per-expert 1000-bin margin histograms, equal as integers;
- the new bias, equal as fp32 bit patterns to the oracle's search over the
  oracle's own histograms, and within one bin width above the exact quantile.
Cases: the K3 router shape (896 experts, top-16) with and without a bias, many
exact ties (dyadic scores), an expert count that is not a multiple of 4, more
than 1024 experts, the 4096-expert limit, margins clamped into the end bins,
no tokens, the histograms of two batches summed (the all-reduce) against the
union, and a target that no histogram reaches (NaN).
"""
import numpy as np
import pytest

from oracle import qb
from workload import gen

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_available():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from latent_moe_expert_amd import _lib
    _lib.load()  # raises when the library is not built: there is no fallback


def _api():
    from latent_moe_expert_amd import layer
    return layer


def _gpu_qb(s: np.ndarray, b, k: int, m_total=None):
    L = _api()
    m, n = s.shape
    dev = torch.device("cuda")
    sd = torch.from_numpy(s).to(dev)
    bd = None if b is None else torch.from_numpy(b).to(dev)
    alpha = torch.full((max(m, 1),), float("nan"), dtype=torch.float32, device=dev)[:m]
    hist = torch.full((n, qb.QB_BINS), -7, dtype=torch.int32, device=dev)
    nb = torch.full((n,), 123.0, dtype=torch.float32, device=dev)
    L.moe_qb_histogram(sd, bd, k, alpha, hist)
    L.moe_qb_bias(hist, m if m_total is None else m_total, k, nb)
    torch.cuda.synchronize()
    return alpha.cpu().numpy(), hist.cpu().numpy().astype(np.int64), nb.cpu().numpy()


def _check(s, b, k, label):
    m, n = s.shape
    print(f"qb case {label}: m={m} n={n} k={k} bias={'yes' if b is not None else 'no'}", flush=True)
    alpha, hist, nb = _gpu_qb(s, b, k)
    ref_alpha = qb.thresholds(s, b, k)
    assert np.array_equal(alpha.view(np.uint32), ref_alpha.view(np.uint32)), label
    ref_hist = qb.histogram(s, b, k)
    assert np.array_equal(hist, ref_hist), (label, np.argwhere(hist != ref_hist)[:5])
    q = qb.target_count(m, n, k)
    ref_bias = qb.bias_from_histogram(ref_hist, q)
    assert np.array_equal(nb.view(np.uint32), ref_bias.view(np.uint32)), label
    ex = qb.exact_bias(s, b, k).astype(np.float64)
    d = nb.astype(np.float64) - ex
    inside = (ex > -2.0 + 1e-6) & (ex < 2.0 - 0.004)        # quantile not clamped into an end bin
    assert np.all(d[inside] >= -1e-6) and np.all(d[inside] <= 0.004 + 1e-6), label
    return alpha, hist, nb


@pytest.mark.parametrize("m,n,k,bias,dyadic", [
    (1000, 896, 16, True, False),     # the K3 router shape
    (1000, 896, 16, False, False),
    (517, 24, 4, False, True),        # many exact ties
    (301, 130, 3, True, True),        # n not a multiple of 4: scalar loads
    (333, 2048, 8, True, False),      # more than 1024 experts: 64 keys per lane
    (64, 4096, 63, True, False),      # the expert limit
    (9, 2, 1, False, False),          # smallest shape
    (257, 17, 16, True, False),       # k + 1 = n: alpha is each token's smallest key
])
def test_qb_matches_oracle(m, n, k, bias, dyadic):
    s = gen.make_router_scores(m, n, seed=3, dyadic=dyadic)
    b = gen.make_selection_bias(n, seed=4) if bias else None
    _check(s, b, k, f"{m}x{n}")


def test_qb_margins_clamped_into_end_bins():
    """Large biases push margins past [-2, 2): they are counted in bin 0 (a bias of
    standard deviation 1.5 lifts the thresholds) or bin 999 (the same shifted by -4 sinks
    them below -1.7, so margins exceed 2), bit-exact with the oracle."""
    m, n, k = 400, 96, 6
    s = gen.make_router_scores(m, n, seed=5)
    b = gen.make_selection_bias(n, seed=6, std=1.5)
    _, hist, _ = _check(s, b, k, "clamped low")
    assert hist[:, 0].sum() > 0
    _, hist, _ = _check(s, (b - np.float32(4.0)).astype(np.float32), k, "clamped high")
    assert hist[:, -1].sum() > 0


def test_qb_no_tokens_gives_zero_histograms():
    L = _api()
    n = 40
    dev = torch.device("cuda")
    s = torch.zeros((0, n), dtype=torch.float32, device=dev)
    alpha = torch.zeros((0,), dtype=torch.float32, device=dev)
    hist = torch.full((n, qb.QB_BINS), 5, dtype=torch.int32, device=dev)
    L.moe_qb_histogram(s, None, 4, alpha, hist)
    torch.cuda.synchronize()
    assert int(hist.abs().sum()) == 0


def test_qb_summed_histograms_equal_the_union():
    """Thresholds are per token, so the histograms of two batches add up (the integer
    all-reduce) to those of their union, and the bias from the sum equals the oracle's
    update over the union."""
    n, k = 896, 16
    s = gen.make_router_scores(1500, n, seed=7)
    b = gen.make_selection_bias(n, seed=8)
    _, h1, _ = _gpu_qb(s[:600], b, k)
    _, h2, _ = _gpu_qb(s[600:], b, k)
    ref_union = qb.histogram(s, b, k)
    assert np.array_equal(h1 + h2, ref_union)
    L = _api()
    hd = torch.from_numpy((h1 + h2).astype(np.int32)).cuda()
    nb = torch.empty(n, dtype=torch.float32, device="cuda")
    L.moe_qb_bias(hd, 1500, k, nb)
    ref = qb.bias_from_histogram(ref_union, qb.target_count(1500, n, k))
    assert np.array_equal(nb.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("m,n,k,bias", [(1000, 896, 16, True), (301, 130, 3, True), (9, 2, 1, False),
                                        (333, 2048, 8, False)])
def test_qb_update_fused_equals_two_calls(m, n, k, bias):
    """moe_qb_update (bias from the LDS histograms in the histogram launch) gives the same
    alpha, histograms and bias, bit for bit, as moe_qb_histogram followed by moe_qb_bias,
    and as the oracle."""
    L = _api()
    s = gen.make_router_scores(m, n, seed=12)
    b = gen.make_selection_bias(n, seed=13) if bias else None
    alpha2, hist2, nb2 = _gpu_qb(s, b, k)
    dev = torch.device("cuda")
    alpha = torch.full((m,), float("nan"), dtype=torch.float32, device=dev)
    hist = torch.full((n, qb.QB_BINS), -7, dtype=torch.int32, device=dev)
    nb = torch.full((n,), 123.0, dtype=torch.float32, device=dev)
    L.moe_qb_update(torch.from_numpy(s).to(dev), None if b is None else torch.from_numpy(b).to(dev), k, alpha, hist,
                    nb)
    torch.cuda.synchronize()
    assert np.array_equal(alpha.cpu().numpy().view(np.uint32), alpha2.view(np.uint32))
    assert np.array_equal(hist.cpu().numpy().astype(np.int64), hist2)
    assert np.array_equal(nb.cpu().numpy().view(np.uint32), nb2.view(np.uint32))
    ref = qb.bias_from_histogram(qb.histogram(s, b, k), qb.target_count(m, n, k))
    assert np.array_equal(nb.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_qb_unreachable_target_is_nan():
    """Histograms that hold fewer than q margins per expert (m_total overstated) give NaN;
    the oracle refuses the same input."""
    m, n, k = 50, 32, 4
    s = gen.make_router_scores(m, n, seed=9)
    _, hist, nb = _gpu_qb(s, None, k, m_total=m * 100)   # q = 625 > 50 margins per expert
    assert np.all(np.isnan(nb))
    with pytest.raises(ValueError):
        qb.bias_from_histogram(hist, qb.target_count(m * 100, n, k))


@pytest.mark.fullsize
def test_qb_full_prefill_batch():
    """Router scores of an 8192-token batch at the K3 shape (896 experts, top-16), with a
    selection bias: everything bit-exact."""
    m, n, k = 8192, 896, 16
    s = gen.make_router_scores(m, n, seed=0)
    b = gen.make_selection_bias(n, seed=0)
    _, hist, nb = _check(s, b, k, "prefill8192")
    assert np.all(hist.sum(axis=1) == m)
