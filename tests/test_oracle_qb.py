"""Pins of oracle/qb.py (Quantile Balancing; readings Q1-Q6 in its docstring)."""
import json
import os

import numpy as np
import pytest

from oracle import qb

GOLD = os.path.join(os.path.dirname(__file__), "golden", "qb_worked_example.json")


def _rand_scores(m, n, seed, dyadic=False):
    rng = np.random.default_rng(seed)
    if dyadic:  # multiples of 2^-12 in (0, 1): every fp32 sum and difference below is exact
        return (rng.integers(1, 4096, size=(m, n)) / 4096.0).astype(np.float32)
    return (1.0 / (1.0 + np.exp(-rng.normal(size=(m, n))))).astype(np.float32)


def test_worked_example():
    g = json.load(open(GOLD))
    s = np.array(g["scores"], np.float32)
    b = np.array(g["bias"], np.float32)
    assert qb.target_count(g["m"], g["n"], g["k"]) == 2
    assert np.array_equal(qb.thresholds(s, b, g["k"]), np.array(g["alpha"], np.float32))
    assert np.array_equal(qb.exact_bias(s, b, g["k"]), np.array(g["exact_bias"], np.float32))


def test_target_count():
    assert qb.target_count(8192, 896, 16) == 146          # 131072 / 896 = 146.29
    assert qb.target_count(4, 2, 1) == 2
    assert qb.target_count(3, 896, 16) == 1               # floor 0 -> at least one


def test_thresholds_match_repeated_max_removal():
    s = _rand_scores(40, 12, 1)
    b = np.random.default_rng(2).normal(0, 0.05, 12).astype(np.float32)
    k = 3
    alpha = qb.thresholds(s, b, k)
    for i in range(s.shape[0]):
        keys = [float(np.float32(s[i, j]) + np.float32(b[j])) for j in range(12)]
        for _ in range(k):                                  # drop the k largest
            keys.remove(max(keys))
        assert alpha[i] == np.float32(max(keys))


def test_exact_bias_is_the_q_th_largest_margin():
    """At least q* margins cross with the new bias and fewer than q* cross strictly: the
    defining property of the q*-th order statistic (ties arise by construction: the expert
    that is a token's own (k+1)-th key has margin exactly -b_j there)."""
    m, n, k = 300, 24, 4
    s = _rand_scores(m, n, 3)
    b = np.random.default_rng(4).normal(0, 0.02, n).astype(np.float32)
    q = qb.target_count(m, n, k)
    mu = qb.margins(s, qb.thresholds(s, b, k)).astype(np.float64)
    new = qb.exact_bias(s, b, k).astype(np.float64)
    for j in range(n):
        assert int(np.sum(mu[:, j] + new[j] >= 0.0)) >= q
        assert int(np.sum(mu[:, j] + new[j] > 0.0)) < q


def test_threshold_ties_at_minus_bias():
    """A token's (k+1)-th expert has margin exactly -b_j."""
    s = _rand_scores(50, 10, 9)
    b = np.random.default_rng(10).normal(0, 0.02, 10).astype(np.float32)
    k = 2
    alpha = qb.thresholds(s, b, k)
    keys = s + b
    for i in range(50):
        j = int(np.argsort(-keys[i], kind="stable")[k])
        assert np.float32(s[i, j] - alpha[i]) == np.float32(-b[j]) or abs(float(s[i, j] - alpha[i] + b[j])) < 1e-7


def test_bias_shift_equivariance():
    """A common shift c of all biases shifts every threshold by c and the new biases by c."""
    s = _rand_scores(64, 16, 5, dyadic=True)
    b = (np.random.default_rng(6).integers(-64, 64, 16) / 1024.0).astype(np.float32)
    c = np.float32(0.25)
    a0, a1 = qb.exact_bias(s, b, 2), qb.exact_bias(s, b + c, 2)
    assert np.array_equal(a1, (a0 + c).astype(np.float32))


def test_bin_index_edges():
    mu = np.array([-3.0, -2.0, -1.5, 0.0, 0.5, 1.996, 1.9999, 2.0, 5.0], np.float32)
    assert qb.bin_index(mu).tolist() == [0, 0, 125, 500, 625, 999, 999, 999, 999]
    # a bin's lower edge lands in that bin
    for t in (1, 17, 250, 499, 998):
        edge = np.float32(np.float32(-2.0) + np.float32(np.float32(t) * np.float32(0.004)))
        assert qb.bin_index(np.array([edge], np.float32))[0] in (t - 1, t)


def test_bias_from_histogram_search():
    h = np.zeros((3, qb.QB_BINS), np.int64)
    h[0, 990:1000] = 1          # suffix reaches 5 at bin 995
    h[1, 700] = 10              # all mass in one bin
    h[2, 0] = 5                 # everything clamped low
    out = qb.bias_from_histogram(h, 5)
    assert out[0] == -np.float32(np.float32(-2.0) + np.float32(np.float32(995) * np.float32(0.004)))
    assert abs(float(out[1]) - (-0.8)) < 1e-6
    assert out[2] == np.float32(2.0)
    with pytest.raises(ValueError):
        qb.bias_from_histogram(h, 11)


def test_histogram_estimate_within_one_bin_of_exact():
    m, n, k = 2048, 64, 8
    s = _rand_scores(m, n, 7)
    b = np.random.default_rng(8).normal(0, 0.05, n).astype(np.float32)
    ex = qb.exact_bias(s, b, k)
    est, hist = qb.qb_bias(s, b, k)
    assert np.all(hist.sum(axis=1) == m)
    d = est.astype(np.float64) - ex.astype(np.float64)
    assert np.all(d >= -1e-6) and np.all(d <= 0.004 + 1e-6), (d.min(), d.max())


def test_dropping_the_plus_one_is_detected():
    """Using the k-th instead of the (k+1)-th key as the threshold changes the worked example."""
    g = json.load(open(GOLD))
    s = np.array(g["scores"], np.float32)
    kth = np.sort(s, axis=1)[:, s.shape[1] - g["k"]]
    assert not np.array_equal(kth, np.array(g["alpha"], np.float32))
