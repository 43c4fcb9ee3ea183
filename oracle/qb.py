"""Quantile Balancing: the per-expert selection bias that matches a target load.
TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

K3 report review, section on Quantile Balancing: with m tokens, n experts and k
experts per token, every expert's target load is q = m*k/n. Top-(k+1) over the
biased router scores gives each token a threshold alpha_i (its (k+1)-th largest
biased score) that an expert must beat. For expert j the new bias is the
router-score quantile at which exactly q of its margins cross that threshold;
the bias only takes part in selection and is applied from the next step on.
At scale the quantile is estimated from 1000-bin integer histograms, one
integer all-reduce per layer and step, with an error bounded by the bin width.

The page's margin equation did not survive extraction. Readings taken here:

  Q1  inputs are the router scores s [m, n] (fp32, sigmoid of the logits, as
      the router computes them) and the current bias b [n] (fp32); the biased
      key is s + b, added in fp32 (the selection key of the router).
  Q2  alpha_i = the (k+1)-th largest biased key of token i (by value; ties
      count with multiplicity).
  Q3  margin mu_ij = s_ij - alpha_i in fp32: token i would pick expert j
      against its fixed threshold when s_ij + b'_j >= alpha_i, i.e. when
      mu_ij + b'_j >= 0.
  Q4  the integer target q* = max(1, floor(m*k / n)).
  Q5  exact update: b'_j = -(the q*-th largest mu_.j), so that q* margins
      (more only on ties) satisfy mu_ij + b'_j >= 0.
  Q6  histogram update: 1000 bins uniform on [-2, 2) (a margin of sigmoid
      scores lies in (-2, 2) while |b| < 1); bin(mu) = floor((mu + 2) * 250)
      in fp32, clamped to [0, 999]; t* = the largest bin whose suffix count
      (bins t*..999) reaches q*; b'_j = -(-2 + t* * 0.004) in fp32 (the lower
      edge of the bin holding the q*-th largest margin), so b'_j lies within
      one bin width above the exact update (or beyond it only for margins
      clamped into the end bins).

Every step that turns a float into an integer (bin) or back (edge) is written
as the fp32 operations listed, so that an fp32 evaluation elsewhere takes the
same decisions.
"""
from __future__ import annotations

import numpy as np

QB_BINS = 1000
QB_LO = np.float32(-2.0)
QB_SCALE = np.float32(250.0)   # bins per unit margin
QB_WIDTH = np.float32(0.004)   # 1 / QB_SCALE as the fp32 constant used for bin edges


def target_count(m: int, n: int, k: int) -> int:
    """Q4: the integer per-expert target load."""
    return max(1, (m * k) // n)


def thresholds(scores: np.ndarray, bias, k: int) -> np.ndarray:
    """Q1, Q2: alpha_i, the (k+1)-th largest biased key of each token (fp32)."""
    s = np.asarray(scores, dtype=np.float32)
    keys = s + (np.zeros(s.shape[1], np.float32) if bias is None else np.asarray(bias, np.float32))
    if k + 1 > keys.shape[1]:
        raise ValueError("k + 1 must not exceed the number of experts")
    # the (k+1)-th largest = element n-(k+1) of the ascending order
    return np.sort(keys, axis=1)[:, keys.shape[1] - (k + 1)].astype(np.float32)


def margins(scores: np.ndarray, alpha: np.ndarray) -> np.ndarray:
    """Q3: mu_ij = s_ij - alpha_i in fp32."""
    return (np.asarray(scores, np.float32) - np.asarray(alpha, np.float32)[:, None]).astype(np.float32)


def exact_bias(scores: np.ndarray, bias, k: int) -> np.ndarray:
    """Q5: b'_j = -(q*-th largest margin of expert j)."""
    s = np.asarray(scores, np.float32)
    m, n = s.shape
    q = target_count(m, n, k)
    mu = margins(s, thresholds(s, bias, k))
    qth = np.sort(mu, axis=0)[m - q, :]          # q-th largest per column
    return (-qth).astype(np.float32)


def bin_index(mu: np.ndarray) -> np.ndarray:
    """Q6: floor((mu + 2) * 250) in fp32, clamped to [0, 999]."""
    t = (np.asarray(mu, np.float32) - QB_LO).astype(np.float32)        # mu + 2, one fp32 rounding
    t = (t * QB_SCALE).astype(np.float32)                                # times 250, one fp32 rounding
    return np.clip(np.floor(t), 0, QB_BINS - 1).astype(np.int64)


def histogram(scores: np.ndarray, bias, k: int) -> np.ndarray:
    """Per-expert margin histograms, int64 [n, 1000]."""
    s = np.asarray(scores, np.float32)
    m, n = s.shape
    idx = bin_index(margins(s, thresholds(s, bias, k)))               # [m, n]
    hist = np.zeros((n, QB_BINS), np.int64)
    for j in range(n):
        hist[j] = np.bincount(idx[:, j], minlength=QB_BINS)
    return hist


def bias_from_histogram(hist: np.ndarray, q: int) -> np.ndarray:
    """Q6: t* = largest bin whose suffix count reaches q; b' = -(-2 + t* * 0.004) in fp32."""
    h = np.asarray(hist, np.int64)
    suffix = np.cumsum(h[:, ::-1], axis=1)[:, ::-1]                      # suffix[j, t] = sum of bins t..999
    ok = suffix >= q
    if not ok[:, 0].all():
        raise ValueError("an expert has fewer than q margins")
    tstar = QB_BINS - 1 - np.argmax(ok[:, ::-1], axis=1)                 # largest t with ok
    edge = (QB_LO + (tstar.astype(np.float32) * QB_WIDTH).astype(np.float32)).astype(np.float32)
    return (-edge).astype(np.float32)


def qb_bias(scores: np.ndarray, bias, k: int):
    """The histogram estimate of the new bias and its histograms (one rank's batch)."""
    s = np.asarray(scores, np.float32)
    m, n = s.shape
    hist = histogram(s, bias, k)
    return bias_from_histogram(hist, target_count(m, n, k)), hist
