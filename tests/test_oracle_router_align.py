"""Pins for the oracle's router (T6, T12) and moe_align_block_size (T11), CPU only."""
import json
import math
import os

import numpy as np
import pytest

from oracle import brute
from oracle.layer import align, align_capacity, route, sigmoid

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _onehot_router(logit_values, H=8, h0=3):
    """Router weights whose logits equal logit_values for x with x[h0] = 1, x[else] = 0."""
    E = len(logit_values)
    W = np.zeros((E, H))
    W[:, h0] = logit_values
    x = np.zeros((1, H))
    x[0, h0] = 1.0
    return x, W


def test_router_closed_form_selection_and_weights():
    a = np.array([0.3, -1.0, 2.0, 0.9, 2.0, -0.2, 1.5, 0.0])
    x, W = _onehot_router(a)
    r = route(x, W, None, k=3, rsf=2.446)
    # largest logits: 2.0 (id 2), 2.0 (id 4), 1.5 (id 6)
    assert r["ids"].tolist() == [[2, 4, 6]]
    s = 1.0 / (1.0 + np.exp(-a[[2, 4, 6]]))
    np.testing.assert_allclose(r["weights"][0], s / s.sum() * 2.446, rtol=1e-15)
    assert math.isclose(r["weights"].sum(), 2.446, rel_tol=1e-14)
    np.testing.assert_allclose(sigmoid(np.array([0.0])), [0.5])


def test_router_tie_goes_to_lower_id_and_flags_near_tie():
    a = np.array([1.0, 2.0, 1.0, 3.0, 1.0])
    x, W = _onehot_router(a)
    r = route(x, W, None, k=3)
    assert r["ids"].tolist() == [[0, 1, 3]]          # three-way tie at 1.0 -> id 0 wins
    assert r["near_tie"][0]
    a2 = np.array([1.0, 2.0, 0.0, 3.0, -1.0])
    x, W = _onehot_router(a2)
    assert not route(x, W, None, k=3)["near_tie"][0]


def test_router_bias_selects_only():
    """The selection bias changes which experts win but not the weight formula."""
    a = np.array([0.0, 0.1, 0.2, 0.3])
    x, W = _onehot_router(a)
    bias = np.array([1.0, 0.0, 0.0, 0.0])
    r = route(x, W, bias, k=2)
    assert r["ids"].tolist() == [[0, 3]]
    s = 1.0 / (1.0 + np.exp(-a[[0, 3]]))
    np.testing.assert_allclose(r["weights"][0], s / s.sum(), rtol=1e-15)


def test_t6_router_statistics():
    rng = np.random.default_rng(5)
    T, H, E, k = 300, 64, 56, 1          # k/E = 1/56 as in the pages (16 of 896)
    x = rng.standard_normal((T, H))
    W = rng.standard_normal((E, H)) / np.sqrt(H)
    for kk in (k, 4):
        r = route(x, W, None, kk)
        ids = r["ids"]
        assert ids.shape == (T, kk)
        assert all(len(set(row)) == kk for row in ids.tolist())      # exactly k distinct
        assert np.all(np.diff(ids, axis=1) > 0)                      # ascending id order
        assert ids.min() >= 0 and ids.max() < E
        np.testing.assert_allclose(r["weights"].sum(axis=1), 1.0, atol=1e-12)
    # the pages' selection rate: 16 of 896 = 1/56 = 1.79%
    r = route(x, W, None, 1)
    assert r["ids"].size / (T * E) == 16 / 896 == 1 / 56
    assert round(100 * 16 / 896, 2) == 1.79


def test_t12_expert_ids_above_255_are_selected():
    rng = np.random.default_rng(1)
    E, H, T, k = 900, 32, 6, 4
    x = rng.standard_normal((T, H))
    W = rng.standard_normal((E, H)) * 0.01
    bias = np.zeros(E)
    bias[[255, 256, 895, 899]] = 5.0
    r = route(x, W, bias, k)
    assert np.all(r["ids"] == np.array([255, 256, 895, 899]))
    al = align(r["ids"], E, 4)
    assert al["counts"][256] == T and al["counts"][899] == T
    assert set(al["expert_ids"][al["expert_ids"] >= 0].tolist()) == {255, 256, 895, 899}


def test_t11_align_worked_example():
    with open(os.path.join(GOLD, "align_worked_example.json")) as f:
        g = json.load(f)
    al = align(np.array(g["ids"]), g["E"], g["B"])
    assert al["cap"] == g["capacity"] == align_capacity(g["T"], g["k"], g["E"], g["B"])
    assert al["counts"].tolist() == g["counts"]
    assert al["sorted_ids"].tolist() == g["sorted_ids"]
    assert al["expert_ids"].tolist() == g["expert_ids"]
    assert al["num_post"] == g["num_post"]
    assert al["inv_pos"].tolist() == g["inv_pos"]


@pytest.mark.parametrize("T,k,E,B,seed", [(5, 2, 8, 4, 0), (37, 6, 40, 16, 1), (16, 16, 896, 16, 2),
                                          (64, 8, 300, 8, 3), (1, 1, 1, 1, 4), (9, 3, 3, 64, 5)])
def test_t11_align_invariants_and_brute_force(T, k, E, B, seed):
    rng = np.random.default_rng(seed)
    ids = np.stack([np.sort(rng.choice(E, size=k, replace=False)) for _ in range(T)]).astype(np.int32)
    al = align(ids, E, B)
    pairs = T * k
    s, ex, n = al["sorted_ids"], al["expert_ids"], al["num_post"]
    valid = s[:n][s[:n] < pairs]
    assert sorted(valid.tolist()) == list(range(pairs))               # every slot exactly once
    assert np.all(s[n:] == pairs) and np.all(ex[n // B:] == -1)
    assert n % B == 0 and n <= al["cap"]
    for e in range(E):
        blocks = np.nonzero(ex == e)[0]
        c = int(al["counts"][e])
        assert len(blocks) == -(-c // B)
        if c:
            seg = s[blocks[0] * B:(blocks[-1] + 1) * B]
            assert np.all(np.diff(seg[:c]) > 0) and np.all(seg[c:] == pairs)
            assert np.all(ids.reshape(-1)[seg[:c]] == e)
    assert np.all(s[al["inv_pos"]] == np.arange(pairs))
    bs, be = brute.align(ids.tolist(), E, B)
    assert s[:n].tolist() == bs and ex[:n // B].tolist() == be


def test_t11_lcm_alignment_serves_two_tile_widths():
    """A layout aligned to lcm(8, 4) = 8 read by a width-4 consumer with expert ids
    expanded to its own tile count gives every width-4 tile a single expert."""
    rng = np.random.default_rng(7)
    T, k, E = 20, 3, 10
    ids = np.stack([np.sort(rng.choice(E, size=k, replace=False)) for _ in range(T)])
    al8 = align(ids, E, 8)
    ex4 = np.repeat(al8["expert_ids"], 2)                 # expanded to width-4 tiles
    flat = ids.reshape(-1)
    s = al8["sorted_ids"]
    for tile in range(al8["num_post"] // 4):
        seg = s[tile * 4:(tile + 1) * 4]
        real = seg[seg < T * k]
        assert np.all(flat[real] == ex4[tile])
    # the misaligned reading (width-8 ids applied to width-4 tiles) gets experts wrong
    wrong = 0
    for tile in range(al8["num_post"] // 4):
        seg = s[tile * 4:(tile + 1) * 4]
        real = seg[seg < T * k]
        wrong += int(np.any(flat[real] != al8["expert_ids"][min(tile, len(al8["expert_ids"]) - 1)]))
    assert wrong > 0
