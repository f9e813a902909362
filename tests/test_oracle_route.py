"""Pins of the oracle's routing: affinity, bias-steered top-K, gates, loads.

Independent checks: a hand-worked example (tests/golden), a pure-Python
selection by repeated maximum, exhaustive enumeration of K-subsets, closed
forms for K = 1 and K = N_r, invariants of gates and loads, and invariance of
the selection under a common shift of the bias.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import moe


def _worked(golden_dir):
    with open(os.path.join(golden_dir, "route_worked_example.json")) as f:
        fx = json.load(f)
    conv = {"ln3": math.log(3.0), "-ln3": -math.log(3.0)}
    e = np.array([[conv.get(v, v) for v in row] for row in fx["centroids"]], dtype=np.float64)
    return fx, np.array(fx["tokens"], dtype=np.float64), e, np.array(fx["bias"], dtype=np.float32)


def test_worked_example(golden_dir):
    fx, u, e, b = _worked(golden_dir)
    ex = fx["expected"]
    r = moe.route(u, e, b, fx["K"])
    np.testing.assert_allclose(r.s, ex["s"], rtol=0, atol=1e-15)
    assert r.idx.tolist() == ex["idx"]
    np.testing.assert_allclose(r.gate, ex["gate"], rtol=0, atol=1e-15)
    assert r.load.tolist() == ex["load"]
    nb = moe.bias_update(b, r.load, u.shape[0], fx["K"])
    assert nb.dtype == np.float32
    np.testing.assert_allclose(nb, ex["bias_after_one_step"], rtol=0, atol=3e-8)


def _brute_select(v_row, K):
    """Pick the largest key K times; equal keys -> the lowest index."""
    chosen = []
    for _ in range(K):
        best = None
        for j in range(len(v_row)):
            if j in chosen:
                continue
            if best is None or v_row[j] > v_row[best]:
                best = j
        chosen.append(best)
    return chosen


def _coarse_inputs(rng, T, Nr, d=3):
    """Inputs whose keys collide often: small-integer u and e give repeated
    logits, and a bias on a coarse grid creates exact ties in s+b."""
    u = rng.integers(-2, 3, (T, d)).astype(np.float64)
    e = rng.integers(-1, 2, (Nr, d)).astype(np.float64) * 0.5
    b = (rng.integers(-2, 3, Nr) * 0.125).astype(np.float32)
    return u, e, b


@pytest.mark.parametrize("Nr,K", [(4, 1), (6, 2), (8, 3), (12, 5), (12, 12)])
def test_select_matches_repeated_maximum(Nr, K):
    rng = np.random.default_rng(Nr * 31 + K)
    for _ in range(3):
        u, e, b = _coarse_inputs(rng, 40, Nr)
        r = moe.route(u, e, b, K)
        for t in range(u.shape[0]):
            assert r.idx[t].tolist() == _brute_select(r.v[t].tolist(), K)


@pytest.mark.parametrize("Nr,K", [(5, 2), (8, 3), (10, 4)])
def test_selected_set_is_the_best_subset(Nr, K):
    """The Top-K set under the order (key desc, index asc) is the K-subset whose
    keys, listed best first, are lexicographically largest."""
    rng = np.random.default_rng(100 + Nr)
    u = rng.normal(size=(12, 4))
    e = rng.normal(size=(Nr, 4))
    b = rng.uniform(-0.3, 0.3, Nr).astype(np.float32)
    r = moe.route(u, e, b, K)
    for t in range(u.shape[0]):
        keyed = lambda S: sorted(((r.v[t, j], -j) for j in S), reverse=True)
        best = max(itertools.combinations(range(Nr), K), key=keyed)
        assert sorted(best) == sorted(r.idx[t].tolist())
        # the set property: every selected key beats every unselected one
        sel = set(r.idx[t].tolist())
        assert min(r.v[t, list(sel)]) >= max([r.v[t, j] for j in range(Nr) if j not in sel] or [-np.inf])


def test_gate_and_load_invariants():
    rng = np.random.default_rng(5)
    T, d, Nr, K = 300, 32, 20, 6
    u = rng.normal(size=(T, d))
    e = rng.normal(size=(Nr, d)) / math.sqrt(d)
    b = rng.uniform(-0.01, 0.01, Nr).astype(np.float32)
    r = moe.route(u, e, b, K)
    assert r.idx.shape == (T, K) and r.gate.shape == (T, K)
    for t in range(T):
        assert len(set(r.idx[t].tolist())) == K                # K distinct experts
    np.testing.assert_allclose(r.gate.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(r.gate > 0)
    # gates are proportional to s (not to s + b)
    ratio = r.gate / np.take_along_axis(r.s, r.idx, axis=1)
    np.testing.assert_allclose(ratio, ratio[:, :1].repeat(K, 1), rtol=1e-12)
    # selection keys appear in non-increasing order
    keys = np.take_along_axis(r.v, r.idx, axis=1)
    assert np.all(np.diff(keys, axis=1) <= 0)
    assert r.load.sum() == T * K and r.load.max() <= T
    assert np.array_equal(r.load, np.bincount(r.idx.ravel(), minlength=Nr))


def test_k_equals_nr_gates_ignore_bias():
    rng = np.random.default_rng(8)
    u = rng.normal(size=(50, 16))
    e = rng.normal(size=(7, 16)) / 4
    s = 1 / (1 + np.exp(-(u @ e.T)))
    for b in (np.zeros(7, np.float32), rng.uniform(-1, 1, 7).astype(np.float32)):
        r = moe.route(u, e, b, 7)
        g_full = np.zeros((50, 7))
        np.put_along_axis(g_full, r.idx, r.gate, axis=1)
        np.testing.assert_allclose(g_full, s / s.sum(axis=1, keepdims=True), rtol=1e-13)


def test_k1_picks_argmax_with_unit_gate():
    rng = np.random.default_rng(9)
    u = rng.normal(size=(64, 8))
    e = rng.normal(size=(9, 8))
    b = rng.uniform(-0.2, 0.2, 9).astype(np.float32)
    r = moe.route(u, e, b, 1)
    assert np.array_equal(r.idx[:, 0], np.argmax(r.v, axis=1))   # argmax returns the first maximum
    assert np.all(r.gate == 1.0)


def test_common_bias_shift_keeps_selection():
    rng = np.random.default_rng(12)
    u = rng.normal(size=(200, 24))
    e = rng.normal(size=(16, 24)) / 5
    b = rng.uniform(-0.05, 0.05, 16).astype(np.float32)
    r0 = moe.route(u, e, b, 4)
    r1 = moe.route(u, e, b + np.float32(0.25), 4)
    safe = (r0.boundary_gap > 1e-9) & np.all(r0.inner_gap > 1e-9, axis=1)
    assert safe.mean() > 0.9
    assert np.array_equal(r0.idx[safe], r1.idx[safe])
    np.testing.assert_allclose(r0.gate[safe], r1.gate[safe], rtol=1e-14)


def test_large_bias_forces_selection_but_not_gate():
    rng = np.random.default_rng(13)
    u = rng.normal(size=(30, 10))
    e = rng.normal(size=(8, 10)) / 3
    b = np.zeros(8, np.float32)
    b[5] = 10.0
    r = moe.route(u, e, b, 3)
    assert np.all(r.idx[:, 0] == 5)
    s5 = 1 / (1 + np.exp(-(u @ e[5])))
    np.testing.assert_allclose(r.score[:, 0], s5, rtol=1e-14)
    assert np.all(r.gate[:, 0] < 1.0)


def test_rejects_bad_k():
    with pytest.raises(ValueError):
        moe.route(np.zeros((2, 3)), np.zeros((4, 3)), np.zeros(4, np.float32), 5)
