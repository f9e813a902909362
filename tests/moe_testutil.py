"""Shared helpers of the tests: comparison rules and GPU-side set-up.

Comparison rules follow the tolerances of the layer's parity contract:
routing indices and loads bit-exact except at near-ties (oracle score gap
< 1e-6), gates within 1e-5, outputs by relative L2 error.
"""
import numpy as np
import torch

NEAR_TIE = 1e-6
GATE_ATOL = 1e-5


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def routing_mismatches(idx_gpu, routing, near=NEAR_TIE):
    """Tokens whose GPU selection differs from the oracle's.

    Returns (bad, tied): `bad` are differences the oracle's own score gaps do
    not allow (must be empty); `tied` are allowed near-tie differences."""
    idx_o = routing.idx
    bad, tied = [], []
    for t in np.nonzero(np.any(idx_gpu != idx_o, axis=1))[0]:
        same_set = set(idx_gpu[t].tolist()) == set(idx_o[t].tolist())
        if not same_set and routing.boundary_gap[t] >= near:
            bad.append(int(t))
            continue
        # order differences are allowed only across near-equal adjacent keys
        ok = True
        if same_set:
            for k in range(idx_o.shape[1]):
                if idx_gpu[t, k] != idx_o[t, k]:
                    gaps = routing.inner_gap[t]
                    lo, hi = max(k - 1, 0), min(k, gaps.shape[0] - 1)
                    if not np.any(gaps[lo:hi + 1] < near):
                        ok = False
        (tied if ok else bad).append(int(t))
    return bad, tied


def check_routing(idx_gpu, gate_gpu, load_gpu, routing, Nr):
    """Assert the GPU routing matches the oracle under the near-tie rule."""
    bad, tied = routing_mismatches(idx_gpu, routing)
    assert not bad, f"routing differs beyond near-ties at tokens {bad[:10]}"
    ok = np.ones(idx_gpu.shape[0], dtype=bool)
    ok[tied] = False
    assert np.array_equal(idx_gpu[ok], routing.idx[ok])
    np.testing.assert_allclose(gate_gpu[ok], routing.gate[ok], rtol=0, atol=GATE_ATOL)
    want_load = np.bincount(idx_gpu.ravel(), minlength=Nr)
    assert np.array_equal(load_gpu, want_load)          # loads consistent with the GPU's own selection
    if not tied:
        assert np.array_equal(load_gpu, routing.load)
    else:   # each tied token moves at most one assignment
        assert np.abs(load_gpu - routing.load).sum() <= 2 * len(tied)
    return ok, tied


def np_of(t: torch.Tensor):
    return t.detach().to("cpu").numpy()


def f64_of(t: torch.Tensor):
    return t.detach().to("cpu", torch.float64).numpy()
