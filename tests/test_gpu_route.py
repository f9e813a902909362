"""GPU parity of moe_route against the oracle's routing: indices and loads
bit-exact except at near-ties (oracle score gap < 1e-6), gates within 1e-5."""
import numpy as np
import pytest
import torch

import sparse_expert_routing_sigmoid_amd as M
import workloads as W
from moe_testutil import check_routing, np_of, f64_of
from oracle import moe as O

pytestmark = pytest.mark.gpu


def _gpu_route(u, e, b, K):
    T, d = u.shape
    Nr = e.shape[0]
    idx = torch.full((T, K), -7, dtype=torch.int32, device="cuda")
    gate = torch.empty((T, K), dtype=torch.float32, device="cuda")
    score = torch.empty((T, K), dtype=torch.float32, device="cuda")
    load = torch.full((Nr,), 12345, dtype=torch.int32, device="cuda")
    ws = torch.empty((M.moe_route_workspace_bytes(T, d, Nr),), dtype=torch.uint8, device="cuda")
    M.moe_route(u, e, b, K, idx, gate, score, load, ws)
    torch.cuda.synchronize()
    return np_of(idx), np_of(gate), np_of(score), np_of(load)


def _run(cfg, step=0, K=None):
    K = cfg.K if K is None else K
    u = W.make_tokens(cfg, step, "cuda")
    e = W.make_centroids(cfg, "cuda")
    b = W.make_bias(cfg, "cuda")
    idx, gate, score, load = _gpu_route(u, e, b, K)
    r = O.route(f64_of(u), f64_of(e), f64_of(b), K)
    ok, tied = check_routing(idx, gate, load, r, cfg.Nr)
    np.testing.assert_allclose(score[ok], r.score[ok], rtol=0, atol=2e-6)
    return r, tied


@pytest.mark.parametrize("name", ["tiny_fp32", "mid_bf16", "v3_decode_fp8w"])
def test_route_configs(name):
    _run(W.CONFIGS[name])


def test_route_v3_prefill_zipf_two_steps():
    cfg = W.CONFIGS["v3_prefill_bf16"]
    for step in range(2):
        r, tied = _run(cfg, step)
        assert len(tied) <= 8


@pytest.mark.parametrize("T,Nr,K", [(1, 16, 4), (3, 16, 1), (17, 16, 16), (70, 1000, 8), (130, 64, 6),
                                    (65, 65, 16), (5, 1, 1)])
def test_route_shapes(T, Nr, K):
    cfg = W.CONFIGS["mid_bf16"].with_(T=T, Nr=Nr, d=512)
    _run(cfg, K=K)


def test_route_exact_ties_go_to_lower_index():
    cfg = W.CONFIGS["tiny_fp32"]
    u = W.make_tokens(cfg, 0, "cuda")
    e = W.make_centroids(cfg, "cuda")
    e[:] = e[0]                                   # identical centroids: s ties everywhere
    b = torch.zeros(cfg.Nr, device="cuda")
    b[9] = 0.5                                    # expert 9 always first, then 0, 1, 2
    idx, gate, _, load = _gpu_route(u, e, b, 4)
    assert np.all(idx == np.array([9, 0, 1, 2]))
    np.testing.assert_allclose(gate, 0.25, atol=1e-7)
    assert load.tolist() == [64, 64, 64] + [0] * 6 + [64] + [0] * 6


def test_route_zero_tokens_zeroes_load():
    e = torch.randn(16, 64, device="cuda")
    b = torch.zeros(16, device="cuda")
    u = torch.empty((0, 64), device="cuda")
    idx, gate, score, load = _gpu_route(u, e, b, 4)
    assert load.tolist() == [0] * 16


def test_route_is_deterministic():
    cfg = W.CONFIGS["mid_bf16"]
    u = W.make_tokens(cfg, 0, "cuda")
    e = W.make_centroids(cfg, "cuda")
    b = W.make_bias(cfg, "cuda")
    a = _gpu_route(u, e, b, cfg.K)
    c = _gpu_route(u, e, b, cfg.K)
    for x, y in zip(a, c):
        assert np.array_equal(x.view(np.uint32) if x.dtype == np.float32 else x,
                              y.view(np.uint32) if y.dtype == np.float32 else y)
