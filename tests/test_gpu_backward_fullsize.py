"""Backward parity at the full bf16 V3 size (T = 8192, d = 7168, 256 routed
+ 1 shared experts, I = 2048, top-8, Zipf loads), in the launch
configuration `bench.py --train` times (MoeLayer, tile_m = 32).

The oracle cannot run the whole backward at this size, so it checks what it
can compute exactly:
- the input gradient du of sampled tokens: a token's du depends only on its
  own experts, so the oracle runs its backward on a layer made of the
  token's K selected experts (K of K selected, the same gates) and the
  shared expert, which gives the full-layer du, gate and score gradients of
  that token;
- the weight gradients of the least loaded, a median and the most loaded
  routed expert, and of every shared expert (every token, the longest
  fp32 sums): dW13_i and dW2_i depend only on the rows of expert i, so the
  oracle's FFN backward on those rows (dy = g * dL/dh', or dL/dh' for a
  shared expert) gives them exactly.
Tokens at a routing near-tie are not sampled, nor experts that hold one.
"""
import numpy as np
import pytest
import torch

import sparse_expert_routing_sigmoid_amd as M
import workloads as W
from moe_testutil import check_routing, f64_of, np_of, rel_l2
from oracle import backward as OB
from oracle import moe as O

pytestmark = pytest.mark.gpu

TOL = 1e-2


@pytest.fixture(scope="module")
def run():
    cfg = W.CONFIGS["v3_prefill_bf16"]
    print(f"[backward fullsize] T={cfg.T} d={cfg.d} E={cfg.E} I={cfg.I} K={cfg.K}", flush=True)
    u = W.make_tokens(cfg, 0, "cuda")
    e = W.make_centroids(cfg, "cuda")
    b = W.make_bias(cfg, "cuda")
    w13, w2 = W.make_expert_weights(cfg, "cuda")
    G = W.make_free((cfg.T, cfg.d), 1.0, 100, "cuda", torch.bfloat16)
    layer = M.MoeLayer(cfg.T, cfg.d, cfg.Nr, cfg.Ns, cfg.I, cfg.K, torch.bfloat16,
                       M.ExpertWeights(M.MOE_BF16, w13, w2), tile_m=32, train=True, grad_dtype=torch.bfloat16)
    layer.forward(u, e, b)
    layer.backward(G, u, e)
    torch.cuda.synchronize()
    print("[backward fullsize] GPU done", flush=True)
    u64, e64, b64, G64 = f64_of(u), f64_of(e), f64_of(b), f64_of(G)
    r = O.route(u64, e64, b64, cfg.K)
    ok, tied = check_routing(np_of(layer.topk_idx), np_of(layer.topk_gate), np_of(layer.expert_load), r, cfg.Nr)
    cache = {}

    def weights(i):
        if i not in cache:
            cache[i] = (f64_of(w13[i]), f64_of(w2[i]))
        return cache[i]

    return dict(cfg=cfg, layer=layer, u=u64, e=e64, b=b64, G=G64, r=r, ok=ok, tied=set(tied), weights=weights)


def test_token_input_gradients_at_full_size(run):
    cfg, layer, r = run["cfg"], run["layer"], run["r"]
    rng = np.random.default_rng(7)
    cand = np.nonzero(run["ok"])[0]
    toks = rng.choice(cand, size=4, replace=False)
    du_gpu = f64_of(layer.du)
    dgate_gpu, dz_gpu = f64_of(layer.dgate), f64_of(layer.dz)
    got, want, dg_got, dg_want = [], [], [], []
    for t in toks:
        sel = r.idx[t]
        experts = list(sel) + list(range(cfg.Nr, cfg.Nr + cfg.Ns))
        w13 = np.stack([run["weights"](i)[0] for i in experts])
        w2 = np.stack([run["weights"](i)[1] for i in experts])
        gr = OB.layer_backward(run["u"][t:t + 1], run["e"][sel], run["b"][sel], w13, w2, cfg.K, cfg.Ns, cfg.K,
                               run["G"][t:t + 1])
        # the mini layer orders its K experts by the same keys as the full one
        assert np.array_equal(np.asarray(sel)[O.route(run["u"][t:t + 1], run["e"][sel], run["b"][sel], cfg.K).idx[0]],
                              sel)
        got.append(du_gpu[t])
        want.append(gr.du[0])
        dg_got.append(np.concatenate([dgate_gpu[t], dz_gpu[t]]))
        dg_want.append(np.concatenate([gr.dgate[0], gr.dz[0]]))
        print(f"token {t}: du rel L2 {rel_l2(du_gpu[t], gr.du[0]):.2e}", flush=True)
    assert rel_l2(np.array(got), np.array(want)) <= TOL
    assert rel_l2(np.array(got) - run["G"][toks], np.array(want) - run["G"][toks]) <= TOL
    assert rel_l2(np.array(dg_got), np.array(dg_want)) <= TOL


def test_expert_weight_gradients_at_full_size(run):
    cfg, layer, r = run["cfg"], run["layer"], run["r"]
    load = r.load
    clean = [i for i in range(cfg.Nr) if load[i] > 0 and not any(t in run["tied"]
                                                                 for t in np.nonzero(np.any(r.idx == i, axis=1))[0])]
    by_load = sorted(clean, key=lambda i: load[i])
    picks = [by_load[0], by_load[len(by_load) // 2], by_load[-1]] + list(range(cfg.Nr, cfg.Nr + cfg.Ns))
    for i in picks:
        w13_i, w2_i = run["weights"](i)
        if i < cfg.Nr:
            ts, ks = np.nonzero(r.idx == i)
            dy = r.gate[ts, ks][:, None] * run["G"][ts]
        else:   # shared expert: every token, gate 1
            ts = np.arange(cfg.T)
            dy = run["G"]
        _, dw13, dw2, _ = OB.ffn_backward(run["u"][ts], w13_i, w2_i, dy)
        e13 = rel_l2(f64_of(layer.dw13[i]), dw13)
        e2 = rel_l2(f64_of(layer.dw2[i]), dw2)
        print(f"expert {i} ({len(ts)} rows): dW13 rel L2 {e13:.2e}, dW2 {e2:.2e}", flush=True)
        assert e13 <= TOL and e2 <= TOL
    idle = np.nonzero(np_of(layer.expert_load) == 0)[0]
    for i in idle[:4]:
        assert torch.count_nonzero(layer.dw13[i]).item() == 0 and torch.count_nonzero(layer.dw2[i]).item() == 0
