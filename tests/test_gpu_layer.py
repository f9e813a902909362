"""GPU parity of the whole layer forward (route -> permute -> expert GEMMs ->
combine, then the bias rule) against the oracle's layer, on the tiny fp32
and the mid bf16 layers.  Outputs are compared on tokens whose routing
matches the oracle (a near-tie may legitimately flip one expert); the FFN
part of the output is checked on its own as well."""
import numpy as np
import pytest
import torch

import sparse_expert_routing_sigmoid_amd as M
import workloads as W
from moe_testutil import check_routing, f64_of, np_of, rel_l2
from oracle import moe as O

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 1e-2}


def build_layer(cfg, tile_m=32):
    w13, w2 = W.make_expert_weights(cfg, "cuda")
    wt = {"f32": M.MOE_F32, "bf16": M.MOE_BF16}[cfg.weights]
    layer = M.MoeLayer(cfg.T, cfg.d, cfg.Nr, cfg.Ns, cfg.I, cfg.K, W.TORCH_DTYPE[cfg.act],
                       M.ExpertWeights(wt, w13, w2), tile_m=tile_m)
    return layer, w13, w2


@pytest.mark.parametrize("name", ["tiny_fp32", "mid_bf16"])
def test_layer_forward(name):
    cfg = W.CONFIGS[name]
    layer, w13, w2 = build_layer(cfg)
    u = W.make_tokens(cfg, 0, "cuda")
    e = W.make_centroids(cfg, "cuda")
    b = W.make_bias(cfg, "cuda")
    out = layer.forward(u, e, b)
    ffn = torch.empty_like(out)
    layer.combine(u, flags=M.MOE_COMBINE_NO_RESIDUAL, out=ffn)
    bias = b.clone()
    layer.update_bias(bias, cfg.gamma)
    torch.cuda.synchronize()

    o = O.layer_forward(f64_of(u), f64_of(e), f64_of(b), f64_of(w13), f64_of(w2), cfg.Nr, cfg.Ns, cfg.K,
                        gamma=cfg.gamma)
    ok, tied = check_routing(np_of(layer.topk_idx), np_of(layer.topk_gate), np_of(layer.expert_load),
                             o.routing, cfg.Nr)
    tol = TOL[cfg.act]
    got = f64_of(out)
    assert np.all(np.isfinite(got))
    assert rel_l2(got[ok], o.out[ok]) <= tol
    assert rel_l2(f64_of(ffn)[ok], (o.out - f64_of(u))[ok]) <= tol
    if not tied:
        assert np.array_equal(np_of(bias).view(np.uint32), o.new_bias.view(np.uint32))


def test_tiny_bias_steps_teacher_forced():
    """Three steps of forward + bias rule; every GPU step starts from the
    oracle's bias, so the trajectories can be compared bit for bit."""
    cfg = W.CONFIGS["tiny_fp32"].with_(steps=3)
    layer, w13, w2 = build_layer(cfg)
    e = W.make_centroids(cfg, "cuda")
    b_o = np.zeros(cfg.Nr, np.float32)
    moved = 0
    for step in range(cfg.steps):
        u = W.make_tokens(cfg, step, "cuda")
        b = torch.from_numpy(b_o.copy()).cuda()
        layer.forward(u, e, b)
        layer.update_bias(b)
        torch.cuda.synchronize()
        o = O.layer_forward(f64_of(u), f64_of(e), b_o, f64_of(w13), f64_of(w2), cfg.Nr, cfg.Ns, cfg.K)
        _, tied = check_routing(np_of(layer.topk_idx), np_of(layer.topk_gate), np_of(layer.expert_load),
                                o.routing, cfg.Nr)
        if not tied:
            assert np.array_equal(np_of(b).view(np.uint32), o.new_bias.view(np.uint32))
        moved += int(np.sum(o.new_bias != b_o))
        b_o = o.new_bias
    assert moved > 0


def test_layer_deterministic():
    cfg = W.CONFIGS["mid_bf16"].with_(T=1024)
    layer, _, _ = build_layer(cfg)
    u = W.make_tokens(cfg, 0, "cuda")
    e = W.make_centroids(cfg, "cuda")
    b = W.make_bias(cfg, "cuda")
    o1 = layer.forward(u, e, b).clone()
    o2 = layer.forward(u, e, b).clone()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_fp8_layer_forward():
    """The E4M3 layer (activations in 1x128 tiles, weights in 128x128 blocks,
    h re-quantised) on a reduced V3 FP8 prefill shape with Zipf-skewed routing,
    against the oracle layer with the same quantisation points (R8)."""
    from test_gpu_gemm import oracle_fp8_weights
    cfg = W.CONFIGS["v3_prefill_fp8"].with_(T=768, d=512, Nr=16, Ns=1, I=256, K=4)
    w13, w2 = W.make_expert_weights(cfg, "cuda")
    layer = M.MoeLayer(cfg.T, cfg.d, cfg.Nr, cfg.Ns, cfg.I, cfg.K, W.TORCH_DTYPE[cfg.act],
                       M.quantize_weights(w13, w2), x_fp8=True, tile_m=32)
    u = W.make_tokens(cfg, 0, "cuda")
    e = W.make_centroids(cfg, "cuda")
    b = W.make_bias(cfg, "cuda")
    out = layer.forward(u, e, b)
    torch.cuda.synchronize()
    w13q, w2q = oracle_fp8_weights(w13, w2)
    o = O.layer_forward(f64_of(u), f64_of(e), f64_of(b), w13q, w2q, cfg.Nr, cfg.Ns, cfg.K,
                        x_quant=True, h_quant=True, gamma=cfg.gamma)
    ok, _ = check_routing(np_of(layer.topk_idx), np_of(layer.topk_gate), np_of(layer.expert_load),
                          o.routing, cfg.Nr)
    got = f64_of(out)
    assert np.all(np.isfinite(got))
    assert rel_l2(got[ok], o.out[ok]) <= 3e-2
    assert rel_l2(got[ok] - f64_of(u)[ok], (o.out - f64_of(u))[ok]) <= 3e-2


def test_w8a16_layer_forward():
    """The decode layer (bf16 activations, E4M3 weights in 128x128 blocks) on
    a reduced V3 decode shape with uniform routing, against the oracle layer
    on the same decoded weights."""
    from test_gpu_gemm import oracle_fp8_weights
    cfg = W.CONFIGS["v3_decode_fp8w"].with_(T=128, d=512, Nr=32, Ns=1, I=256, K=4)
    w13, w2 = W.make_expert_weights(cfg, "cuda")
    layer = M.MoeLayer(cfg.T, cfg.d, cfg.Nr, cfg.Ns, cfg.I, cfg.K, W.TORCH_DTYPE[cfg.act],
                       M.quantize_weights(w13, w2), tile_m=32)
    u = W.make_tokens(cfg, 0, "cuda")
    e = W.make_centroids(cfg, "cuda")
    b = W.make_bias(cfg, "cuda")
    out = layer.forward(u, e, b)
    torch.cuda.synchronize()
    w13q, w2q = oracle_fp8_weights(w13, w2)
    o = O.layer_forward(f64_of(u), f64_of(e), f64_of(b), w13q, w2q, cfg.Nr, cfg.Ns, cfg.K, gamma=cfg.gamma)
    ok, _ = check_routing(np_of(layer.topk_idx), np_of(layer.topk_gate), np_of(layer.expert_load),
                          o.routing, cfg.Nr)
    got = f64_of(out)
    assert np.all(np.isfinite(got))
    assert rel_l2(got[ok], o.out[ok]) <= 1e-2
    assert rel_l2(got[ok] - f64_of(u)[ok], (o.out - f64_of(u))[ok]) <= 1e-2


def test_moe_forward_one_call_matches_layer():
    """The one-call moe_forward gives the same output and bias step as
    MoeLayer on the same inputs (bit for bit: the same kernels)."""
    cfg = W.CONFIGS["mid_bf16"].with_(T=256, d=512, Nr=16, Ns=1, I=256, K=4)
    w13, w2 = W.make_expert_weights(cfg, "cuda")
    weights = M.ExpertWeights(M.MOE_BF16, w13, w2)
    u, e, b = W.make_tokens(cfg, 0, "cuda"), W.make_centroids(cfg, "cuda"), W.make_bias(cfg, "cuda")
    layer = M.MoeLayer(cfg.T, cfg.d, cfg.Nr, cfg.Ns, cfg.I, cfg.K, torch.bfloat16, weights, tile_m=32)
    ref = layer.forward(u, e, b).clone()
    b_ref = b.clone()
    layer.update_bias(b_ref, cfg.gamma)
    b_one = b.clone()
    out, one = M.moe_forward(u, e, b_one, weights, cfg.K, cfg.Ns, update_bias=True, gamma=cfg.gamma)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert torch.equal(b_one, b_ref)
    assert torch.equal(one.topk_idx, layer.topk_idx)
