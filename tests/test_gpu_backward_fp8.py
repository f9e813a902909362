"""The backward with its input-gradient products on E4M3 operands
(moe_expert_gemm_backward_w8, MoeLayer(dgrad_weights=...)) against the fp64
oracle's layer_backward(fp8_dgrad=True) on the same seeded inputs.

The oracle quantises the same bf16 weights in 128x128 blocks and, like the
GPU, decides the 1x128 codes of the activation gradients from their bf16
values (dy, then [da | db] computed at the bf16 pre-activations), so the two
sides quantise the same values up to fp32 accumulation order.  Tolerances:
relative L2 <= 5e-3 for what flows through the E4M3 products of the
backward (du, its expert part and dW13: the E4M3 bound of 3e-2 would only
apply if the codes were decided from different values), 1e-2 for the
paths that do not (dW2, gate and score gradients, de)."""
import numpy as np
import pytest
import torch

import sparse_expert_routing_sigmoid_amd as M
import workloads as W
from moe_testutil import check_routing, f64_of, np_of, rel_l2
from oracle import backward as OB
from oracle import moe as O

pytestmark = pytest.mark.gpu

TOL8, TOL, MIRROR = 3e-2, 1e-2, 5e-3
BASE = W.CONFIGS["mid_bf16"]
CASES = {
    "small": BASE.with_(T=256, d=512, Nr=16, Ns=1, I=256, K=4),
    # I % 256 == 128: the last N tile of the down dgrad is half a tile
    "ragged": BASE.with_(T=300, d=768, Nr=12, Ns=2, I=384, K=3),
    "mid_reduced": BASE.with_(T=1024, d=1024, Nr=32, Ns=2, I=640, K=6),
    # 16 N tiles of d: the gate/up dgrad's items in groups of row tiles
    "wide": BASE.with_(T=2304, d=4096, Nr=8, Ns=1, I=1024, K=2),
}


def build(cfg, grad_dtype=torch.float32):
    w13, w2 = W.make_expert_weights(cfg, "cuda")
    w8 = M.quantize_weights(w13, w2)
    layer = M.MoeLayer(cfg.T, cfg.d, cfg.Nr, cfg.Ns, cfg.I, cfg.K, torch.bfloat16,
                       M.ExpertWeights(M.MOE_BF16, w13, w2), tile_m=32, train=True, grad_dtype=grad_dtype,
                       dgrad_weights=w8)
    u = W.make_tokens(cfg, 0, "cuda")
    e = W.make_centroids(cfg, "cuda")
    b = W.make_bias(cfg, "cuda")
    return layer, w13, w2, u, e, b


@pytest.mark.parametrize("name", list(CASES))
def test_fp8_dgrad_backward_matches_oracle(name):
    cfg = CASES[name]
    print(f"fp8-dgrad backward parity {name}: {cfg}", flush=True)
    layer, w13, w2, u, e, b = build(cfg)
    layer.forward(u, e, b)
    G = W.make_free((cfg.T, cfg.d), 1.0, 100, "cuda", torch.bfloat16)
    du, de, dw13, dw2 = layer.backward(G, u, e)
    torch.cuda.synchronize()

    u64, e64, b64, w13_64, w2_64, G64 = map(f64_of, (u, e, b, w13, w2, G))
    r = O.route(u64, e64, b64, cfg.K)
    ok, tied = check_routing(np_of(layer.topk_idx), np_of(layer.topk_gate), np_of(layer.expert_load), r, cfg.Nr)
    assert not tied, "seeded inputs hold a near-tie; the gradients would not be comparable"
    gr = OB.layer_backward(u64, e64, b64, w13_64, w2_64, cfg.Nr, cfg.Ns, cfg.K, G64, fp8_dgrad=True)
    errs8 = {"du": rel_l2(f64_of(du), gr.du), "du_ffn": rel_l2(f64_of(du) - G64 - gr.du_router, gr.du_ffn),
             "dw13": rel_l2(f64_of(dw13), gr.dw13)}
    errs = {"dw2": rel_l2(f64_of(dw2), gr.dw2), "de": rel_l2(f64_of(de), gr.de),
            "dgate": rel_l2(f64_of(layer.dgate), gr.dgate), "dz": rel_l2(f64_of(layer.dz), gr.dz)}
    print(errs8, errs, flush=True)
    for k, v in errs8.items():
        assert v <= MIRROR, (k, v)
    for k, v in errs.items():
        assert v <= TOL, (k, v)
    # the E4M3 products do differ from the exact ones
    exact = OB.layer_backward(u64, e64, b64, w13_64, w2_64, cfg.Nr, cfg.Ns, cfg.K, G64)
    assert rel_l2(f64_of(du) - G64 - gr.du_router, exact.du_ffn) > 1e-3


def test_fp8_dgrad_zero_gradient_and_determinism():
    cfg = CASES["mid_reduced"]
    layer, w13, w2, u, e, b = build(cfg, grad_dtype=torch.bfloat16)
    layer.forward(u, e, b)
    G0 = torch.zeros((cfg.T, cfg.d), dtype=torch.bfloat16, device="cuda")
    for t in layer.backward(G0, u, e):
        assert torch.count_nonzero(t).item() == 0
    G = W.make_free((cfg.T, cfg.d), 1.0, 101, "cuda", torch.bfloat16)
    first = [t.clone() for t in layer.backward(G, u, e)]
    second = layer.backward(G, u, e)
    torch.cuda.synchronize()
    for a, c in zip(first, second):
        assert torch.equal(a, c)
        assert torch.isfinite(a.float()).all()


def test_fp8_dgrad_rejects_bf16_weights():
    cfg = CASES["small"]
    w13, w2 = W.make_expert_weights(cfg, "cuda")
    with pytest.raises(ValueError):
        M.MoeLayer(cfg.T, cfg.d, cfg.Nr, cfg.Ns, cfg.I, cfg.K, torch.bfloat16, M.ExpertWeights(M.MOE_BF16, w13, w2),
                   train=True, dgrad_weights=M.ExpertWeights(M.MOE_BF16, w13, w2))


TRAIN_CASES = {
    "small": CASES["small"],
    # several row tiles per expert; the FP8 forward needs I % 256 == 0
    "mid": BASE.with_(T=1024, d=1024, Nr=32, Ns=2, I=512, K=6),
}


@pytest.mark.parametrize("name", list(TRAIN_CASES))
def test_fp8_training_step_matches_oracle(name):
    """MoeLayer(train=True, x_fp8=True, E4M3 weights, wgrad_fp8=False): the
    E4M3 training forward (keeping [a|b] and the E4M3 h in bf16) and the
    backward with E4M3 input-gradient products and bf16 weight gradients
    (moe_expert_gemm_backward_w8), against layer_backward(fp8_train=True) on
    the oracle's own 128x128 quantisation of the same bf16 weights."""
    from oracle.e4m3 import dequantize_tiles, quantize_tiles
    cfg = TRAIN_CASES[name]
    print(f"fp8 training step parity {name}: {cfg}", flush=True)
    w13, w2 = W.make_expert_weights(cfg, "cuda")
    w8 = M.quantize_weights(w13, w2)
    layer = M.MoeLayer(cfg.T, cfg.d, cfg.Nr, cfg.Ns, cfg.I, cfg.K, torch.bfloat16, w8, x_fp8=True, tile_m=32,
                       train=True, wgrad_fp8=False)
    plain = M.MoeLayer(cfg.T, cfg.d, cfg.Nr, cfg.Ns, cfg.I, cfg.K, torch.bfloat16, w8, x_fp8=True, tile_m=32)
    u, e, b = W.make_tokens(cfg, 0, "cuda"), W.make_centroids(cfg, "cuda"), W.make_bias(cfg, "cuda")
    out = layer.forward(u, e, b).clone()
    out_plain = plain.forward(u, e, b)
    G = W.make_free((cfg.T, cfg.d), 1.0, 100, "cuda", torch.bfloat16)
    du, de, dw13, dw2 = layer.backward(G, u, e)
    torch.cuda.synchronize()
    assert torch.equal(out, out_plain)   # the training forward computes the same layer output

    u64, e64, b64, G64 = map(f64_of, (u, e, b, G))
    r = O.route(u64, e64, b64, cfg.K)
    ok, tied = check_routing(np_of(layer.topk_idx), np_of(layer.topk_gate), np_of(layer.expert_load), r, cfg.Nr)
    assert not tied, "seeded inputs hold a near-tie; the gradients would not be comparable"
    deq = lambda w: dequantize_tiles(*quantize_tiles(w.astype(np.float32), 128, 128), 128, 128)
    w13q = np.stack([deq(x) for x in f64_of(w13)])
    w2q = np.stack([deq(x) for x in f64_of(w2)])
    gr = OB.layer_backward(u64, e64, b64, w13q, w2q, cfg.Nr, cfg.Ns, cfg.K, G64, fp8_train=True)
    errs = {"du": rel_l2(f64_of(du), gr.du), "du_ffn": rel_l2(f64_of(du) - G64 - gr.du_router, gr.du_ffn),
            "dw13": rel_l2(f64_of(dw13), gr.dw13), "dw2": rel_l2(f64_of(dw2), gr.dw2),
            "de": rel_l2(f64_of(de), gr.de), "dgate": rel_l2(f64_of(layer.dgate), gr.dgate),
            "dz": rel_l2(f64_of(layer.dz), gr.dz)}
    print(errs, flush=True)
    for k, v in errs.items():
        # du and dW13 pass through the E4M3 input-gradient products; dW2, de,
        # dgate and dz through none of the backward's
        assert v <= (MIRROR if k in ("du", "du_ffn", "dw13") else TOL), (k, v)


def test_fp8_dgrad_experts_without_rows_and_no_tokens():
    """Experts that receive no row get zero weight and centroid gradients on
    the E4M3 path too, and a step without tokens writes zeros."""
    cfg = CASES["small"].with_(T=8, Nr=64, K=2)
    layer, w13, w2, u, e, b = build(cfg)
    for t in (layer.dw13, layer.dw2, layer.de):
        t.fill_(float("nan"))
    layer.forward(u, e, b)
    G = W.make_free((cfg.T, cfg.d), 1.0, 102, "cuda", torch.bfloat16)
    du, de, dw13, dw2 = layer.backward(G, u, e)
    torch.cuda.synchronize()
    idle = np.nonzero(np_of(layer.expert_load) == 0)[0]
    assert idle.size > 0
    assert torch.count_nonzero(dw13[idle]).item() == 0 and torch.count_nonzero(dw2[idle]).item() == 0
    assert torch.count_nonzero(de[idle]).item() == 0
    gr = OB.layer_backward(*map(f64_of, (u, e, b, w13, w2)), cfg.Nr, cfg.Ns, cfg.K, f64_of(G), fp8_dgrad=True)
    for name, got, want in (("du", du, gr.du), ("dw13", dw13, gr.dw13), ("dw2", dw2, gr.dw2)):
        assert rel_l2(f64_of(got), want) <= TOL8, name

    cfg0 = CASES["small"].with_(T=0)
    layer, w13, w2, u, e, b = build(cfg0)
    for t in (layer.dw13, layer.dw2, layer.de):
        t.fill_(float("nan"))
    layer.forward(u, e, b)
    du, de, dw13, dw2 = layer.backward(torch.empty((0, cfg0.d), dtype=torch.bfloat16, device="cuda"), u, e)
    torch.cuda.synchronize()
    for t in (de, dw13, dw2):
        assert torch.count_nonzero(t).item() == 0


def test_fp8_training_step_single_token():
    """One token on the E4M3 training path: one row per selected expert."""
    from oracle.e4m3 import dequantize_tiles, quantize_tiles
    cfg = TRAIN_CASES["small"].with_(T=1)
    w13, w2 = W.make_expert_weights(cfg, "cuda")
    w8 = M.quantize_weights(w13, w2)
    layer = M.MoeLayer(cfg.T, cfg.d, cfg.Nr, cfg.Ns, cfg.I, cfg.K, torch.bfloat16, w8, x_fp8=True, tile_m=32,
                       train=True, wgrad_fp8=False)
    u, e, b = W.make_tokens(cfg, 0, "cuda"), W.make_centroids(cfg, "cuda"), W.make_bias(cfg, "cuda")
    layer.forward(u, e, b)
    G = W.make_free((cfg.T, cfg.d), 1.0, 103, "cuda", torch.bfloat16)
    du, de, dw13, dw2 = layer.backward(G, u, e)
    torch.cuda.synchronize()
    deq = lambda w: dequantize_tiles(*quantize_tiles(w.astype(np.float32), 128, 128), 128, 128)
    w13q = np.stack([deq(x) for x in f64_of(w13)])
    w2q = np.stack([deq(x) for x in f64_of(w2)])
    gr = OB.layer_backward(*map(f64_of, (u, e, b)), w13q, w2q, cfg.Nr, cfg.Ns, cfg.K, f64_of(G), fp8_train=True)
    for name, got, want in (("du", du, gr.du), ("de", de, gr.de), ("dw13", dw13, gr.dw13), ("dw2", dw2, gr.dw2)):
        assert rel_l2(f64_of(got), want) <= TOL8, name
