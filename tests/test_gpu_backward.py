"""The backward pass on the GPU against the fp64 backward oracle
(oracle/backward.py) on the same seeded inputs: input, centroid and weight
gradients, the gate gradients, the saved pre-activations, and the
degenerate cases (zero output gradient, no tokens, experts with no rows).
Tolerance: relative L2 <= 1e-2, the bf16 bound of the forward (every stored
intermediate is bf16, 2^-9 relative, and the sums are fp32)."""
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
BASE = W.CONFIGS["mid_bf16"]
CASES = {
    # one 256-row tile per expert at most, full N tiles
    "small": BASE.with_(T=256, d=512, Nr=16, Ns=1, I=256, K=4),
    # I % 256 == 128 (a half N tile), ragged segments, two shared experts
    "ragged": BASE.with_(T=300, d=768, Nr=12, Ns=2, I=384, K=3),
    # several row tiles per expert and a longer K loop
    "mid_reduced": BASE.with_(T=1024, d=1024, Nr=32, Ns=2, I=640, K=6),
    # 16 N tiles of d, where the gate/up dgrad runs an expert's items in
    # groups of 8 row tiles, N-tile major; the shared expert has 9 row tiles
    # (a group of 8 and one of 1).  I / d near the V3 layer's, so that the
    # FFN part of du is not small next to the router part
    "wide": BASE.with_(T=2304, d=4096, Nr=8, Ns=1, I=1024, K=2),
}


def build(cfg, grad_dtype=torch.float32):
    w13, w2 = W.make_expert_weights(cfg, "cuda")
    layer = M.MoeLayer(cfg.T, cfg.d, cfg.Nr, cfg.Ns, cfg.I, cfg.K, torch.bfloat16,
                       M.ExpertWeights(M.MOE_BF16, w13, w2), tile_m=32, train=True, grad_dtype=grad_dtype)
    u = W.make_tokens(cfg, 0, "cuda")
    e = W.make_centroids(cfg, "cuda")
    b = W.make_bias(cfg, "cuda")
    return layer, w13, w2, u, e, b


def grad_out(cfg, seed=0):
    return W.make_free((cfg.T, cfg.d), 1.0, 100 + seed, "cuda", torch.bfloat16)


@pytest.mark.parametrize("name", list(CASES))
def test_backward_matches_oracle(name):
    cfg = CASES[name]
    print(f"backward parity {name}: {cfg}", flush=True)
    layer, w13, w2, u, e, b = build(cfg)
    out = layer.forward(u, e, b).clone()
    G = grad_out(cfg)
    du, de, dw13, dw2 = layer.backward(G, u, e)
    torch.cuda.synchronize()

    u64, e64, b64, w13_64, w2_64, G64 = map(f64_of, (u, e, b, w13, w2, G))
    r = O.route(u64, e64, b64, cfg.K)
    ok, tied = check_routing(np_of(layer.topk_idx), np_of(layer.topk_gate), np_of(layer.expert_load), r, cfg.Nr)
    assert not tied, "seeded inputs hold a near-tie; the gradients would not be comparable"

    # the training forward gives the same output as the plain forward
    plain = M.MoeLayer(cfg.T, cfg.d, cfg.Nr, cfg.Ns, cfg.I, cfg.K, torch.bfloat16,
                       M.ExpertWeights(M.MOE_BF16, w13, w2), tile_m=32)
    out_plain = plain.forward(u, e, b)
    torch.cuda.synchronize()
    assert torch.equal(out, out_plain)

    # saved pre-activations [a | b] of every token row
    row_token = np_of(layer.row_token)
    seg = np_of(layer.seg_offset)
    ab = f64_of(layer.ab)
    for ex in range(cfg.E):
        rows = np.arange(seg[ex], seg[ex + 1])
        rows = rows[row_token[rows] >= 0]
        want = u64[row_token[rows]] @ w13_64[ex].T
        assert rel_l2(ab[rows], want) <= TOL, ex

    gr = OB.layer_backward(u64, e64, b64, w13_64, w2_64, cfg.Nr, cfg.Ns, cfg.K, G64)
    errs = {"du": rel_l2(f64_of(du), gr.du), "de": rel_l2(f64_of(de), gr.de),
            "dw13": rel_l2(f64_of(dw13), gr.dw13), "dw2": rel_l2(f64_of(dw2), gr.dw2),
            "dgate": rel_l2(f64_of(layer.dgate), gr.dgate), "dz": rel_l2(f64_of(layer.dz), gr.dz),
            "du_ffn+router": rel_l2(f64_of(du) - G64, gr.du - G64)}
    print(errs, flush=True)
    for k, v in errs.items():
        assert v <= TOL, (k, v)


def test_zero_output_gradient_gives_zero_gradients():
    cfg = CASES["small"]
    layer, w13, w2, u, e, b = build(cfg)
    layer.forward(u, e, b)
    G = torch.zeros((cfg.T, cfg.d), dtype=torch.bfloat16, device="cuda")
    du, de, dw13, dw2 = layer.backward(G, u, e)
    torch.cuda.synchronize()
    for t in (du, de, dw13, dw2, layer.dgate, layer.dz):
        assert torch.count_nonzero(t).item() == 0


def test_backward_is_deterministic():
    cfg = CASES["mid_reduced"]
    layer, w13, w2, u, e, b = build(cfg, grad_dtype=torch.bfloat16)
    layer.forward(u, e, b)
    G = grad_out(cfg, 1)
    first = [t.clone() for t in layer.backward(G, u, e)]
    layer.forward(u, e, b)
    second = layer.backward(G, u, e)
    torch.cuda.synchronize()
    for a, c in zip(first, second):
        assert torch.equal(a, c)


def test_experts_without_rows_get_zero_gradients():
    """8 tokens over 64 routed experts: most experts receive no row; their
    weight and centroid gradients must be written as zeros."""
    cfg = CASES["small"].with_(T=8, Nr=64, K=2)
    layer, w13, w2, u, e, b = build(cfg)
    layer.dw13.fill_(float("nan"))
    layer.dw2.fill_(float("nan"))
    layer.de.fill_(float("nan"))
    layer.forward(u, e, b)
    G = grad_out(cfg, 2)
    du, de, dw13, dw2 = layer.backward(G, u, e)
    torch.cuda.synchronize()
    load = np_of(layer.expert_load)
    idle = np.nonzero(load == 0)[0]
    assert idle.size > 0
    assert torch.count_nonzero(dw13[idle]).item() == 0 and torch.count_nonzero(dw2[idle]).item() == 0
    assert torch.count_nonzero(de[idle]).item() == 0
    u64, e64, b64, w13_64, w2_64, G64 = map(f64_of, (u, e, b, w13, w2, G))
    gr = OB.layer_backward(u64, e64, b64, w13_64, w2_64, cfg.Nr, cfg.Ns, cfg.K, G64)
    for got, want in ((du, gr.du), (de, gr.de), (dw13, gr.dw13), (dw2, gr.dw2)):
        assert rel_l2(f64_of(got), want) <= TOL


def test_no_tokens():
    cfg = CASES["small"].with_(T=0)
    layer, w13, w2, u, e, b = build(cfg)
    layer.dw13.fill_(float("nan"))
    layer.dw2.fill_(float("nan"))
    layer.de.fill_(float("nan"))
    layer.forward(u, e, b)
    G = torch.empty((0, cfg.d), dtype=torch.bfloat16, device="cuda")
    du, de, dw13, dw2 = layer.backward(G, u, e)
    torch.cuda.synchronize()
    assert du.shape[0] == 0
    for t in (de, dw13, dw2):
        assert torch.count_nonzero(t).item() == 0


def oracle_grads(cfg, u, e, b, w13, w2, G):
    return OB.layer_backward(*map(f64_of, (u, e, b, w13, w2)), cfg.Nr, cfg.Ns, cfg.K, f64_of(G))


@pytest.mark.parametrize("shape", [dict(T=1), dict(T=96, Nr=8, K=8), dict(T=200, Nr=1, K=1)],
                         ids=["single_token", "every_expert_selected", "single_routed_expert"])
def test_backward_degenerate_routings(shape):
    """One token; K = N_r (every token selects every routed expert); N_r =
    K = 1 (every gate is 1, so no gradient reaches the centroid)."""
    cfg = CASES["small"].with_(**shape)
    layer, w13, w2, u, e, b = build(cfg)
    layer.forward(u, e, b)
    G = grad_out(cfg, 3)
    du, de, dw13, dw2 = layer.backward(G, u, e)
    torch.cuda.synchronize()
    gr = oracle_grads(cfg, u, e, b, w13, w2, G)
    for name, got, want in (("du", du, gr.du), ("dw13", dw13, gr.dw13), ("dw2", dw2, gr.dw2)):
        assert rel_l2(f64_of(got), want) <= TOL, name
    if cfg.Nr == cfg.K == 1:
        # g = s / s = 1 whatever s: the centroid and gate-score gradients are 0
        assert np.all(np.abs(f64_of(layer.dz)) <= 1e-6)
        assert np.all(np.abs(f64_of(de)) <= 1e-5)
    else:
        assert rel_l2(f64_of(de), gr.de) <= TOL


def test_backward_fp32_gradient_tensors():
    """dL/dh' given in fp32 and du requested in fp32 through the C ABI; the
    expert-row gradient dy stays bf16 (the GEMMs' operand type)."""
    cfg = CASES["small"]
    layer, w13, w2, u, e, b = build(cfg)
    layer.forward(u, e, b)
    G = grad_out(cfg, 4).float() * 0.5 + 1e-3      # values no bf16 tensor holds
    M.moe_combine_backward(G, layer.y, layer.inv_row, layer.topk_gate, layer.topk_score, layer.seg_offset,
                           cfg.Nr, cfg.Ns, layer.dy, layer.dgate, layer.dz, layer.dz_row)
    M.moe_expert_gemm_backward(u, w13, w2, layer.h, layer.ab, layer.dy, cfg.T, cfg.K, cfg.Nr, cfg.Ns, cfg.d, cfg.I,
                               32, layer.seg_offset, layer.row_token, layer.tile_map, layer.n_tiles, layer.bwd_ws,
                               layer.dx, layer.dw13, layer.dw2)
    du = torch.empty((cfg.T, cfg.d), dtype=torch.float32, device="cuda")
    M.moe_route_backward(G, layer.dx, u, e, layer.topk_idx, layer.inv_row, layer.dz, layer.dz_row,
                         layer.seg_offset, layer.row_token, cfg.Nr, cfg.Ns, du, layer.de)
    torch.cuda.synchronize()
    gr = oracle_grads(cfg, u, e, b, w13, w2, G)
    assert rel_l2(f64_of(du), gr.du) <= TOL
    assert rel_l2(f64_of(du) - f64_of(G), gr.du - f64_of(G)) <= TOL
    assert rel_l2(f64_of(layer.de), gr.de) <= TOL
    assert rel_l2(f64_of(layer.dgate), gr.dgate) <= TOL


@pytest.mark.parametrize("tile_m", [1, 256])
def test_backward_segment_padding(tile_m):
    """Segments padded to 1 row (no padding) and to 256 rows (every segment
    a whole tile): padding rows must neither contribute nor be read."""
    cfg = CASES["small"].with_(T=200, K=5)
    w13, w2 = W.make_expert_weights(cfg, "cuda")
    layer = M.MoeLayer(cfg.T, cfg.d, cfg.Nr, cfg.Ns, cfg.I, cfg.K, torch.bfloat16,
                       M.ExpertWeights(M.MOE_BF16, w13, w2), tile_m=tile_m, train=True)
    u, e, b = W.make_tokens(cfg, 0, "cuda"), W.make_centroids(cfg, "cuda"), W.make_bias(cfg, "cuda")
    layer.dy.fill_(float("nan"))          # padding rows of the row buffers hold NaN
    layer.dx.fill_(float("nan"))
    layer.forward(u, e, b)
    G = grad_out(cfg, 5)
    du, de, dw13, dw2 = layer.backward(G, u, e)
    torch.cuda.synchronize()
    gr = oracle_grads(cfg, u, e, b, w13, w2, G)
    for name, got, want in (("du", du, gr.du), ("de", de, gr.de), ("dw13", dw13, gr.dw13), ("dw2", dw2, gr.dw2)):
        assert rel_l2(f64_of(got), want) <= TOL, name


def test_backward_top16():
    """K = 16, the largest K the library takes."""
    cfg = CASES["small"].with_(T=128, Nr=32, K=16)
    layer, w13, w2, u, e, b = build(cfg)
    layer.forward(u, e, b)
    G = grad_out(cfg, 6)
    du, de, dw13, dw2 = layer.backward(G, u, e)
    torch.cuda.synchronize()
    gr = oracle_grads(cfg, u, e, b, w13, w2, G)
    for name, got, want in (("du", du, gr.du), ("de", de, gr.de), ("dw13", dw13, gr.dw13), ("dw2", dw2, gr.dw2),
                            ("dz", layer.dz, gr.dz)):
        assert rel_l2(f64_of(got), want) <= TOL, name
