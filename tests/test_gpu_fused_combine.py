"""moe_expert_gemm_combine: the combine equation fused into the down
projection (every expert row added to its token's row of an fp32 output by
atomic adds), against the fp64 oracle's layer forward and against the
deterministic moe_expert_gemm + moe_combine on the same inputs.

The fused sum adds the same fp32 terms in an order that is not fixed, so it
matches the deterministic path with fp32 expert rows to fp32 rounding (rel
L2 <= 1e-5), and the oracle within the layer tolerance (1e-2 bf16, 3e-2
E4M3), the FFN part on its own too."""
import numpy as np
import pytest
import torch

import sparse_expert_routing_sigmoid_amd as M
import workloads as W
from moe_testutil import check_routing, f64_of, np_of, rel_l2
from oracle import e4m3 as OE
from oracle import moe as O

pytestmark = pytest.mark.gpu

BASE = W.CONFIGS["mid_bf16"]
CASES = {
    "bf16_small": (BASE.with_(T=512, d=512, Nr=16, Ns=1, I=256, K=4), False),
    "bf16_mid": (BASE.with_(T=1024, d=1024, Nr=32, Ns=2, I=640, K=6), False),
    "fp8_small": (BASE.with_(T=512, d=512, Nr=16, Ns=1, I=512, K=4), True),
}
FLAGS = [0, M.MOE_COMBINE_NO_RESIDUAL, M.MOE_COMBINE_NO_SHARED, M.MOE_COMBINE_NO_ROUTED | M.MOE_COMBINE_NO_RESIDUAL]


def layer_of(cfg, fp8):
    w13, w2 = W.make_expert_weights(cfg, "cuda")
    if fp8:
        w13 = w13.float()
        w2 = w2.float()
        weights = M.quantize_weights(w13, w2)
    else:
        weights = M.ExpertWeights(M.MOE_BF16, w13, w2)
    layer = M.MoeLayer(cfg.T, cfg.d, cfg.Nr, cfg.Ns, cfg.I, cfg.K, torch.bfloat16, weights, x_fp8=fp8, tile_m=32,
                       out_dtype=torch.float32)
    return layer, weights, w13, w2


def fused(layer, cfg, u, flags):
    w = layer.w
    x, xs = (layer.xq, layer.xs) if layer.x_fp8 else (u, None)
    if layer.x_fp8:
        M.fp8_quantize_tiles(u, 1, layer.xq, layer.xs)
    ws = torch.empty((M.moe_gemm_combine_workspace_bytes(cfg.T, cfg.K, cfg.Nr, cfg.Ns, cfg.d, cfg.I, 32, layer.x_t,
                                                         w.w_t),), dtype=torch.uint8, device="cuda")
    out = torch.full((cfg.T, cfg.d), float("nan"), dtype=torch.float32, device="cuda")
    M.moe_expert_gemm_combine(x, xs, w.w_t, w.w13, w.w13_scale, w.w2, w.w2_scale, cfg.T, cfg.K, cfg.Nr, cfg.Ns, cfg.d,
                              cfg.I, 32, layer.seg_offset, layer.row_token, layer.tile_map, layer.n_tiles,
                              layer.inv_row, layer.topk_gate, u, ws, out, flags, x_t=layer.x_t)
    return out


@pytest.mark.parametrize("flags", FLAGS)
@pytest.mark.parametrize("name", list(CASES))
def test_fused_combine_matches_deterministic_and_oracle(name, flags):
    cfg, fp8 = CASES[name]
    print(f"fused combine {name} flags {flags}: {cfg}", flush=True)
    layer, weights, w13, w2 = layer_of(cfg, fp8)
    u, e, b = W.make_tokens(cfg, 0, "cuda"), W.make_centroids(cfg, "cuda"), W.make_bias(cfg, "cuda")
    layer.route(u, e, b)
    layer.permute()
    got = fused(layer, cfg, u, flags)
    layer.experts(u)                                  # deterministic path, fp32 expert rows
    det = layer.combine(u, flags=flags).clone()
    torch.cuda.synchronize()
    g, dt = f64_of(got), f64_of(det)
    assert np.all(np.isfinite(g))
    assert rel_l2(g, dt) <= 1e-5, rel_l2(g, dt)

    u64 = f64_of(u)
    r = O.route(u64, f64_of(e), f64_of(b), cfg.K)
    _, tied = check_routing(np_of(layer.topk_idx), np_of(layer.topk_gate), np_of(layer.expert_load), r, cfg.Nr)
    assert not tied
    if fp8:
        deq = lambda m: OE.dequantize_tiles(*OE.quantize_tiles(m, 128, 128), 128, 128)
        w13o = np.stack([deq(x) for x in w13.cpu().numpy()])
        w2o = np.stack([deq(x) for x in w2.cpu().numpy()])
    else:
        w13o, w2o = f64_of(w13), f64_of(w2)
    lf = O.layer_forward(u64, f64_of(e), f64_of(b), w13o, w2o, cfg.Nr, cfg.Ns, cfg.K, x_quant=fp8, h_quant=fp8)
    want = O.combine(u64, lf.y_shared, lf.y_routed, r.gate, residual=not flags & 1, shared=not flags & 2,
                     routed=not flags & 4)
    tol = 3e-2 if fp8 else 1e-2
    err = rel_l2(g, want)
    print(f"  rel L2 vs deterministic {rel_l2(g, dt):.2e}, vs oracle {err:.2e}", flush=True)
    assert err <= tol
    if not flags & 1:
        assert rel_l2(g - u64, want - u64) <= tol


def test_fused_combine_full_size_bf16():
    """The 8192-token V3 bf16 prefill layer in the benchmark's launch
    configuration: the fused output equals the deterministic path with fp32
    expert rows to fp32 rounding, token by token."""
    cfg = W.CONFIGS["v3_prefill_bf16"]
    print(f"fused combine full size: {cfg.name}", flush=True)
    layer, weights, w13, w2 = layer_of(cfg, False)
    del w13, w2
    u, e, b = W.make_tokens(cfg, 0, "cuda"), W.make_centroids(cfg, "cuda"), W.make_bias(cfg, "cuda")
    layer.route(u, e, b)
    layer.permute()
    got = fused(layer, cfg, u, 0)
    layer.experts(u)
    det = layer.combine(u).clone()
    torch.cuda.synchronize()
    diff = (got.double() - det.double())
    per_tok = (diff.norm(dim=1) / det.double().sub(u.double()).norm(dim=1)).max().item()
    total = (diff.norm() / det.double().norm()).item()
    print(f"  rel L2 {total:.2e}, worst token FFN part {per_tok:.2e}", flush=True)
    assert torch.isfinite(got).all()
    assert total <= 1e-6 and per_tok <= 1e-5
