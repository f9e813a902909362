"""E4M3 weight gradients at the full V3 size on the E4M3 training step
(T = 8192, d = 7168, 256 routed + 1 shared experts, I = 2048, top-8, Zipf
loads), in the launch configuration `bench.py --train --config
v3_train_fp8` times (MoeLayer, tile_m = 32, bf16 gradients).

dW2_e = R(dy_e)^T R(h_e) and dW13_e = R([da | db]_e)^T R(x_e) (reading B5)
depend only on the rows of expert e, and R works column by column, so a
block of columns of both operands gives the matching block of dW exactly.
For the least loaded, a median and the most loaded routed expert and the
shared expert (8192 rows, 64 runs), blocks of 256 x 256 outputs are
recomputed by oracle.backward.fp8_wgrad from the GPU's own bf16 operands:
dy and h as the layer keeps them, x = Q(u) decoded, [da | db] from the head
of the backward's workspace, where moe_expert_gemm_backward_f8 leaves it.
The comparison allows the accumulation error of the scaled matrix
instruction (BLOCK_ACC, see test_gpu_backward_f8.py), fp32 rounding and one
bf16 rounding."""
import numpy as np
import pytest
import torch

import sparse_expert_routing_sigmoid_amd as M
import workloads as W
from moe_testutil import f64_of, np_of
from oracle import backward as OB
from test_gpu_backward_f8 import BLOCK_ACC

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def run():
    cfg = W.CONFIGS["v3_train_fp8"]
    print(f"[f8 backward fullsize] T={cfg.T} d={cfg.d} E={cfg.E} I={cfg.I} K={cfg.K}", flush=True)
    u, e, b = W.make_tokens(cfg, 0, "cuda"), W.make_centroids(cfg, "cuda"), W.make_bias(cfg, "cuda")
    w13, w2 = W.make_expert_weights(cfg, "cuda")
    w8 = M.quantize_weights(w13, w2)
    del w13, w2
    layer = M.MoeLayer(cfg.T, cfg.d, cfg.Nr, cfg.Ns, cfg.I, cfg.K, torch.bfloat16, w8, x_fp8=True, tile_m=32,
                       train=True, grad_dtype=torch.bfloat16)
    assert layer.wgrad_fp8
    G = W.make_free((cfg.T, cfg.d), 1.0, 100, "cuda", torch.bfloat16)
    layer.forward(u, e, b)
    layer.backward(G, u, e)
    torch.cuda.synchronize()
    print("[f8 backward fullsize] GPU done", flush=True)
    P = layer.P_max
    dab = layer.bwd_ws[:P * 2 * cfg.I * 2].view(torch.bfloat16).view(P, 2 * cfg.I)
    loads = np_of(layer.expert_load)
    order = np.argsort(loads, kind="stable")
    live = order[loads[order] > 0]
    picks = [int(live[0]), int(live[live.size // 2]), int(live[-1])] + list(range(cfg.Nr, cfg.Nr + cfg.Ns))
    return dict(cfg=cfg, layer=layer, dab=dab, picks=picks, so=np_of(layer.seg_offset), rt=np_of(layer.row_token))


def check_block(name, got, a_rows, b_rows):
    ra, rb = OB.quantize_token_runs(a_rows), OB.quantize_token_runs(b_rows)
    want = ra.T @ rb
    n = a_rows.shape[0]
    sab = np.abs(ra).T @ np.abs(rb)
    bound = (BLOCK_ACC + (n + 4) * 2.0 ** -24) * sab + np.abs(want) * 2.0 ** -8 * (1 + 1e-6) + 1e-30
    bad = np.abs(got - want) > bound
    assert not bad.any(), (name, int(bad.sum()), float(np.abs(got - want).max()))


@pytest.mark.parametrize("which", ["dw2", "dw13"])
def test_weight_gradient_blocks_at_full_size(run, which):
    cfg, layer, so, rt = run["cfg"], run["layer"], run["so"], run["rt"]
    rng = np.random.default_rng(11 if which == "dw2" else 12)
    for i in run["picks"]:
        rows = np.arange(so[i], so[i + 1])
        rows = rows[rt[rows] >= 0]
        if which == "dw2":
            M_dim, N_dim = cfg.d, cfg.I
        else:
            M_dim, N_dim = 2 * cfg.I, cfg.d
        m0 = int(rng.integers(0, M_dim // 256)) * 256
        n0 = int(rng.integers(0, N_dim // 256)) * 256
        r_t = torch.from_numpy(rows).cuda()
        if which == "dw2":
            a = f64_of(layer.dy.index_select(0, r_t)[:, m0:m0 + 256])
            bm = f64_of(layer.h.index_select(0, r_t)[:, n0:n0 + 256])
            got = f64_of(layer.dw2[i, m0:m0 + 256, n0:n0 + 256])
        else:
            a = f64_of(run["dab"].index_select(0, r_t)[:, m0:m0 + 256])
            tok = torch.from_numpy(rt[rows].astype(np.int64)).cuda()
            bm = f64_of(layer.xdq.index_select(0, tok)[:, n0:n0 + 256])
            got = f64_of(layer.dw13[i, m0:m0 + 256, n0:n0 + 256])
        print(f"  {which} expert {i}: {rows.size} rows, block ({m0}, {n0})", flush=True)
        check_block(f"{which}[{i}]", got, a, bm)
