"""GPU parity of moe_expert_gemm against the oracle's per-row expert FFN on
the oracle's own layout: every real row y[row] = FFN_seg(x[row_token[row]])."""
import numpy as np
import pytest
import torch

import sparse_expert_routing_sigmoid_amd as M
import workloads as W
from moe_testutil import f64_of, np_of, rel_l2
from oracle import moe as O
from test_gpu_permute import make_idx

pytestmark = pytest.mark.gpu


def upload_layout(lay):
    c = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    tiles = torch.zeros((max(lay.n_tiles, 1), 4), dtype=torch.int32)
    tiles[: lay.n_tiles] = torch.from_numpy(lay.tile_map)
    return c(lay.seg_offset), c(lay.row_token), tiles.cuda(), torch.tensor([lay.n_tiles], dtype=torch.int32).cuda()


def gpu_expert_rows(cfg, x, x_scale, weights, lay, tile_m, y_dtype):
    seg, rt, tm, nt = upload_layout(lay)
    T = cfg.T
    x_t = M.dtype_code(x)
    P = len(lay.row_token)
    ws = torch.empty((M.moe_gemm_workspace_bytes(T, cfg.K, cfg.Nr, cfg.Ns, cfg.d, cfg.I, tile_m, x_t,
                                                 weights.w_t),), dtype=torch.uint8, device="cuda")
    y = torch.full((P, cfg.d), float("nan"), dtype=y_dtype, device="cuda")
    # the layout is sized for this tile_m and K, so the capacities agree
    assert P == M.moe_permute_rows(T, cfg.K, cfg.Nr, cfg.Ns, tile_m)
    M.moe_expert_gemm(x, x_scale, weights.w_t, weights.w13, weights.w13_scale, weights.w2, weights.w2_scale,
                      T, cfg.K, cfg.Nr, cfg.Ns, cfg.d, cfg.I, tile_m, seg, rt, tm, nt, ws, y)
    torch.cuda.synchronize()
    return f64_of(y)


def run_case(cfg, idx, tile_m=16, y_dtype=None, tol=1e-2):
    u = W.make_tokens(cfg, 0, "cuda")
    w13, w2 = W.make_expert_weights(cfg, "cuda")
    wt = M.MOE_F32 if cfg.weights == "f32" else M.MOE_BF16
    weights = M.ExpertWeights(wt, w13, w2)
    lay = O.permute_layout(idx.numpy(), cfg.Nr, cfg.Ns, tile_m, M.MOE_TILE_ROWS)
    y_dtype = u.dtype if y_dtype is None else y_dtype
    y = gpu_expert_rows(cfg, u, None, weights, lay, tile_m, y_dtype)
    want = O.expert_rows(f64_of(u), f64_of(w13), f64_of(w2), lay, cfg.Nr, cfg.Ns)
    real = lay.row_token[: lay.seg_offset[-1]] >= 0
    got = y[: lay.seg_offset[-1]][real]
    ref = want[real]
    assert np.all(np.isfinite(got))
    err = rel_l2(got, ref)
    assert err <= tol, err
    # every segment on its own (catches a wrong expert or a wrong tile)
    for s in range(cfg.E):
        r0, r1 = lay.seg_offset[s], lay.seg_offset[s + 1]
        m = lay.row_token[r0:r1] >= 0
        if m.any():
            assert rel_l2(y[r0:r1][m], want[r0:r1][m]) <= 2 * tol, s
    return err


def test_f32_tiny_layer_rows():
    cfg = W.CONFIGS["tiny_fp32"]
    idx = make_idx(cfg.T, cfg.Nr, cfg.K, 3)
    assert run_case(cfg, idx, tile_m=32, tol=1e-5) < 1e-5


@pytest.mark.parametrize("T,I,tile_m", [(300, 128, 16), (300, 192, 32), (77, 64, 1), (600, 256, 256)])
def test_bf16_ragged_tiles(T, I, tile_m):
    cfg = W.CONFIGS["mid_bf16"].with_(T=T, d=256, I=I, Nr=8, Ns=1, K=2)
    idx = make_idx(T, cfg.Nr, cfg.K, T + I, hot=[5])        # expert 5 gets every token: > 256 rows
    run_case(cfg, idx, tile_m=tile_m)


def test_bf16_f32_output():
    cfg = W.CONFIGS["mid_bf16"].with_(T=200, d=384, I=128, Nr=6, Ns=2, K=3)
    run_case(cfg, make_idx(cfg.T, cfg.Nr, cfg.K, 9), y_dtype=torch.float32)


def test_bf16_mid_config_rows():
    cfg = W.CONFIGS["mid_bf16"]
    u = W.make_tokens(cfg, 0, "cpu")
    r = O.route(f64_of(u), f64_of(W.make_centroids(cfg, "cpu")), f64_of(W.make_bias(cfg, "cpu")), cfg.K)
    run_case(cfg, torch.from_numpy(r.idx), tile_m=32)


@pytest.mark.parametrize("T,d,I,Ns,tile_m,ydt", [(700, 512, 256, 2, 32, torch.bfloat16),
                                                 (700, 512, 256, 1, 16, torch.float32),
                                                 (1030, 768, 384, 1, 1, torch.bfloat16),
                                                 (64, 2048, 1024, 1, 32, torch.bfloat16)])
def test_bf16_persistent_kernel_shapes(T, d, I, Ns, tile_m, ydt):
    """Shapes the persistent XCD-aware kernel takes (d % 256 == 0, I % 128 == 0):
    segments of 1..T rows, multi-tile segments, partial 32-row groups."""
    cfg = W.CONFIGS["mid_bf16"].with_(T=T, d=d, I=I, Nr=12, Ns=Ns, K=3)
    idx = make_idx(T, cfg.Nr, cfg.K, T + d, hot=[4, 9])
    run_case(cfg, idx, tile_m=tile_m, y_dtype=ydt)


# ------------------------------------------------------------ E4M3 x E4M3 --
def oracle_fp8_weights(w13, w2):
    """Each expert matrix through the oracle's 128x128 block quantiser, decoded."""
    from oracle.e4m3 import dequantize_tiles, quantize_tiles
    deq = lambda m: dequantize_tiles(*quantize_tiles(m, 128, 128), 128, 128)
    a13, a2 = np_of(w13).astype(np.float32), np_of(w2).astype(np.float32)
    return (np.stack([deq(a13[e]) for e in range(a13.shape[0])]),
            np.stack([deq(a2[e]) for e in range(a2.shape[0])]))


def run_fp8_case(cfg, idx, tile_m=32, y_dtype=torch.bfloat16, tol=3e-2):
    """GPU: u and the weights quantised by fp8_quantize_tiles, both GEMMs on
    E4M3 codes, h re-quantised in 1x128 tiles.  Oracle: the same
    quantisation points on the oracle's own quantiser (R8), in fp64."""
    u = W.make_tokens(cfg, 0, "cuda")
    w13, w2 = W.make_expert_weights(cfg, "cuda")
    weights = M.quantize_weights(w13, w2)
    xq = torch.empty((cfg.T, cfg.d), dtype=torch.uint8, device="cuda")
    xs = torch.empty((cfg.T, cfg.d // 128), dtype=torch.float32, device="cuda")
    M.fp8_quantize_tiles(u, 1, xq, xs)
    lay = O.permute_layout(idx.numpy(), cfg.Nr, cfg.Ns, tile_m, M.MOE_TILE_ROWS)
    y = gpu_expert_rows(cfg, xq, xs, weights, lay, tile_m, y_dtype)
    w13q, w2q = oracle_fp8_weights(w13, w2)
    want = O.expert_rows(O.quantize_activations(f64_of(u)), w13q, w2q, lay, cfg.Nr, cfg.Ns, h_quant=True)
    real = lay.row_token[: lay.seg_offset[-1]] >= 0
    got = y[: lay.seg_offset[-1]][real]
    assert np.all(np.isfinite(got))
    err = rel_l2(got, want[real])
    assert err <= tol, err
    for s in range(cfg.E):
        r0, r1 = lay.seg_offset[s], lay.seg_offset[s + 1]
        m = lay.row_token[r0:r1] >= 0
        if m.any():
            assert rel_l2(y[r0:r1][m], want[r0:r1][m]) <= 2 * tol, s
    return err


@pytest.mark.parametrize("T,d,I,Nr,Ns,tile_m,ydt", [(300, 256, 256, 12, 1, 16, torch.bfloat16),
                                                    (700, 512, 256, 12, 2, 32, torch.bfloat16),
                                                    (700, 512, 512, 12, 1, 16, torch.float32),
                                                    (1030, 768, 256, 12, 1, 1, torch.bfloat16),
                                                    (600, 256, 256, 12, 1, 256, torch.bfloat16),
                                                    (64, 2048, 1024, 12, 1, 32, torch.bfloat16),
                                                    (40, 8192, 256, 4, 1, 64, torch.bfloat16)])
def test_fp8_persistent_kernel_shapes(T, d, I, Nr, Ns, tile_m, ydt):
    """E4M3 x E4M3 kernel: ragged segments, tiles of 1..256 rows, several
    K blocks, both output types, and the largest supported d (64 K blocks)."""
    cfg = W.CONFIGS["v3_prefill_fp8"].with_(T=T, d=d, I=I, Nr=Nr, Ns=Ns, K=3)
    idx = make_idx(T, cfg.Nr, cfg.K, T + d + 1, hot=[2, Nr - 1])
    err = run_fp8_case(cfg, idx, tile_m=tile_m, y_dtype=ydt)
    assert err < 1e-2, err     # well inside the bound: both sides use the same codes


def test_fp8_rejects_unsupported_shapes():
    cfg = W.CONFIGS["v3_prefill_fp8"].with_(T=32, d=384, I=256, Nr=4, Ns=1, K=2)
    idx = make_idx(cfg.T, cfg.Nr, cfg.K, 5)
    with pytest.raises(M.MoeError, match="fp8 path needs"):
        run_fp8_case(cfg, idx)


# ------------------------------------------------ bf16 x E4M3 (decode path) --
def run_w8_case(cfg, idx, tile_m=32, y_dtype=torch.bfloat16, tol=1e-2):
    """GPU: bf16 rows, weights quantised by fp8_quantize_tiles (128x128
    blocks), h kept in bf16.  Oracle: the same weights through its own
    quantiser, decoded, fp64 products."""
    u = W.make_tokens(cfg, 0, "cuda")
    w13, w2 = W.make_expert_weights(cfg, "cuda")
    weights = M.quantize_weights(w13, w2)
    lay = O.permute_layout(idx.numpy(), cfg.Nr, cfg.Ns, tile_m, M.MOE_TILE_ROWS)
    y = gpu_expert_rows(cfg, u, None, weights, lay, tile_m, y_dtype)
    w13q, w2q = oracle_fp8_weights(w13, w2)
    want = O.expert_rows(f64_of(u), w13q, w2q, lay, cfg.Nr, cfg.Ns)
    real = lay.row_token[: lay.seg_offset[-1]] >= 0
    got = y[: lay.seg_offset[-1]][real]
    assert np.all(np.isfinite(got))
    err = rel_l2(got, want[real])
    assert err <= tol, err
    for s in range(cfg.E):
        r0, r1 = lay.seg_offset[s], lay.seg_offset[s + 1]
        m = lay.row_token[r0:r1] >= 0
        if m.any():
            assert rel_l2(y[r0:r1][m], want[r0:r1][m]) <= 2 * tol, s
    return err


@pytest.mark.parametrize("T,d,I,Nr,Ns,tile_m,ydt", [(128, 512, 256, 16, 1, 32, torch.bfloat16),
                                                    (128, 512, 512, 16, 1, 16, torch.float32),
                                                    (300, 256, 256, 12, 2, 1, torch.bfloat16),
                                                    (600, 768, 256, 12, 1, 256, torch.bfloat16),
                                                    (50, 2048, 1024, 24, 1, 32, torch.bfloat16),
                                                    (20, 8192, 256, 4, 1, 64, torch.bfloat16)])
def test_w8a16_decode_kernel_shapes(T, d, I, Nr, Ns, tile_m, ydt):
    """bf16 activations x E4M3 weights: segments of 1 to several hundred rows
    (16- and 32-row passes, several passes per tile), shared segments, both
    output types, and d = 8192 (64 scale blocks along K)."""
    cfg = W.CONFIGS["v3_decode_fp8w"].with_(T=T, d=d, I=I, Nr=Nr, Ns=Ns, K=3)
    idx = make_idx(T, cfg.Nr, cfg.K, T + d + 2, hot=[1, Nr - 2])
    err = run_w8_case(cfg, idx, tile_m=tile_m, y_dtype=ydt)
    assert err < 5e-3, err


def test_w8a16_rejects_unsupported_shapes():
    cfg = W.CONFIGS["v3_decode_fp8w"].with_(T=16, d=384, I=256, Nr=4, Ns=1, K=2)
    with pytest.raises(M.MoeError, match="bf16 x E4M3 path needs"):
        run_w8_case(cfg, make_idx(cfg.T, cfg.Nr, cfg.K, 6))
