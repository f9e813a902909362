"""Degenerate and boundary cases of the whole layer on the GPU, against the
oracle: no tokens, a single token on every GEMM path, every expert selected
(K = N_r), a single routed expert, zero weights (h' = u), and E4M3 tiles of
zeros or at the format's extremes."""
import numpy as np
import pytest
import torch

import sparse_expert_routing_sigmoid_amd as M
import workloads as W
from moe_testutil import check_routing, f64_of, np_of, rel_l2
from oracle import e4m3 as OE
from oracle import moe as O

pytestmark = pytest.mark.gpu


def oracle_weights(w13, w2, fp8):
    if not fp8:
        return f64_of(w13), f64_of(w2)
    deq = lambda m: OE.dequantize_tiles(*OE.quantize_tiles(m, 128, 128), 128, 128)
    a13, a2 = np_of(w13).astype(np.float32), np_of(w2).astype(np.float32)
    return (np.stack([deq(a13[e]) for e in range(a13.shape[0])]),
            np.stack([deq(a2[e]) for e in range(a2.shape[0])]))


def run_layer(cfg, tol, zero_weights=False):
    """One forward + bias rule of cfg on the GPU and in the oracle."""
    w13, w2 = W.make_expert_weights(cfg, "cuda")
    if zero_weights:
        w13.zero_()
        w2.zero_()
    fp8w = cfg.weights == "e4m3"
    weights = M.quantize_weights(w13, w2) if fp8w else M.ExpertWeights(
        M.MOE_F32 if cfg.weights == "f32" else M.MOE_BF16, w13, w2)
    layer = M.MoeLayer(cfg.T, cfg.d, cfg.Nr, cfg.Ns, cfg.I, cfg.K, W.TORCH_DTYPE[cfg.act], weights,
                       x_fp8=cfg.x_fp8, tile_m=32)
    u = W.make_tokens(cfg, 0, "cuda")
    e = W.make_centroids(cfg, "cuda")
    b = W.make_bias(cfg, "cuda")
    out = layer.forward(u, e, b)
    bias = b.clone()
    layer.update_bias(bias, cfg.gamma)
    torch.cuda.synchronize()
    w13o, w2o = oracle_weights(w13, w2, fp8w)
    o = O.layer_forward(f64_of(u), f64_of(e), f64_of(b), w13o, w2o, cfg.Nr, cfg.Ns, cfg.K,
                        x_quant=cfg.x_fp8, h_quant=cfg.x_fp8, gamma=cfg.gamma)
    if cfg.T == 0:
        assert out.shape[0] == 0
        assert np.array_equal(np_of(layer.expert_load), np.zeros(cfg.Nr, np.int32))
        return o, out
    ok, tied = check_routing(np_of(layer.topk_idx), np_of(layer.topk_gate), np_of(layer.expert_load),
                             o.routing, cfg.Nr)
    got = f64_of(out)
    assert np.all(np.isfinite(got))
    if zero_weights:
        assert np.array_equal(got[ok], f64_of(u)[ok])      # FFN terms are exactly 0: h' = u
    else:
        assert rel_l2(got[ok], o.out[ok]) <= tol
        assert rel_l2(got[ok] - f64_of(u)[ok], (o.out - f64_of(u))[ok]) <= tol
    if not tied:
        assert np.array_equal(np_of(bias).view(np.uint32), o.new_bias.view(np.uint32))
    return o, out


SMALL = dict(d=512, Nr=16, Ns=1, I=256, K=4)
PATHS = [("tiny_fp32", 1e-5), ("mid_bf16", 1e-2), ("v3_decode_fp8w", 1e-2), ("v3_prefill_fp8", 3e-2)]


@pytest.mark.parametrize("name,tol", PATHS)
def test_no_tokens(name, tol):
    run_layer(W.CONFIGS[name].with_(T=0, **SMALL), tol)


@pytest.mark.parametrize("name,tol", PATHS)
def test_single_token(name, tol):
    run_layer(W.CONFIGS[name].with_(T=1, **SMALL), tol)


@pytest.mark.parametrize("name,tol", PATHS)
def test_every_expert_selected(name, tol):
    """K = N_r: every token goes to every routed expert; gates are s / sum s."""
    cfg = W.CONFIGS[name].with_(T=96, **dict(SMALL, Nr=8, K=8))
    o, _ = run_layer(cfg, tol)
    assert np.all(o.routing.load == cfg.T)


@pytest.mark.parametrize("name,tol", PATHS)
def test_single_routed_expert(name, tol):
    """N_r = K = 1: every gate is 1 and one segment holds every token."""
    run_layer(W.CONFIGS[name].with_(T=300, **dict(SMALL, Nr=1, K=1)), tol)


@pytest.mark.parametrize("name,tol", PATHS)
def test_zero_weights_give_the_residual(name, tol):
    run_layer(W.CONFIGS[name].with_(T=200, **SMALL), tol, zero_weights=True)


def test_fp8_tiles_of_zeros_and_extremes():
    """1x128 tiles that are all zero (scale 1), hold the largest and smallest
    normal E4M3 magnitudes times a power of two, or a single non-zero value:
    GPU codes and scales equal the oracle's bit for bit."""
    rows, cols = 6, 256
    x = np.zeros((rows, cols), np.float32)
    x[1, :128] = 448.0 * 2.0 ** -20                           # amax exactly 448 * 2^k
    x[1, 128:] = np.linspace(-3e-3, 3e-3, 128, dtype=np.float32)
    x[2, 5] = -7.0                                            # a lone value
    x[3, :] = 2.0 ** -6 * 2.0 ** 10                           # all equal
    x[4, ::2] = 1e-37                                         # tiny values: the k >= -126 floor
    x[5, :] = np.float32(2.0 ** 120)                          # huge values
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    s = torch.empty((rows, cols // 128), dtype=torch.float32, device="cuda")
    M.fp8_quantize_tiles(torch.from_numpy(x).cuda(), 1, q, s)
    torch.cuda.synchronize()
    codes, scales = OE.quantize_tiles(x, 1, 128)
    assert np.array_equal(np_of(q), codes)
    assert np.array_equal(np_of(s).view(np.uint32), scales.view(np.uint32))
    assert np_of(s)[0].tolist() == [1.0, 1.0]                 # all-zero tiles


def test_misaligned_data_tensors_are_rejected():
    """Data tensors are accessed 16 bytes at a time: a view two bytes off is
    refused on the host with MOE_EINVAL, before anything is launched."""
    cfg = W.CONFIGS["mid_bf16"].with_(T=64, **SMALL)
    w13, w2 = W.make_expert_weights(cfg, "cuda")
    layer = M.MoeLayer(cfg.T, cfg.d, cfg.Nr, cfg.Ns, cfg.I, cfg.K, torch.bfloat16,
                       M.ExpertWeights(M.MOE_BF16, w13, w2), tile_m=32)
    u = W.make_tokens(cfg, 0, "cuda")
    e = W.make_centroids(cfg, "cuda")
    b = W.make_bias(cfg, "cuda")
    base = torch.empty(u.numel() + 8, dtype=u.dtype, device="cuda")
    u_off = base[1:1 + u.numel()].view(u.shape)
    u_off.copy_(u)
    assert u_off.data_ptr() % 16 == 2
    with pytest.raises(M.MoeError) as err:
        layer.route(u_off, e, b)
    assert err.value.status == M.MOE_EINVAL
    layer.route(u, e, b)
    layer.permute()
    with pytest.raises(M.MoeError) as err:
        layer.experts(u_off)
    assert err.value.status == M.MOE_EINVAL
    layer.experts(u)
    with pytest.raises(M.MoeError) as err:
        layer.combine(u_off)
    assert err.value.status == M.MOE_EINVAL
    q = torch.empty((cfg.T, cfg.d), dtype=torch.uint8, device="cuda")
    s = torch.empty((cfg.T, cfg.d // 128), dtype=torch.float32, device="cuda")
    with pytest.raises(M.MoeError) as err:
        M.fp8_quantize_tiles(u_off, 1, q, s)
    assert err.value.status == M.MOE_EINVAL
    out = layer.combine(u)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
