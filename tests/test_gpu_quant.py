"""GPU parity of fp8_quantize_tiles against the oracle's quantiser: codes and
scales must be bit-identical (the scale rule and the rounding are specified
in IEEE fp32 on both sides)."""
import numpy as np
import pytest
import torch

import sparse_expert_routing_sigmoid_amd as M
import workloads as W
from moe_testutil import np_of
from oracle import e4m3

pytestmark = pytest.mark.gpu


def _gpu_quant(x, tile_rows):
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    s = torch.empty((rows // tile_rows, cols // 128), dtype=torch.float32, device="cuda")
    M.fp8_quantize_tiles(x, tile_rows, q, s)
    torch.cuda.synchronize()
    return np_of(q), np_of(s)


def _special_rows(cols):
    """Rows whose tiles hold 448 (scale exactly 1) plus every midpoint between
    neighbouring E4M3 values and the values one fp32 ulp either side of it."""
    pos = e4m3.DECODE_TABLE[:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(-np.inf))
    vals = np.concatenate([mids, up, dn, pos.astype(np.float32), -mids, -up, -dn])
    n_per_tile = 127
    tiles = []
    for i in range(0, len(vals), n_per_tile):
        t = np.zeros(128, np.float32)
        chunk = vals[i:i + n_per_tile]
        t[:len(chunk)] = chunk
        t[127] = 448.0
        tiles.append(t)
    flat = np.concatenate(tiles)
    pad = (-len(flat)) % cols
    flat = np.concatenate([flat, np.tile(np.r_[np.zeros(127, np.float32), np.float32(448.0)], pad // 128)])
    return flat.reshape(-1, cols)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("tile_rows", [1, 128])
def test_quantize_bit_exact(dtype, tile_rows):
    rows, cols = 256, 640
    x = W.make_free((rows, cols), 1.0, 1 + tile_rows, "cpu")
    x *= torch.logspace(-6, 3, rows)[:, None]            # tiles spanning many scales
    x[3, :128] = 0.0                                     # an all-zero 1x128 tile
    x[:128, 512:] = 0.0                                  # an all-zero 128x128 block
    x[7] *= 1e-30                                        # tiny values (fp32 subnormal range)
    x = x.to(dtype)
    q, s = _gpu_quant(x.cuda(), tile_rows)
    qo, so = e4m3.quantize_tiles(x.to(torch.float32).numpy(), tile_rows, 128)
    assert np.array_equal(s.view(np.uint32), so.view(np.uint32))
    assert np.array_equal(q, qo)


def test_rounding_at_every_midpoint():
    x = torch.from_numpy(_special_rows(1024))
    q, s = _gpu_quant(x.cuda(), 1)
    qo, so = e4m3.quantize_tiles(x.numpy(), 1, 128)
    assert np.all(so == 1.0)
    assert np.array_equal(s, so)
    assert np.array_equal(q, qo)


def test_dense_sweep_with_unit_scale():
    """Every 64th fp32 pattern in [0, 448] (plus signs), scale forced to 1."""
    pos = np.arange(0, 0x43E00000 + 1, 64, dtype=np.uint32).view(np.float32)
    vals = np.concatenate([pos, -pos])
    vals = vals[: len(vals) // (127 * 8) * (127 * 8)].reshape(-1, 127)
    x = np.concatenate([vals, np.full((vals.shape[0], 1), 448.0, np.float32)], axis=1).reshape(-1, 1024)
    q, _ = _gpu_quant(torch.from_numpy(x).cuda(), 1)
    qo, _ = e4m3.quantize_tiles(x, 1, 128)
    assert np.array_equal(q, qo)


def test_weight_blocks_of_an_expert_tensor():
    cfg = W.CONFIGS["v3_decode_fp8w"].with_(Nr=2, Ns=1, d=256, I=128)
    w13, w2 = W.make_expert_weights(cfg, "cuda")
    ew = M.quantize_weights(w13, w2)
    torch.cuda.synchronize()
    for e in range(cfg.E):
        qo, so = e4m3.quantize_tiles(w13[e].cpu().numpy(), 128, 128)
        assert np.array_equal(np_of(ew.w13[e]), qo) and np.array_equal(np_of(ew.w13_scale[e]), so)
        qo, so = e4m3.quantize_tiles(w2[e].cpu().numpy(), 128, 128)
        assert np.array_equal(np_of(ew.w2[e]), qo) and np.array_equal(np_of(ew.w2_scale[e]), so)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("tile_rows", [1, 128])
def test_dequantize_is_code_times_scale(out_dtype, tile_rows):
    """fp8_dequantize_tiles: each of the 254 finite codes, under scales
    from 2^-100 to 2^40, gives exactly the oracle's decoded value (exact in
    bf16 for these scales)."""
    rows, cols = 256, 640
    rng = np.random.default_rng(30 + tile_rows)
    codes = rng.integers(0, 256, size=(rows, cols), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x7E                 # no NaN patterns
    finite = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    codes[0, :finite.size] = finite                      # every finite code once
    nsc = (rows // tile_rows, cols // 128)
    scales = np.exp2(rng.integers(-100, 41, size=nsc)).astype(np.float32)
    q, s = torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda()
    out = torch.empty((rows, cols), dtype=out_dtype, device="cuda")
    M.fp8_dequantize_tiles(q, s, tile_rows, out)
    torch.cuda.synchronize()
    want = e4m3.dequantize_tiles(codes, scales, tile_rows, 128)
    assert np.array_equal(out.to("cpu", torch.float64).numpy(), want)


def test_dequantize_round_trip_of_activations():
    """Quantise then dequantise on the GPU: the oracle's quantised u."""
    from oracle import moe as O
    x = W.make_free((64, 1024), 1.0, 33, "cuda", torch.bfloat16)
    q = torch.empty((64, 1024), dtype=torch.uint8, device="cuda")
    s = torch.empty((64, 8), dtype=torch.float32, device="cuda")
    out = torch.empty((64, 1024), dtype=torch.bfloat16, device="cuda")
    M.fp8_quantize_tiles(x, 1, q, s)
    M.fp8_dequantize_tiles(q, s, 1, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.to("cpu", torch.float64).numpy(), O.quantize_activations(x.to("cpu", torch.float64).numpy()))
