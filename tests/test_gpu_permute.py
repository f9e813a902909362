"""GPU parity of moe_permute against the oracle's layout definition: every
output (segment offsets, row tokens including padding, inverse rows, tile
map, tile count) must be bit-identical."""
import numpy as np
import pytest
import torch

import sparse_expert_routing_sigmoid_amd as M
import workloads as W
from moe_testutil import np_of
from oracle import moe as O

pytestmark = pytest.mark.gpu


def make_idx(T, Nr, K, seed, hot=None):
    """Distinct experts per token from a seeded random ranking; `hot` experts
    are pushed to the front so their segments get long."""
    r = W.make_free((T, Nr), 1.0, seed, "cpu")
    if hot is not None:
        for n, h in enumerate(hot):          # earlier hot experts rank higher
            r[:, h] += 10.0 * (len(hot) - n)
    return torch.argsort(r, dim=1, descending=True, stable=True)[:, :K].to(torch.int32).contiguous()


def gpu_permute(idx, Nr, Ns, tile_m):
    T, K = idx.shape
    P = M.moe_permute_rows(T, K, Nr, Ns, tile_m)
    tiles = M.moe_permute_tiles_max(T, K, Nr, Ns, tile_m)
    dev = dict(dtype=torch.int32, device="cuda")
    seg = torch.full((Nr + Ns + 1,), -9, **dev)
    row_token = torch.full((P,), -9, **dev)
    inv_row = torch.full((T, K), -9, **dev)
    tile_map = torch.full((tiles, 4), -9, **dev)
    n_tiles = torch.full((1,), -9, **dev)
    ws = torch.empty((M.moe_permute_workspace_bytes(T, K, Nr, Ns),), dtype=torch.uint8, device="cuda")
    M.moe_permute(idx.cuda(), Nr, Ns, tile_m, seg, row_token, inv_row, tile_map, n_tiles, ws)
    torch.cuda.synchronize()
    return np_of(seg), np_of(row_token), np_of(inv_row), np_of(tile_map), int(n_tiles.item())


def check(idx, Nr, Ns, tile_m):
    lay = O.permute_layout(idx.numpy(), Nr, Ns, tile_m, M.MOE_TILE_ROWS)
    seg, row_token, inv_row, tile_map, n = gpu_permute(idx, Nr, Ns, tile_m)
    assert np.array_equal(seg, lay.seg_offset)
    assert np.array_equal(row_token, lay.row_token)
    assert np.array_equal(inv_row, lay.inv_row)
    assert n == lay.n_tiles
    assert np.array_equal(tile_map[:n], lay.tile_map)


@pytest.mark.parametrize("T", [1, 255, 256, 257, 3000])
@pytest.mark.parametrize("tile_m", [1, 16, 32, 256])
def test_permute_matches_layout(T, tile_m):
    check(make_idx(T, 64, 6, T + tile_m), 64, 2, tile_m)


@pytest.mark.parametrize("Nr,Ns,K", [(16, 0, 4), (16, 1, 16), (256, 1, 8), (1000, 3, 8), (1021, 3, 2)])
def test_permute_expert_counts(Nr, Ns, K):
    check(make_idx(777, Nr, K, Nr + K), Nr, Ns, 32)


def test_permute_one_expert_takes_every_token():
    idx = make_idx(1500, 32, 4, 5, hot=[7, 3])
    assert np.all(idx[:, 0].numpy() == 7)
    check(idx, 32, 1, 16)


def test_permute_zero_tokens():
    idx = torch.zeros((0, 4), dtype=torch.int32)
    seg, row_token, _, _, n = gpu_permute(idx, 16, 1, 32)
    assert n == 0 and np.all(seg == 0) and np.all(row_token == -1)


def test_permute_v3_shape_zipf_routing_deterministic():
    cfg = W.CONFIGS["v3_prefill_bf16"]
    idx = make_idx(cfg.T, cfg.Nr, cfg.K, 11, hot=list(range(0, 256, 37)))
    check(idx, cfg.Nr, cfg.Ns, 32)
    a = gpu_permute(idx, cfg.Nr, cfg.Ns, 32)
    b = gpu_permute(idx, cfg.Nr, cfg.Ns, 32)
    for x, y in zip(a[:4], b[:4]):
        assert np.array_equal(x, y)
