"""moe_permute_noalloc (no workspace argument: the library's own scratch
array) against moe_permute with a caller workspace, through the C ABI: the
same layout bit for bit on two calls in a row, the second with a smaller
input, and sizes beyond the scratch array rejected on the host."""
import ctypes

import numpy as np
import pytest
import torch

import sparse_expert_routing_sigmoid_amd as M

pytestmark = pytest.mark.gpu


def topk_indices(T, Nr, K, skew, seed):
    """K distinct experts per token, drawn with weights rank^-skew."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    w = torch.arange(1, Nr + 1, device="cuda", dtype=torch.float32) ** (-skew)
    w = w[torch.randperm(Nr, device="cuda", generator=g)]
    return torch.multinomial(w.expand(T, Nr).contiguous(), K, replacement=False, generator=g).to(torch.int32).contiguous()


def layout(idx, Nr, Ns, tile_m, noalloc):
    T, K = idx.shape
    P = M.moe_permute_rows(T, K, Nr, Ns, tile_m)
    tiles = M.moe_permute_tiles_max(T, K, Nr, Ns, tile_m)
    i32 = dict(dtype=torch.int32, device="cuda")
    out = dict(seg_offset=torch.full((Nr + Ns + 1,), -7, **i32), row_token=torch.full((P,), -7, **i32),
               inv_row=torch.full((T, K), -7, **i32), tile_map=torch.full((tiles, 4), -7, **i32),
               n_tiles=torch.full((1,), -7, **i32))
    if noalloc:
        M.moe_permute_noalloc(idx, Nr, Ns, tile_m, out["seg_offset"], out["row_token"], out["inv_row"],
                              out["tile_map"], out["n_tiles"])
    else:
        ws = torch.empty((M.moe_permute_workspace_bytes(T, K, Nr, Ns),), dtype=torch.uint8, device="cuda")
        M.moe_permute(idx, Nr, Ns, tile_m, out["seg_offset"], out["row_token"], out["inv_row"], out["tile_map"],
                      out["n_tiles"], ws)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


CASES = [  # (T, Nr, Ns, K, tile_m, skew): the second smaller than the first
    (8192, 256, 1, 8, 32, 1.1),
    (300, 64, 2, 6, 16, 0.0),
]


def test_noalloc_permute_equals_permute_on_two_calls():
    for n, (T, Nr, Ns, K, tile_m, skew) in enumerate(CASES):
        print(f"noalloc permute call {n}: T={T} Nr={Nr} Ns={Ns} K={K} tile_m={tile_m}", flush=True)
        idx = topk_indices(T, Nr, K, skew, 40 + n)
        got = layout(idx, Nr, Ns, tile_m, noalloc=True)
        want = layout(idx, Nr, Ns, tile_m, noalloc=False)
        for k in want:
            assert np.array_equal(got[k], want[k]), (n, k)
        assert got["n_tiles"][0] > 0 and got["seg_offset"][-1] >= T * (K + Ns)


def test_noalloc_permute_rejects_sizes_beyond_its_scratch():
    L = M.lib()
    cap = L.moe_permute_noalloc_scratch_bytes()
    assert cap == 4 << 20
    T, K, Nr, Ns = 1 << 21, 8, 1024, 1
    assert M.moe_permute_workspace_bytes(T, K, Nr, Ns) > cap
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: the call fails on the host
    st = L.moe_permute_noalloc(fake, T, K, Nr, Ns, 32, fake, fake, fake, fake, fake, None)
    assert st == M.MOE_EWORKSPACE
    assert b"4 MiB" in L.moe_last_error()
