"""GPU parity of moe_combine (against the oracle's combine equation) and of
moe_bias_update (bit-exact against the oracle's bias rule)."""
import numpy as np
import pytest
import torch

import sparse_expert_routing_sigmoid_amd as M
import workloads as W
from moe_testutil import f64_of, np_of, rel_l2
from oracle import moe as O
from test_gpu_permute import make_idx

pytestmark = pytest.mark.gpu


def _setup(T, d, Nr, Ns, K, ydt, seed):
    idx = make_idx(T, Nr, K, seed)
    lay = O.permute_layout(idx.numpy(), Nr, Ns, 16, M.MOE_TILE_ROWS)
    P = len(lay.row_token)
    y = W.make_free((P, d), 0.3, seed + 1, "cpu", ydt)
    gate = torch.rand((T, K), generator=W.generator(99, 7, seed + 2, "cpu"))
    gate = gate / gate.sum(1, keepdim=True)
    return idx, lay, y, gate


@pytest.mark.parametrize("udt,ydt,odt", [(torch.float32, torch.float32, torch.float32),
                                          (torch.bfloat16, torch.bfloat16, torch.bfloat16),
                                          (torch.bfloat16, torch.bfloat16, torch.float32),
                                          (torch.bfloat16, torch.float32, torch.bfloat16)])
@pytest.mark.parametrize("flags", [0, M.MOE_COMBINE_NO_RESIDUAL, M.MOE_COMBINE_NO_SHARED | M.MOE_COMBINE_NO_ROUTED,
                                   M.MOE_COMBINE_NO_RESIDUAL | M.MOE_COMBINE_NO_SHARED])
def test_combine(udt, ydt, odt, flags):
    T, d, Nr, Ns, K = 300, 2056, 24, 2, 5
    idx, lay, y, gate = _setup(T, d, Nr, Ns, K, ydt, 40)
    u = W.make_free((T, d), 1.0, 41, "cpu", udt)
    out = torch.empty((T, d), dtype=odt, device="cuda")
    M.moe_combine(u.cuda(), y.cuda(), torch.from_numpy(lay.inv_row).cuda(), gate.cuda(),
                  torch.from_numpy(lay.seg_offset).cuda(), Nr, Ns, out, flags)
    torch.cuda.synchronize()
    yf = f64_of(y)
    y_routed = yf[lay.inv_row]                                    # [T, K, d]
    y_shared = np.stack([yf[lay.seg_offset[Nr + j]: lay.seg_offset[Nr + j] + T] for j in range(Ns)])
    want = O.combine(f64_of(u), y_shared, y_routed, f64_of(gate),
                     residual=not flags & 1, shared=not flags & 2, routed=not flags & 4)
    got = f64_of(out)
    tol = 1e-6 if odt == torch.float32 else 4e-3
    assert rel_l2(got, want) <= tol
    if odt == torch.float32:
        np.testing.assert_allclose(got, want, rtol=1e-5, atol=1e-5)


def test_combine_deterministic():
    T, d, Nr, Ns, K = 64, 7168, 256, 1, 8
    idx, lay, y, gate = _setup(T, d, Nr, Ns, K, torch.bfloat16, 50)
    u = W.make_free((T, d), 1.0, 51, "cuda", torch.bfloat16)
    args = (u, y.cuda(), torch.from_numpy(lay.inv_row).cuda(), gate.cuda(), torch.from_numpy(lay.seg_offset).cuda(),
            Nr, Ns)
    o1 = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    o2 = torch.empty_like(o1)
    M.moe_combine(*args, o1)
    M.moe_combine(*args, o2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


@pytest.mark.parametrize("Nr,T,K", [(16, 64, 4), (256, 8192, 8), (6, 3, 2), (1000, 1000, 7), (64, 4096, 6)])
def test_bias_update_bit_exact(Nr, T, K):
    g = W.generator(99, 7, Nr, "cpu")
    load = torch.multinomial(torch.ones(Nr), T * K, replacement=True, generator=g).bincount(minlength=Nr)
    if (T * K) % Nr == 0:
        load[0] = T * K // Nr                              # a load exactly at the mean: unchanged
    b = (torch.rand(Nr, generator=g) - 0.5) * 0.02
    bias = b.clone().cuda()
    M.moe_bias_update(load.to(torch.int32).cuda(), T * K, 0.001, bias)
    torch.cuda.synchronize()
    want = O.bias_update(b.numpy(), load.numpy(), T, K)
    assert np.array_equal(np_of(bias).view(np.uint32), want.view(np.uint32))
