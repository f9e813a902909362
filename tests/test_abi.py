"""CPU checks of the C-ABI library: it loads, exports every symbol the public
header declares, and rejects bad arguments on the host, before any launch,
with the documented status codes.  No call here reaches a kernel."""
import ctypes
import os
import re

import pytest

import sparse_expert_routing_sigmoid_amd as M
from oracle import moe as omoe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mi355x.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?(?:(?:unsigned|signed|long)\s+)*[A-Za-z_][A-Za-z0-9_]*(?:\s+|\s*\*+\s*)"
                       r"([a-z0-9_]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    L = M.lib()
    names = _declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(M.SIGNATURES)


def test_abi_version_and_status_strings():
    L = M.lib()
    assert L.moe_abi_version() == 5
    assert L.moe_status_str(0) == b"MOE_OK"
    assert L.moe_status_str(3) == b"MOE_EWORKSPACE"


@pytest.mark.parametrize("T,K,Nr,Ns,tile_m", [(64, 4, 16, 1, 32), (8192, 8, 256, 1, 32), (5, 3, 9, 2, 1),
                                             (0, 2, 4, 1, 16), (128, 8, 256, 1, 16)])
def test_row_bound_matches_oracle(T, K, Nr, Ns, tile_m):
    assert M.moe_permute_rows(T, K, Nr, Ns, tile_m) == omoe.permuted_rows_max(T, K, Nr, Ns, tile_m)
    tiles = M.moe_permute_tiles_max(T, K, Nr, Ns, tile_m)
    assert tiles >= M.moe_permute_rows(T, K, Nr, Ns, tile_m) // M.MOE_TILE_ROWS + 1


def _status(fn, *args):
    st = fn(*args)
    return st, M.lib().moe_last_error().decode()


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every case fails on the host


def test_route_rejects_bad_arguments():
    L = M.lib()
    ws = 1 << 30
    good = dict(u=FAKE, ut=M.MOE_BF16, e=FAKE, b=FAKE, T=4, d=64, Nr=16, K=4, idx=FAKE, gate=FAKE, score=None,
                load=FAKE, ws=FAKE, wsb=ws, st=None)

    def call(**kw):
        a = dict(good, **kw)
        return _status(L.moe_route, a["u"], a["ut"], a["e"], a["b"], a["T"], a["d"], a["Nr"], a["K"], a["idx"],
                       a["gate"], a["score"], a["load"], a["ws"], a["wsb"], a["st"])

    assert call(u=None)[0] == M.MOE_EINVAL
    assert call(load=None)[0] == M.MOE_EINVAL
    assert call(K=0)[0] == M.MOE_EINVAL
    assert call(K=17, Nr=32)[0] == M.MOE_EINVAL
    assert call(K=5, Nr=4)[0] == M.MOE_EINVAL
    assert call(Nr=1025)[0] == M.MOE_EINVAL
    assert call(d=60)[0] == M.MOE_EINVAL
    assert call(ut=M.MOE_E4M3)[0] == M.MOE_EINVAL
    st, msg = call(wsb=16)
    assert st == M.MOE_EWORKSPACE and "workspace" in msg


def test_permute_rejects_bad_arguments():
    L = M.lib()
    args = [FAKE, 8, 2, 4, 1, 32, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None]

    def call(i, v):
        a = list(args)
        a[i] = v
        return L.moe_permute(*a)

    assert call(5, 3) == M.MOE_EINVAL        # tile_m not a power of two
    assert call(5, 512) == M.MOE_EINVAL      # tile_m above MOE_TILE_ROWS
    assert call(2, 5) == M.MOE_EINVAL        # K > Nr
    assert call(0, None) == M.MOE_EINVAL     # NULL topk_idx
    assert call(12, 4) == M.MOE_EWORKSPACE


def test_gemm_rejects_bad_arguments():
    L = M.lib()
    base = [FAKE, M.MOE_BF16, None, M.MOE_BF16, FAKE, None, FAKE, None, 64, 4, 16, 1, 256, 128, 32,
            FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, FAKE, M.MOE_BF16, None]

    def call(**kw):
        a = list(base)
        pos = dict(x_t=1, x_scale=2, w_t=3, w13_scale=5, d=12, I=13, ws_bytes=20, y_t=22, x=0)
        for k, v in kw.items():
            a[pos[k]] = v
        return L.moe_expert_gemm(*a)

    assert call(x=None) == M.MOE_EINVAL
    assert call(x_t=M.MOE_F32) == M.MOE_EUNSUPPORTED                     # f32 x with bf16 weights
    assert call(w_t=M.MOE_E4M3) == M.MOE_EINVAL                          # fp8 weights without scales
    assert call(x_t=M.MOE_E4M3, w_t=M.MOE_E4M3, w13_scale=FAKE) == M.MOE_EINVAL  # no x_scale / w2_scale
    assert call(ws_bytes=10) == M.MOE_EWORKSPACE
    assert call(d=200) == M.MOE_EUNSUPPORTED                             # MFMA path needs d % 128 == 0
    assert call(y_t=M.MOE_E4M3) == M.MOE_EINVAL


def test_combine_bias_quant_reject_bad_arguments():
    L = M.lib()
    assert L.moe_combine(FAKE, M.MOE_BF16, FAKE, M.MOE_BF16, FAKE, FAKE, FAKE, 4, 100, 2, 8, 1, 0, FAKE,
                         M.MOE_BF16, None) == M.MOE_EINVAL            # d % 8 != 0
    assert L.moe_combine(FAKE, M.MOE_BF16, FAKE, M.MOE_BF16, FAKE, FAKE, FAKE, 4, 64, 2, 8, 1, 8, FAKE,
                         M.MOE_BF16, None) == M.MOE_EINVAL            # unknown flag
    assert L.moe_combine(FAKE, M.MOE_BF16, FAKE, M.MOE_BF16, FAKE, FAKE, FAKE, 4, 64, 2, 8, 1, 0, FAKE,
                         M.MOE_BF16, None) == M.MOE_EINVAL            # out aliases y
    assert L.moe_bias_update(None, 4, 8, 0.001, FAKE, None) == M.MOE_EINVAL
    assert L.moe_bias_update(FAKE, 4, -1, 0.001, FAKE, None) == M.MOE_EINVAL
    assert L.moe_bias_update(FAKE, 4, 8, float("nan"), FAKE, None) == M.MOE_EINVAL
    assert L.fp8_quantize_tiles(FAKE, M.MOE_BF16, 4, 100, 1, 128, FAKE, FAKE, None) == M.MOE_EINVAL
    assert L.fp8_quantize_tiles(FAKE, M.MOE_BF16, 100, 128, 128, 128, FAKE, FAKE, None) == M.MOE_EINVAL
    assert L.fp8_quantize_tiles(FAKE, M.MOE_BF16, 4, 128, 2, 128, FAKE, FAKE, None) == M.MOE_EINVAL
    assert L.fp8_quantize_tiles(FAKE, M.MOE_E4M3, 4, 128, 1, 128, FAKE, FAKE, None) == M.MOE_EINVAL
    assert L.fp8_dequantize_tiles(FAKE, FAKE, 4, 100, 1, 128, FAKE, M.MOE_BF16, None) == M.MOE_EINVAL
    assert L.fp8_dequantize_tiles(FAKE, FAKE, 100, 128, 128, 128, FAKE, M.MOE_BF16, None) == M.MOE_EINVAL
    assert L.fp8_dequantize_tiles(FAKE, FAKE, 4, 128, 1, 128, FAKE, M.MOE_E4M3, None) == M.MOE_EINVAL
    assert L.fp8_dequantize_tiles(None, FAKE, 4, 128, 1, 128, FAKE, M.MOE_F32, None) == M.MOE_EINVAL


def test_fused_combine_rejects_bad_arguments():
    L = M.lib()
    fake, fake_out = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000)   # never dereferenced
    T, K, Nr, Ns, d, I = 512, 4, 16, 1, 512, 256

    def call(x_t=M.MOE_BF16, w_t=M.MOE_BF16, flags=0, out=fake_out, u_t=M.MOE_BF16, d=d):
        return L.moe_expert_gemm_combine(fake, x_t, None, w_t, fake, None, fake, None, T, K, Nr, Ns, d, I, 32,
                                         fake, fake, fake, fake, fake, fake, fake, u_t, flags, fake, 1 << 40, out,
                                         None)
    assert call(x_t=M.MOE_F32, w_t=M.MOE_F32) == M.MOE_EUNSUPPORTED      # only the persistent MFMA paths
    assert call(x_t=M.MOE_BF16, w_t=M.MOE_E4M3) == M.MOE_EUNSUPPORTED    # nor the decode path
    assert call(flags=8) == M.MOE_EINVAL
    assert call(out=fake) == M.MOE_EINVAL                                 # out aliases u
    assert call(u_t=M.MOE_E4M3) == M.MOE_EINVAL
    assert call(d=520) == M.MOE_EUNSUPPORTED                               # bf16 persistent needs d % 256 == 0
    assert b"persistent" in L.moe_last_error() or b"256" in L.moe_last_error()


def test_python_binding_raises_with_message():
    import torch
    with pytest.raises(M.MoeError, match="MOE_EINVAL"):
        M._check(M.lib().moe_bias_update(None, 4, 8, 0.001, FAKE, None))


def test_backward_entry_points_reject_bad_arguments():
    L = M.lib()
    F = FAKE
    T, K, Nr, Ns, d, I, tm = 64, 4, 16, 1, 512, 256, 32
    big = 1 << 34
    gb = lambda **kw: _status(L.moe_expert_gemm_backward, *[kw.get(k, v) for k, v in dict(
        x=F, w13=F, w2=F, h=F, ab=F, dy=F, T=T, K=K, Nr=Nr, Ns=Ns, d=d, I=I, tm=tm, so=F, rt=F, tmap=F, nt=F,
        ws=F, wsb=big, dx=F, dw13=F, dw2=F, dwt=M.MOE_F32, st=None).items()])
    assert gb(I=192)[0] == M.MOE_EUNSUPPORTED           # I % 128 != 0
    assert gb(d=384)[0] == M.MOE_EUNSUPPORTED           # d % 256 != 0
    assert gb(dwt=M.MOE_E4M3)[0] == M.MOE_EINVAL
    assert gb(K=17)[0] == M.MOE_EINVAL
    assert gb(dw13=None)[0] == M.MOE_EINVAL
    assert gb(dy=ctypes.c_void_p(0x1002))[0] == M.MOE_EINVAL   # misaligned
    assert gb(wsb=16)[0] == M.MOE_EWORKSPACE
    need = M.moe_gemm_backward_workspace_bytes(T, K, Nr, Ns, d, I, tm)
    assert need >= M.moe_permute_rows(T, K, Nr, Ns, tm) * 2 * I * 2 + 8 * ((Nr + 7) // 8) * 4
    g8 = lambda **kw: _status(L.moe_expert_gemm_backward_w8, *[kw.get(k, v) for k, v in dict(
        x=F, w13=F, w13s=F, w2=F, w2s=F, h=F, ab=F, dy=F, T=T, K=K, Nr=Nr, Ns=Ns, d=d, I=I, tm=tm, so=F, rt=F,
        tmap=F, nt=F, ws=F, wsb=big, dx=F, dw13=F, dw2=F, dwt=M.MOE_BF16, st=None).items()])
    assert g8(I=192)[0] == M.MOE_EUNSUPPORTED
    assert g8(d=16640)[0] == M.MOE_EUNSUPPORTED         # more than 128 scale blocks along d
    assert g8(I=8320)[0] == M.MOE_EUNSUPPORTED
    assert g8(w2s=None)[0] == M.MOE_EINVAL
    assert g8(dwt=M.MOE_E4M3)[0] == M.MOE_EINVAL
    assert g8(wsb=16)[0] == M.MOE_EWORKSPACE
    P = M.moe_permute_rows(T, K, Nr, Ns, tm)
    need8 = M.moe_gemm_backward_w8_workspace_bytes(T, K, Nr, Ns, d, I, tm)
    assert need8 >= P * 2 * I * 2 + P * 2 * I + P * d + P * (2 * I + d) // 128 * 4
    assert g8(wsb=need8 - 1)[0] == M.MOE_EWORKSPACE
    f8 = lambda **kw: _status(L.moe_expert_gemm_backward_f8, *[kw.get(k, v) for k, v in dict(
        x=F, w13=F, w13s=F, w2=F, w2s=F, h=F, ab=F, dy=F, T=T, K=K, Nr=Nr, Ns=Ns, d=d, I=I, tm=tm, so=F, rt=F,
        tmap=F, nt=F, ws=F, wsb=big, dx=F, dw13=F, dw2=F, dwt=M.MOE_BF16, st=None).items()])
    assert f8(I=192)[0] == M.MOE_EUNSUPPORTED
    assert f8(d=16640)[0] == M.MOE_EUNSUPPORTED
    assert f8(w13s=None)[0] == M.MOE_EINVAL
    assert f8(dwt=M.MOE_E4M3)[0] == M.MOE_EINVAL
    assert f8(h=ctypes.c_void_p(0x1008))[0] == M.MOE_EINVAL   # misaligned
    need_f8 = M.moe_gemm_backward_f8_workspace_bytes(T, K, Nr, Ns, d, I, tm)
    runs = M.fp8_quantize_runs_max(P, Nr + Ns)
    assert runs == (P + 127 * (Nr + Ns)) // 128
    # the E4M3 dgrad workspace, the run codes of h, x, dy and [da|db], four run-scale arrays
    assert need_f8 >= need8 + P * (I + d) + P * (d + 2 * I) + runs * (2 * d + 3 * I) * 4 + (Nr + Ns + 1) * 4
    assert f8(wsb=need_f8 - 1)[0] == M.MOE_EWORKSPACE
    assert M.moe_gemm_backward_f8_workspace_bytes(-1, K, Nr, Ns, d, I, tm) == 0
    qr = lambda **kw: _status(L.fp8_quantize_runs, *[kw.get(k, v) for k, v in dict(
        x=F, xt=M.MOE_BF16, xr=P, cols=d, rt=F, g=0, so=F, n=Nr + Ns, P=P, ro=F, q=F, sc=F, st=None).items()])
    assert qr(cols=200)[0] == M.MOE_EINVAL               # cols % 128 != 0
    assert qr(xt=M.MOE_E4M3)[0] == M.MOE_EINVAL
    assert qr(n=0)[0] == M.MOE_EINVAL
    assert qr(xr=P - 1)[0] == M.MOE_EINVAL              # x has fewer rows than the layout
    assert qr(xr=8, g=1, so=None)[0] == M.MOE_EINVAL
    assert qr(P=-1)[0] == M.MOE_EINVAL
    assert qr(q=ctypes.c_void_p(0x1004))[0] == M.MOE_EINVAL
    assert qr(cols=1 << 20, P=1 << 20, xr=1 << 20)[0] == M.MOE_EUNSUPPORTED
    assert M.fp8_quantize_runs_max(-5, 3) == 0
    gt = lambda **kw: _status(L.moe_expert_gemm_train, *[kw.get(k, v) for k, v in dict(
        x=F, w13=F, w2=F, T=T, K=K, Nr=Nr, Ns=Ns, d=d, I=I, tm=tm, so=F, rt=F, tmap=F, nt=F, ws=F, wsb=big,
        h=F, ab=F, y=F, yt=M.MOE_BF16, st=None).items()])
    assert gt(d=640)[0] == M.MOE_EUNSUPPORTED
    assert gt(ab=None)[0] == M.MOE_EINVAL
    assert gt(yt=M.MOE_E4M3)[0] == M.MOE_EINVAL
    assert gt(wsb=0)[0] == M.MOE_EWORKSPACE
    cb = lambda **kw: _status(L.moe_combine_backward, *[kw.get(k, v) for k, v in dict(
        g=F, gt=M.MOE_BF16, y=F, yt=M.MOE_BF16, inv=F, gate=F, score=F, so=F, T=T, d=d, K=K, Nr=Nr, Ns=Ns,
        dy=F, dg=F, dz=F, dzr=F, st=None).items()])
    assert cb(d=12)[0] == M.MOE_EINVAL
    assert cb(score=None)[0] == M.MOE_EINVAL
    assert cb(gt=M.MOE_E4M3)[0] == M.MOE_EINVAL
    rb = lambda **kw: _status(L.moe_route_backward, *[kw.get(k, v) for k, v in dict(
        g=F, gt=M.MOE_BF16, dx=F, u=F, ut=M.MOE_BF16, e=F, idx=F, inv=F, dz=F, dzr=F, so=F, rt=F, T=T, d=d, K=K,
        Nr=Nr, Ns=Ns, du=F, dut=M.MOE_F32, de=F, st=None).items()])
    assert rb(de=None)[0] == M.MOE_EINVAL
    assert rb(dut=M.MOE_E4M3)[0] == M.MOE_EINVAL
    assert rb(K=Nr + 1)[0] == M.MOE_EINVAL
