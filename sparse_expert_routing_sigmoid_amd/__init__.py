"""Python binding of libmoe_mi355x (DeepSeekMoE layer forward and backward on MI355X).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Tensors are torch tensors on the current HIP device; their data
pointers and torch's current stream go through ctypes to the C ABI declared
in include/moe_mi355x.h, with the same entry-point names.

There is no CPU fallback: importing works without a GPU (so the library can
be inspected), but every compute call raises if the library is missing.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mi355x.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP = range(5)
MOE_F32, MOE_BF16, MOE_E4M3 = 0, 1, 2
MOE_COMBINE_NO_RESIDUAL, MOE_COMBINE_NO_SHARED, MOE_COMBINE_NO_ROUTED = 1, 2, 4
MOE_TILE_ROWS = 256
MOE_MAX_K = 16
MOE_MAX_EXPERTS = 1024

# Every symbol the header declares, with its ctypes signature.
_vp, _i, _ll, _sz, _f, _u = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong, ctypes.c_size_t, ctypes.c_float, ctypes.c_uint
SIGNATURES = {
    "moe_abi_version": (_i, []),
    "moe_status_str": (ctypes.c_char_p, [_i]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_route_workspace_bytes": (_sz, [_i, _i, _i]),
    "moe_route": (_i, [_vp, _i, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_permute_rows": (_sz, [_i, _i, _i, _i, _i]),
    "moe_permute_tiles_max": (_sz, [_i, _i, _i, _i, _i]),
    "moe_permute_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "moe_permute": (_i, [_vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_permute_noalloc_scratch_bytes": (_sz, []),
    "moe_permute_noalloc": (_i, [_vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_gemm_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i, _i]),
    "moe_expert_gemm": (_i, [_vp, _i, _vp, _i, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i,
                             _vp, _vp, _vp, _vp, _vp, _sz, _vp, _i, _vp]),
    "moe_gemm_combine_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i, _i]),
    "moe_expert_gemm_combine": (_i, [_vp, _i, _vp, _i, _vp, _vp, _vp, _vp] + [_i] * 7 + [_vp] * 6 +
                                [_vp, _i, _u, _vp, _sz, _vp, _vp]),
    "moe_combine": (_i, [_vp, _i, _vp, _i, _vp, _vp, _vp, _i, _i, _i, _i, _i, _u, _vp, _i, _vp]),
    "moe_bias_update": (_i, [_vp, _i, _ll, _f, _vp, _vp]),
    "fp8_quantize_tiles": (_i, [_vp, _i, _ll, _ll, _i, _i, _vp, _vp, _vp]),
    "fp8_dequantize_tiles": (_i, [_vp, _vp, _ll, _ll, _i, _i, _vp, _i, _vp]),
    "moe_gemm_train_workspace_bytes": (_sz, [_i] * 7),
    "moe_expert_gemm_train": (_i, [_vp] * 3 + [_i] * 7 + [_vp] * 5 + [_sz] + [_vp] * 3 + [_i, _vp]),
    "moe_combine_backward": (_i, [_vp, _i, _vp, _i] + [_vp] * 4 + [_i] * 5 + [_vp] * 5),
    "moe_gemm_backward_workspace_bytes": (_sz, [_i] * 7),
    "moe_expert_gemm_backward": (_i, [_vp] * 6 + [_i] * 7 + [_vp] * 5 + [_sz] + [_vp] * 3 + [_i, _vp]),
    "moe_gemm_train_w8_workspace_bytes": (_sz, [_i] * 7),
    "moe_expert_gemm_train_w8": (_i, [_vp] * 6 + [_i] * 7 + [_vp] * 5 + [_sz] + [_vp] * 3 + [_i, _vp]),
    "moe_gemm_backward_w8_workspace_bytes": (_sz, [_i] * 7),
    "moe_expert_gemm_backward_w8": (_i, [_vp] * 8 + [_i] * 7 + [_vp] * 5 + [_sz] + [_vp] * 3 + [_i, _vp]),
    "moe_gemm_backward_f8_workspace_bytes": (_sz, [_i] * 7),
    "moe_expert_gemm_backward_f8": (_i, [_vp] * 8 + [_i] * 7 + [_vp] * 5 + [_sz] + [_vp] * 3 + [_i, _vp]),
    "fp8_quantize_runs_max": (_ll, [_ll, _i]),
    "fp8_quantize_runs": (_i, [_vp, _i, _ll, _i, _vp, _i, _vp, _i, _ll, _vp, _vp, _vp, _vp]),
    "moe_route_backward": (_i, [_vp, _i, _vp, _vp, _i] + [_vp] * 7 + [_i] * 5 + [_vp, _i, _vp, _vp]),
}

_lib = None


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_status_name(status)}: {msg}")
        self.status = status


def _status_name(s: int) -> str:
    return {0: "MOE_OK", 1: "MOE_EINVAL", 2: "MOE_EUNSUPPORTED", 3: "MOE_EWORKSPACE", 4: "MOE_EHIP"}.get(s, str(s))


def lib() -> ctypes.CDLL:
    """Load libmoe_mi355x.so (built by `python -m sparse_expert_routing_sigmoid_amd.build`)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_expert_routing_sigmoid_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int):
    if status != MOE_OK:
        raise MoeError(status, lib().moe_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        if t.numel() and not t.is_contiguous():
            raise ValueError("tensor must be contiguous")
        return t.data_ptr() if t.numel() else None
    return t


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.uint8:
        return MOE_E4M3
    raise ValueError(f"unsupported dtype {t.dtype}")


# ------------------------------------------------------------------ sizes --
def moe_route_workspace_bytes(T, d, Nr):
    return lib().moe_route_workspace_bytes(T, d, Nr)


def moe_permute_rows(T, K, Nr, Ns, tile_m):
    return lib().moe_permute_rows(T, K, Nr, Ns, tile_m)


def moe_permute_tiles_max(T, K, Nr, Ns, tile_m):
    return lib().moe_permute_tiles_max(T, K, Nr, Ns, tile_m)


def moe_permute_workspace_bytes(T, K, Nr, Ns):
    return lib().moe_permute_workspace_bytes(T, K, Nr, Ns)


def moe_gemm_workspace_bytes(T, K, Nr, Ns, d, I, tile_m, x_t, w_t):
    return lib().moe_gemm_workspace_bytes(T, K, Nr, Ns, d, I, tile_m, x_t, w_t)


def moe_gemm_train_workspace_bytes(T, K, Nr, Ns, d, I, tile_m):
    return lib().moe_gemm_train_workspace_bytes(T, K, Nr, Ns, d, I, tile_m)


def moe_gemm_backward_workspace_bytes(T, K, Nr, Ns, d, I, tile_m):
    return lib().moe_gemm_backward_workspace_bytes(T, K, Nr, Ns, d, I, tile_m)


def _nbytes(t):
    return t.numel() * t.element_size() if t is not None else 0


# ------------------------------------------------------------ entry points --
def moe_route(u, centroids, bias, K, topk_idx, topk_gate, topk_score, expert_load, ws, stream=None):
    T, d = u.shape
    Nr = centroids.shape[0]
    _check(lib().moe_route(_ptr(u), dtype_code(u), _ptr(centroids), _ptr(bias), T, d, Nr, K,
                           _ptr(topk_idx), _ptr(topk_gate), _ptr(topk_score), _ptr(expert_load),
                           _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream)))


def moe_permute(topk_idx, Nr, Ns, tile_m, seg_offset, row_token, inv_row, tile_map, n_tiles, ws, stream=None):
    T, K = topk_idx.shape
    _check(lib().moe_permute(_ptr(topk_idx), T, K, Nr, Ns, tile_m, _ptr(seg_offset), _ptr(row_token),
                             _ptr(inv_row), _ptr(tile_map), _ptr(n_tiles), _ptr(ws),
                             ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream)))


def moe_permute_noalloc(topk_idx, Nr, Ns, tile_m, seg_offset, row_token, inv_row, tile_map, n_tiles, stream=None):
    """moe_permute with the library's own scratch array: allocates nothing."""
    T, K = topk_idx.shape
    _check(lib().moe_permute_noalloc(_ptr(topk_idx), T, K, Nr, Ns, tile_m, _ptr(seg_offset), _ptr(row_token),
                                     _ptr(inv_row), _ptr(tile_map), _ptr(n_tiles), _stream(stream)))


def moe_expert_gemm(x, x_scale, w_t, w13, w13_scale, w2, w2_scale, T, K, Nr, Ns, d, I, tile_m,
                    seg_offset, row_token, tile_map, n_tiles, ws, y, x_t=None, stream=None):
    x_t = dtype_code(x) if x_t is None else x_t
    _check(lib().moe_expert_gemm(_ptr(x), x_t, _ptr(x_scale), w_t, _ptr(w13), _ptr(w13_scale), _ptr(w2),
                                 _ptr(w2_scale), T, K, Nr, Ns, d, I, tile_m, _ptr(seg_offset), _ptr(row_token),
                                 _ptr(tile_map), _ptr(n_tiles), _ptr(ws),
                                 ws.numel() * ws.element_size() if ws is not None else 0,
                                 _ptr(y), dtype_code(y), _stream(stream)))


def moe_gemm_combine_workspace_bytes(T, K, Nr, Ns, d, I, tile_m, x_t, w_t):
    return lib().moe_gemm_combine_workspace_bytes(T, K, Nr, Ns, d, I, tile_m, x_t, w_t)


def moe_expert_gemm_combine(x, x_scale, w_t, w13, w13_scale, w2, w2_scale, T, K, Nr, Ns, d, I, tile_m, seg_offset,
                            row_token, tile_map, n_tiles, inv_row, topk_gate, u, ws, out, flags=0, x_t=None,
                            stream=None):
    """Expert GEMMs with the combine fused into the down projection (fp32
    atomics; not bitwise reproducible); out [T, d] fp32."""
    x_t = dtype_code(x) if x_t is None else x_t
    _check(lib().moe_expert_gemm_combine(_ptr(x), x_t, _ptr(x_scale), w_t, _ptr(w13), _ptr(w13_scale), _ptr(w2),
                                         _ptr(w2_scale), T, K, Nr, Ns, d, I, tile_m, _ptr(seg_offset),
                                         _ptr(row_token), _ptr(tile_map), _ptr(n_tiles), _ptr(inv_row),
                                         _ptr(topk_gate), _ptr(u), dtype_code(u), flags, _ptr(ws), _nbytes(ws),
                                         _ptr(out), _stream(stream)))


def moe_expert_gemm_train(x, w13, w2, T, K, Nr, Ns, d, I, tile_m, seg_offset, row_token, tile_map, n_tiles,
                          ws, h, ab, y, stream=None):
    _check(lib().moe_expert_gemm_train(_ptr(x), _ptr(w13), _ptr(w2), T, K, Nr, Ns, d, I, tile_m, _ptr(seg_offset),
                                       _ptr(row_token), _ptr(tile_map), _ptr(n_tiles), _ptr(ws), _nbytes(ws),
                                       _ptr(h), _ptr(ab), _ptr(y), dtype_code(y), _stream(stream)))


def moe_combine_backward(grad_out, y, inv_row, topk_gate, topk_score, seg_offset, Nr, Ns, dy, dgate, dz, dz_row,
                         stream=None):
    T, d = grad_out.shape
    K = inv_row.shape[1]
    _check(lib().moe_combine_backward(_ptr(grad_out), dtype_code(grad_out), _ptr(y), dtype_code(y), _ptr(inv_row),
                                      _ptr(topk_gate), _ptr(topk_score), _ptr(seg_offset), T, d, K, Nr, Ns, _ptr(dy),
                                      _ptr(dgate), _ptr(dz), _ptr(dz_row), _stream(stream)))


def moe_expert_gemm_backward(x, w13, w2, h, ab, dy, T, K, Nr, Ns, d, I, tile_m, seg_offset, row_token, tile_map,
                             n_tiles, ws, dx, dw13, dw2, stream=None):
    _check(lib().moe_expert_gemm_backward(_ptr(x), _ptr(w13), _ptr(w2), _ptr(h), _ptr(ab), _ptr(dy), T, K, Nr, Ns,
                                          d, I, tile_m, _ptr(seg_offset), _ptr(row_token), _ptr(tile_map),
                                          _ptr(n_tiles), _ptr(ws), _nbytes(ws), _ptr(dx), _ptr(dw13), _ptr(dw2),
                                          dtype_code(dw13), _stream(stream)))


def moe_gemm_train_w8_workspace_bytes(T, K, Nr, Ns, d, I, tile_m):
    return lib().moe_gemm_train_w8_workspace_bytes(T, K, Nr, Ns, d, I, tile_m)


def moe_expert_gemm_train_w8(xq, xs, w8: "ExpertWeights", T, K, Nr, Ns, d, I, tile_m, seg_offset, row_token,
                             tile_map, n_tiles, ws, h, ab, y, stream=None):
    """The E4M3 expert GEMMs keeping h and [a | b] (bf16) for the backward;
    xq / xs: u in 1x128 E4M3 tiles (fp8_quantize_tiles)."""
    if w8.w_t != MOE_E4M3:
        raise ValueError("moe_expert_gemm_train_w8 needs E4M3 weights")
    _check(lib().moe_expert_gemm_train_w8(_ptr(xq), _ptr(xs), _ptr(w8.w13), _ptr(w8.w13_scale), _ptr(w8.w2),
                                          _ptr(w8.w2_scale), T, K, Nr, Ns, d, I, tile_m, _ptr(seg_offset),
                                          _ptr(row_token), _ptr(tile_map), _ptr(n_tiles), _ptr(ws), _nbytes(ws),
                                          _ptr(h), _ptr(ab), _ptr(y), dtype_code(y), _stream(stream)))


def moe_gemm_backward_w8_workspace_bytes(T, K, Nr, Ns, d, I, tile_m):
    return lib().moe_gemm_backward_w8_workspace_bytes(T, K, Nr, Ns, d, I, tile_m)


def moe_expert_gemm_backward_w8(x, w8: "ExpertWeights", h, ab, dy, T, K, Nr, Ns, d, I, tile_m, seg_offset, row_token,
                                tile_map, n_tiles, ws, dx, dw13, dw2, stream=None):
    """moe_expert_gemm_backward with the input-gradient products on E4M3
    operands; w8: the E4M3 expert weights (quantize_weights)."""
    if w8.w_t != MOE_E4M3:
        raise ValueError("moe_expert_gemm_backward_w8 needs E4M3 weights")
    _check(lib().moe_expert_gemm_backward_w8(_ptr(x), _ptr(w8.w13), _ptr(w8.w13_scale), _ptr(w8.w2),
                                             _ptr(w8.w2_scale), _ptr(h), _ptr(ab), _ptr(dy), T, K, Nr, Ns, d, I,
                                             tile_m, _ptr(seg_offset), _ptr(row_token), _ptr(tile_map),
                                             _ptr(n_tiles), _ptr(ws), _nbytes(ws), _ptr(dx), _ptr(dw13), _ptr(dw2),
                                             dtype_code(dw13), _stream(stream)))


def moe_gemm_backward_f8_workspace_bytes(T, K, Nr, Ns, d, I, tile_m):
    return lib().moe_gemm_backward_f8_workspace_bytes(T, K, Nr, Ns, d, I, tile_m)


def moe_expert_gemm_backward_f8(x, w8: "ExpertWeights", h, ab, dy, T, K, Nr, Ns, d, I, tile_m, seg_offset, row_token,
                                tile_map, n_tiles, ws, dx, dw13, dw2, stream=None):
    """moe_expert_gemm_backward_w8 with the weight-gradient products on E4M3
    operands too (runs of 128 rows along the tokens)."""
    if w8.w_t != MOE_E4M3:
        raise ValueError("moe_expert_gemm_backward_f8 needs E4M3 weights")
    _check(lib().moe_expert_gemm_backward_f8(_ptr(x), _ptr(w8.w13), _ptr(w8.w13_scale), _ptr(w8.w2),
                                             _ptr(w8.w2_scale), _ptr(h), _ptr(ab), _ptr(dy), T, K, Nr, Ns, d, I,
                                             tile_m, _ptr(seg_offset), _ptr(row_token), _ptr(tile_map),
                                             _ptr(n_tiles), _ptr(ws), _nbytes(ws), _ptr(dx), _ptr(dw13), _ptr(dw2),
                                             dtype_code(dw13), _stream(stream)))


def fp8_quantize_runs_max(P, n_seg):
    return lib().fp8_quantize_runs_max(P, n_seg)


def fp8_quantize_runs(x, row_token, gather, seg_offset, P, run_offset, q, scale, stream=None):
    """E4M3 along the rows of the permuted layout: each segment of
    seg_offset in runs of 128 rows, one power-of-two scale per run and
    column.  x [P, cols], or with gather [rows, cols] read at row_token."""
    rows, cols = x.shape
    _check(lib().fp8_quantize_runs(_ptr(x), dtype_code(x), rows, cols, _ptr(row_token), int(bool(gather)),
                                   _ptr(seg_offset), seg_offset.shape[0] - 1, P, _ptr(run_offset), _ptr(q),
                                   _ptr(scale), _stream(stream)))


def moe_route_backward(grad_out, dx, u, centroids, topk_idx, inv_row, dz, dz_row, seg_offset, row_token, Nr, Ns,
                       du, de, stream=None):
    T, d = u.shape
    K = topk_idx.shape[1]
    _check(lib().moe_route_backward(_ptr(grad_out), dtype_code(grad_out), _ptr(dx), _ptr(u), dtype_code(u),
                                    _ptr(centroids), _ptr(topk_idx), _ptr(inv_row), _ptr(dz), _ptr(dz_row),
                                    _ptr(seg_offset), _ptr(row_token), T, d, K, Nr, Ns, _ptr(du), dtype_code(du),
                                    _ptr(de), _stream(stream)))


def moe_combine(u, y, inv_row, topk_gate, seg_offset, Nr, Ns, out, flags=0, stream=None):
    T, d = u.shape
    K = inv_row.shape[1]
    _check(lib().moe_combine(_ptr(u), dtype_code(u), _ptr(y), dtype_code(y), _ptr(inv_row), _ptr(topk_gate),
                             _ptr(seg_offset), T, d, K, Nr, Ns, flags, _ptr(out), dtype_code(out), _stream(stream)))


def moe_bias_update(expert_load, total_assign, gamma, bias, stream=None):
    _check(lib().moe_bias_update(_ptr(expert_load), bias.shape[0], int(total_assign), float(gamma), _ptr(bias),
                                 _stream(stream)))


def fp8_quantize_tiles(x, tile_rows, q, scale, tile_cols=128, stream=None):
    """Quantise x viewed as [rows, cols] = [numel / last dim, last dim]."""
    cols = x.shape[-1]
    rows = x.numel() // cols if cols else 0
    _check(lib().fp8_quantize_tiles(_ptr(x), dtype_code(x), rows, cols, tile_rows, tile_cols, _ptr(q), _ptr(scale),
                                    _stream(stream)))


def fp8_dequantize_tiles(q, scale, tile_rows, out, tile_cols=128, stream=None):
    """Values of E4M3 tiles (code x tile scale) into out (fp32 or bf16), q
    viewed as [numel / last dim, last dim]."""
    cols = q.shape[-1]
    rows = q.numel() // cols if cols else 0
    _check(lib().fp8_dequantize_tiles(_ptr(q), _ptr(scale), rows, cols, tile_rows, tile_cols, _ptr(out),
                                      dtype_code(out), _stream(stream)))


# ------------------------------------------------------- layer plumbing --
@dataclass
class ExpertWeights:
    """Expert weights as the library reads them: W13 [E, 2I, d], W2 [E, d, I]
    (bf16/fp32 tensors, or E4M3 codes (uint8) with fp32 block scales)."""
    w_t: int
    w13: torch.Tensor
    w2: torch.Tensor
    w13_scale: torch.Tensor | None = None
    w2_scale: torch.Tensor | None = None


def quantize_weights(w13: torch.Tensor, w2: torch.Tensor, stream=None) -> ExpertWeights:
    """E4M3 codes + 128x128 block scales of fp32/bf16 expert weights, made by
    fp8_quantize_tiles (one 128x128 block per scale)."""
    E, twoI, d = w13.shape
    I = w2.shape[2]
    q13 = torch.empty((E, twoI, d), dtype=torch.uint8, device=w13.device)
    s13 = torch.empty((E, twoI // 128, d // 128), dtype=torch.float32, device=w13.device)
    q2 = torch.empty((E, d, I), dtype=torch.uint8, device=w2.device)
    s2 = torch.empty((E, d // 128, I // 128), dtype=torch.float32, device=w2.device)
    fp8_quantize_tiles(w13, 128, q13, s13, stream=stream)
    fp8_quantize_tiles(w2, 128, q2, s2, stream=stream)
    return ExpertWeights(MOE_E4M3, q13, q2, s13, s2)


class MoeLayer:
    """Buffers and call order of one DeepSeekMoE layer forward.

    Allocates every output and workspace once (torch, on `device`) and runs
    moe_route -> moe_permute -> [fp8_quantize_tiles] -> moe_expert_gemm ->
    moe_combine, then moe_bias_update when a step ends.  No host
    synchronisation happens inside forward()."""

    def __init__(self, T, d, Nr, Ns, I, K, act_dtype, weights: ExpertWeights, x_fp8=False,
                 tile_m=32, out_dtype=None, device="cuda", train=False, grad_dtype=None, dgrad_weights=None,
                 fused_combine=False, wgrad_fp8=None):
        self.T, self.d, self.Nr, self.Ns, self.I, self.K = T, d, Nr, Ns, I, K
        self.tile_m, self.x_fp8, self.w = tile_m, x_fp8, weights
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        P = moe_permute_rows(T, K, Nr, Ns, tile_m)
        tiles = moe_permute_tiles_max(T, K, Nr, Ns, tile_m)
        self.P_max, self.tiles_max = P, tiles
        self.topk_idx = torch.empty((T, K), **i32)
        self.topk_gate = torch.empty((T, K), **f32)
        self.topk_score = torch.empty((T, K), **f32)
        self.expert_load = torch.empty((Nr,), **i32)
        self.route_ws = torch.empty((max(moe_route_workspace_bytes(T, d, Nr), 1),), dtype=torch.uint8, device=dev)
        self.seg_offset = torch.empty((Nr + Ns + 1,), **i32)
        self.row_token = torch.empty((P,), **i32)
        self.inv_row = torch.empty((T, K), **i32)
        self.tile_map = torch.empty((tiles, 4), **i32)
        self.n_tiles = torch.empty((1,), **i32)
        self.perm_ws = torch.empty((max(moe_permute_workspace_bytes(T, K, Nr, Ns), 1),), dtype=torch.uint8,
                                   device=dev)
        self.x_t = MOE_E4M3 if x_fp8 else (MOE_BF16 if act_dtype == torch.bfloat16 else MOE_F32)
        if x_fp8:
            self.xq = torch.empty((T, d), dtype=torch.uint8, device=dev)
            self.xs = torch.empty((T, d // 128), **f32)
        self.gemm_ws = torch.empty((max(moe_gemm_workspace_bytes(T, K, Nr, Ns, d, I, tile_m, self.x_t,
                                                                  weights.w_t), 1),),
                                   dtype=torch.uint8, device=dev)
        out_dtype = act_dtype if out_dtype is None else out_dtype
        self.fused = fused_combine
        if fused_combine:
            # moe_expert_gemm_combine: no y rows; the output is fp32
            self.fc_ws = torch.empty((max(moe_gemm_combine_workspace_bytes(T, K, Nr, Ns, d, I, tile_m, self.x_t,
                                                                           weights.w_t), 1),),
                                     dtype=torch.uint8, device=dev)
            self.out = torch.empty((T, d), dtype=torch.float32, device=dev)
        else:
            self.y = torch.empty((P, d), dtype=out_dtype, device=dev)
            self.out = torch.empty((T, d), dtype=out_dtype, device=dev)
        self.train = train
        if train:
            # the training forward keeps h and the pre-activations [a | b]
            # for the backward: bf16 activations with bf16 weights, or the
            # E4M3 path (x_fp8 with E4M3 weights, which the backward's
            # input-gradient products then use too)
            self.train_fp8 = x_fp8 and weights.w_t == MOE_E4M3
            if act_dtype != torch.bfloat16 or not (self.train_fp8 or (not x_fp8 and weights.w_t == MOE_BF16)):
                raise ValueError("training needs bf16 activations with bf16 weights, or x_fp8 with E4M3 weights")
            if self.train_fp8:
                if dgrad_weights is not None and dgrad_weights is not weights:
                    raise ValueError("the E4M3 training path uses its own weights for the backward")
                dgrad_weights = weights
            bf16 = dict(dtype=torch.bfloat16, device=dev)
            E = Nr + Ns
            self.h = torch.empty((P, I), **bf16)
            self.ab = torch.empty((P, 2 * I), **bf16)
            tws = moe_gemm_train_w8_workspace_bytes if self.train_fp8 else moe_gemm_train_workspace_bytes
            self.train_ws = torch.empty((max(tws(T, K, Nr, Ns, d, I, tile_m), 1),), dtype=torch.uint8, device=dev)
            gd = (torch.bfloat16 if self.train_fp8 else weights.w13.dtype) if grad_dtype is None else grad_dtype
            self.dy = torch.empty((P, d), **bf16)
            self.dx = torch.empty((P, d), **bf16)
            self.dgate = torch.empty((T, K), **f32)
            self.dz = torch.empty((T, K), **f32)
            self.dz_row = torch.empty((P,), **f32)
            # dgrad_weights: E4M3 copies of the weights (quantize_weights); the
            # backward then runs its input-gradient products on E4M3 operands
            self.dgrad_w = dgrad_weights
            # the E4M3 step's gate/up weight gradient takes Q(u), the operand
            # its forward multiplied (straight-through quantisers)
            self.xdq = torch.empty((T, d), **bf16) if self.train_fp8 else None
            if dgrad_weights is not None and dgrad_weights.w_t != MOE_E4M3:
                raise ValueError("dgrad_weights must be E4M3 weights")
            # wgrad_fp8: the weight gradients on E4M3 operands too
            # (moe_expert_gemm_backward_f8); the E4M3 training step's default
            self.wgrad_fp8 = self.train_fp8 if wgrad_fp8 is None else bool(wgrad_fp8)
            if self.wgrad_fp8 and not self.train_fp8:
                raise ValueError("wgrad_fp8 needs the E4M3 training path (x_fp8 with E4M3 weights)")
            if dgrad_weights is None:
                ws_fn = moe_gemm_backward_workspace_bytes
            else:
                ws_fn = moe_gemm_backward_f8_workspace_bytes if self.wgrad_fp8 else moe_gemm_backward_w8_workspace_bytes
            self.bwd_ws = torch.empty((max(ws_fn(T, K, Nr, Ns, d, I, tile_m), 1),), dtype=torch.uint8, device=dev)
            self.dw13 = torch.empty((E, 2 * I, d), dtype=gd, device=dev)
            self.dw2 = torch.empty((E, d, I), dtype=gd, device=dev)
            self.du = torch.empty((T, d), dtype=act_dtype, device=dev)
            self.de = torch.empty((Nr, d), **f32)

    def route(self, u, centroids, bias, stream=None):
        moe_route(u, centroids, bias, self.K, self.topk_idx, self.topk_gate, self.topk_score, self.expert_load,
                  self.route_ws, stream)

    def permute(self, stream=None):
        moe_permute(self.topk_idx, self.Nr, self.Ns, self.tile_m, self.seg_offset, self.row_token, self.inv_row,
                    self.tile_map, self.n_tiles, self.perm_ws, stream)

    def experts(self, u, stream=None):
        w = self.w
        if self.x_fp8:
            fp8_quantize_tiles(u, 1, self.xq, self.xs, stream=stream)
            x, xs = self.xq, self.xs
        else:
            x, xs = u, None
        if self.train:
            if self.train_fp8:
                moe_expert_gemm_train_w8(x, xs, w, self.T, self.K, self.Nr, self.Ns, self.d, self.I, self.tile_m,
                                         self.seg_offset, self.row_token, self.tile_map, self.n_tiles, self.train_ws,
                                         self.h, self.ab, self.y, stream)
            else:
                moe_expert_gemm_train(u, w.w13, w.w2, self.T, self.K, self.Nr, self.Ns, self.d, self.I, self.tile_m,
                                      self.seg_offset, self.row_token, self.tile_map, self.n_tiles, self.train_ws,
                                      self.h, self.ab, self.y, stream)
            return
        moe_expert_gemm(x, xs, w.w_t, w.w13, w.w13_scale, w.w2, w.w2_scale, self.T, self.K, self.Nr, self.Ns,
                        self.d, self.I, self.tile_m, self.seg_offset, self.row_token, self.tile_map, self.n_tiles,
                        self.gemm_ws, self.y, x_t=self.x_t, stream=stream)

    def combine(self, u, flags=0, out=None, stream=None):
        out = self.out if out is None else out
        moe_combine(u, self.y, self.inv_row, self.topk_gate, self.seg_offset, self.Nr, self.Ns, out, flags, stream)
        return out

    def experts_combine(self, u, flags=0, stream=None):
        """Expert GEMMs with the combine fused into the down projection
        (moe_expert_gemm_combine); returns the fp32 layer output."""
        w = self.w
        if self.x_fp8:
            fp8_quantize_tiles(u, 1, self.xq, self.xs, stream=stream)
            x, xs = self.xq, self.xs
        else:
            x, xs = u, None
        moe_expert_gemm_combine(x, xs, w.w_t, w.w13, w.w13_scale, w.w2, w.w2_scale, self.T, self.K, self.Nr, self.Ns,
                                self.d, self.I, self.tile_m, self.seg_offset, self.row_token, self.tile_map,
                                self.n_tiles, self.inv_row, self.topk_gate, u, self.fc_ws, self.out, flags,
                                x_t=self.x_t, stream=stream)
        return self.out

    def forward(self, u, centroids, bias, stream=None):
        self.route(u, centroids, bias, stream)
        self.permute(stream)
        if self.fused:
            return self.experts_combine(u, stream=stream)
        self.experts(u, stream)
        return self.combine(u, stream=stream)

    def backward(self, grad_out, u, centroids, stream=None):
        """Gradients of the last training forward for dL/dh' = grad_out:
        returns (du, de, dW13, dW2); the bias gets none."""
        if not self.train:
            raise RuntimeError("backward needs a layer built with train=True")
        w = self.w
        moe_combine_backward(grad_out, self.y, self.inv_row, self.topk_gate, self.topk_score, self.seg_offset,
                             self.Nr, self.Ns, self.dy, self.dgate, self.dz, self.dz_row, stream)
        if self.dgrad_w is None:
            moe_expert_gemm_backward(u, w.w13, w.w2, self.h, self.ab, self.dy, self.T, self.K, self.Nr, self.Ns,
                                     self.d, self.I, self.tile_m, self.seg_offset, self.row_token, self.tile_map,
                                     self.n_tiles, self.bwd_ws, self.dx, self.dw13, self.dw2, stream)
        else:
            x = u
            if self.train_fp8:
                fp8_dequantize_tiles(self.xq, self.xs, 1, self.xdq, stream=stream)
                x = self.xdq
            bwd = moe_expert_gemm_backward_f8 if self.wgrad_fp8 else moe_expert_gemm_backward_w8
            bwd(x, self.dgrad_w, self.h, self.ab, self.dy, self.T, self.K, self.Nr, self.Ns, self.d, self.I,
                self.tile_m, self.seg_offset, self.row_token, self.tile_map, self.n_tiles, self.bwd_ws, self.dx,
                self.dw13, self.dw2, stream)
        moe_route_backward(grad_out, self.dx, u, centroids, self.topk_idx, self.inv_row, self.dz, self.dz_row,
                           self.seg_offset, self.row_token, self.Nr, self.Ns, self.du, self.de, stream)
        return self.du, self.de, self.dw13, self.dw2

    def update_bias(self, bias, gamma=0.001, stream=None):
        moe_bias_update(self.expert_load, self.T * self.K, gamma, bias, stream)


def moe_forward(u, centroids, bias, weights: ExpertWeights, K, Ns, update_bias=False, gamma=0.001, x_fp8=False,
                tile_m=32, out_dtype=None, stream=None):
    """One DeepSeekMoE layer forward in a single call: route, permute,
    [quantise u], expert GEMMs, combine, and optionally the end-of-step bias
    rule (the bias tensor is updated in place).  Allocates the layer's
    buffers on every call (MoeLayer keeps them across steps).  Returns
    (out, layer): the layer holds the routing, loads and layout of the call.

    u [T, d] (fp32/bf16), centroids [N_r, d] fp32, bias [N_r] fp32,
    weights: ExpertWeights of the N_r routed + Ns shared experts."""
    T, d = u.shape
    Nr = centroids.shape[0]
    I = weights.w2.shape[2]
    layer = MoeLayer(T, d, Nr, Ns, I, K, u.dtype, weights, x_fp8=x_fp8, tile_m=tile_m, out_dtype=out_dtype,
                     device=u.device)
    out = layer.forward(u, centroids, bias, stream)
    if update_bias:
        layer.update_bias(bias, gamma, stream)
    return out, layer
