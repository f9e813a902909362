"""Plain fp64 CPU oracle of the DeepSeekMoE layer backward (test infrastructure).

THIS IS TEST INFRASTRUCTURE.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it; the HIP library shares nothing
with it.  Every step is the derivative of the corresponding forward step of
oracle/moe.py, written out in fp64 with NumPy matmuls.

Sources: the forward equations of the "DeepSeek-V3 Technical Report" reading
guide (xyznot.com), Method section 2 ([RG-MoE]: combine equation, affinity
sentence, gate equation, bias rule), with the readings R1 (gate = s / sum of
the selected s), R2 (selection order), R6 (SwiGLU FFN) and R7 (shared gate 1,
residual) of oracle/moe.py.  The pages print no backward pass; it follows
from the forward by the chain rule:

  out_t = u_t + sum_j FFN_j(u_t) + sum_k g_{t,k} FFN_{i_k}(u_t)
  g_{t,k} = s_{t,k} / S_t,  S_t = sum_k s_{t,k},  s = sigmoid(u_t . e_i)
  FFN(x) = W2 (SiLU(a) * b),  [a; b] = W13 x

Reading B1: the selection (top-K of s + b) is piecewise constant, so it gets
no derivative: gradients flow through the gates of the selected experts
only, and the bias b gets none.  This holds everywhere except on the
measure-zero set of exact ties, where the layer is not differentiable.

FP8 variant (ffn_backward_fp8): the same page's "Key ideas" FP8 bullet puts
every tensor in E4M3 with 1x128 tiles for activations and 128x128 blocks for
weights.  Reading B2: the two input-gradient products (dh = dy W2 and
dx = [da | db] W13) take the activation gradient in 1x128 tiles along their
K axis and the weights in the forward's 128x128 blocks, each tile with its
power-of-two scale (R10 of oracle/moe.py).  The weight-gradient products stay
unquantised: their K axis is the token axis, along which the pages give no
tiling.

Reading B4 (the precision in which an E4M3 code is decided): activations and
activation gradients are bf16 tensors, as every activation of the layer is
stored.  So dy and [da | db] are rounded to bf16 (through fp32, round to
nearest even) before their 1x128 quantisation, and the SwiGLU backward is
evaluated at the pre-activations a, b as the training forward keeps them,
rounded to bf16.  The codes are then decided from the same values the GPU
quantises; the weight gradients, which decide no code, use the unrounded
fp64 values.

FP8 training step (ffn_backward_fp8_train): the forward of the FP8 path
(oracle/moe.py, R8: x in 1x128 tiles, h re-quantised in 1x128 tiles, the
weights in 128x128 blocks) followed by the backward of readings B2 and B4.
Reading B3: every quantiser of the forward passes the gradient straight
through (it is the identity when differentiated), so each weight gradient
uses the quantised operand that its forward product multiplied: dW2 the
quantised h, dW13 the quantised expert input Q(x).

Reading B5 (E4M3 weight gradients, fp8_wgrad=True): the weight-gradient
products dW2 = dy^T Q(h) and dW13 = [da | db]^T Q(x) sum over one expert's
rows, the token axis, and the pages give no tile shape along it.  B2's rule
for activation operands (1x128 tiles along the product's K axis) is kept:
both operands are quantised column by column in runs of 128 consecutive
rows of the expert, its rows taken in token order, the last run shorter
(as if padded with zero rows), each run with its own power-of-two scale.
The codes are decided from bf16 values (B4): dy and [da | db] are rounded
to bf16 first; Q(h) and Q(x) are decoded E4M3 values, exact in bf16, and
are quantised again along the token axis.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .e4m3 import dequantize_tiles, quantize_tiles
from .moe import route, sigmoid


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def silu(a: np.ndarray) -> np.ndarray:
    return a * sigmoid(a)


def silu_grad(a: np.ndarray) -> np.ndarray:
    """d/da [a * sigmoid(a)] = sigmoid(a) * (1 + a * (1 - sigmoid(a)))."""
    sg = sigmoid(a)
    return sg * (1.0 + a * (1.0 - sg))


@dataclass
class LayerGrads:
    du: np.ndarray      # [T, d]       dL/du (residual + experts + router)
    de: np.ndarray      # [N_r, d]     dL/de (centroids)
    dw13: np.ndarray    # [E, 2I, d]   dL/dW13 (gate rows, then up rows)
    dw2: np.ndarray     # [E, d, I]    dL/dW2
    dgate: np.ndarray   # [T, K]       dL/dg of the selected experts
    dz: np.ndarray      # [T, K]       dL/d(u_t . e_i) of the selected experts
    du_ffn: np.ndarray  # [T, d]       the part of du that flows through the expert FFNs
    du_router: np.ndarray  # [T, d]    the part of du that flows through the gates


def ffn_backward(x: np.ndarray, w13: np.ndarray, w2: np.ndarray, dy: np.ndarray):
    """Backward of y = W2 (SiLU(a) * b), [a; b] = W13 x, for rows x [n, d]
    and output gradients dy [n, d].  Returns (dx [n, d], dw13 [2I, d],
    dw2 [d, I], y [n, d])."""
    x, w13, w2, dy = _f64(x), _f64(w13), _f64(w2), _f64(dy)
    I = w2.shape[1]
    ab = x @ w13.T
    a, b = ab[:, :I], ab[:, I:]
    h = silu(a) * b
    y = h @ w2.T
    dw2 = dy.T @ h                      # [d, I]
    dh = dy @ w2                        # [n, I]
    da = dh * b * silu_grad(a)
    db = dh * silu(a)
    dab = np.concatenate([da, db], axis=1)   # [n, 2I]
    dw13 = dab.T @ x                    # [2I, d]
    dx = dab @ w13                      # [n, d]
    return dx, dw13, dw2, y


def round_bf16(x: np.ndarray) -> np.ndarray:
    """x as the GPU stores an fp32 result in bf16 (reading B4): rounded to
    fp32, then to the nearest bf16, ties to even.  bf16 keeps the sign, the 8
    exponent bits and the top 7 fraction bits of an fp32, so rounding adds
    half of the dropped 16-bit field (minus one unless the kept lowest bit is
    set) and truncates.  Returns fp64 (exact).  Finite input only."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    if not np.all(np.isfinite(f)):
        raise ValueError("round_bf16: non-finite input")
    bits = f.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32).astype(np.float64)


def _q_act(g: np.ndarray) -> np.ndarray:
    """g rounded to fp32, then through 1x128 E4M3 tiles (code x scale, fp64):
    the forward's activation quantiser (R8)."""
    q, s = quantize_tiles(np.asarray(g, dtype=np.float64).astype(np.float32), 1, 128)
    return dequantize_tiles(q, s, 1, 128)


def _q_grad(g: np.ndarray) -> np.ndarray:
    """An activation gradient as the E4M3 backward products take it: rounded
    to bf16 (B4), then through 1x128 E4M3 tiles (B2)."""
    return _q_act(round_bf16(g))


def fp8_tile_matmul(g: np.ndarray, w: np.ndarray) -> np.ndarray:
    """g [n, K] @ w [K, N] with both operands in E4M3 (reading B2): g, whose
    values must be exact in fp32, in 1x128 tiles along K, w in 128x128 blocks
    of its stored layout; the dequantised values (code x power-of-two scale,
    exact) are multiplied in fp64."""
    wq, ws = quantize_tiles(np.asarray(w, dtype=np.float64).astype(np.float32), 128, 128)
    gq, gs = quantize_tiles(np.asarray(g), 1, 128)
    return dequantize_tiles(gq, gs, 1, 128) @ dequantize_tiles(wq, ws, 128, 128)


def quantize_token_runs(m: np.ndarray) -> np.ndarray:
    """Reading B5: m [n, C] (values exact in fp32; the n rows of one expert in
    token order) through E4M3 with one power-of-two scale per column and run
    of 128 consecutive rows, the last run shorter.  Returns the decoded values
    (code x scale, fp64, exact)."""
    m = np.asarray(m, dtype=np.float64)
    n, C = m.shape
    if n == 0:
        return np.zeros((0, C))
    padded = np.zeros((-(-n // 128) * 128, C))
    padded[:n] = m                       # zero rows change no run's largest magnitude
    q, s = quantize_tiles(padded, 128, 1)
    return dequantize_tiles(q, s, 128, 1)[:n]


def fp8_wgrad(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """a^T b [M, N] over the rows of one expert (a [n, M], b [n, N], values
    exact in fp32) with both operands in E4M3 runs along the rows (reading
    B5); the decoded values are multiplied in fp64."""
    return quantize_token_runs(a).T @ quantize_token_runs(b)


def ffn_backward_fp8(x: np.ndarray, w13: np.ndarray, w2: np.ndarray, dy: np.ndarray):
    """ffn_backward with the input-gradient products in E4M3 (readings B2,
    B4): dh = Q(bf16(dy)) Q(W2), dx = Q(bf16([da | db])) Q(W13), with da, db
    evaluated at the bf16 pre-activations; the weight gradients use the
    unquantised dy and [da | db].  Returns (dx, dw13, dw2, y)."""
    x, w13, w2, dy = _f64(x), _f64(w13), _f64(w2), _f64(dy)
    I = w2.shape[1]
    ab = x @ w13.T
    a, b = ab[:, :I], ab[:, I:]
    h = silu(a) * b
    y = h @ w2.T
    dw2 = dy.T @ h
    dh = fp8_tile_matmul(round_bf16(dy), w2)
    ar, br = round_bf16(a), round_bf16(b)
    da = dh * br * silu_grad(ar)
    db = dh * silu(ar)
    dab = np.concatenate([da, db], axis=1)
    dw13 = dab.T @ x
    dx = fp8_tile_matmul(round_bf16(dab), w13)
    return dx, dw13, dw2, y


def ffn_backward_fp8_train(x: np.ndarray, w13q: np.ndarray, w2q: np.ndarray, dy: np.ndarray,
                           fp8_wgrad_products: bool = False):
    """Forward and backward of one expert on the FP8 training path (readings
    B2-B4).  x [n, d] the expert's input rows as stored; w13q [2I, d], w2q
    [d, I] the decoded E4M3 weights (code x block scale).
      forward:  [a; b] = W13q Q(x),  h = Q(SiLU(a) b),  y = W2q h
      backward: dW2 = dy^T h,  dh = Q(bf16(dy)) W2q,  da, db at bf16(a), bf16(b),
                dW13 = [da | db]^T Q(x),  dx = Q(bf16([da | db])) W13q
    Q: 1x128 E4M3 tiles along the row.  fp8_wgrad_products: the two weight
    gradients on E4M3 operands (reading B5),
                dW2 = R(bf16(dy))^T R(h),  dW13 = R(bf16([da | db]))^T R(Q(x))
    with R the runs of 128 rows of quantize_token_runs.  Returns (dx, dw13,
    dw2, y)."""
    x, w13q, w2q, dy = _f64(x), _f64(w13q), _f64(w2q), _f64(dy)
    I = w2q.shape[1]
    xq = _q_act(x)
    ab = xq @ w13q.T
    a, b = ab[:, :I], ab[:, I:]
    h = _q_act(silu(a) * b)
    y = h @ w2q.T
    dw2 = fp8_wgrad(round_bf16(dy), h) if fp8_wgrad_products else dy.T @ h
    dh = _q_grad(dy) @ w2q
    ar, br = round_bf16(a), round_bf16(b)
    da = dh * br * silu_grad(ar)
    db = dh * silu(ar)
    dab = np.concatenate([da, db], axis=1)
    dw13 = fp8_wgrad(round_bf16(dab), xq) if fp8_wgrad_products else dab.T @ xq
    dx = _q_grad(dab) @ w13q
    return dx, dw13, dw2, y


def layer_backward(u, e, b, w13, w2, Nr: int, Ns: int, K: int, grad_out, fp8_dgrad: bool = False,
                   fp8_train: bool = False, fp8_wgrad: bool = False) -> LayerGrads:
    """Gradients of L = sum(grad_out * out) for the layer of
    oracle.moe.layer_forward (bf16 / fp32 path, no FP8 quantisation).

    u [T, d], e [N_r, d], b [N_r], w13 [N_r+N_s, 2I, d], w2 [N_r+N_s, d, I],
    grad_out [T, d] = dL/dout.  fp8_dgrad: every expert's backward is
    ffn_backward_fp8 instead of ffn_backward.  fp8_train: the whole FP8
    training step, ffn_backward_fp8_train, with w13 / w2 the decoded E4M3
    weights; the router still sees the unquantised u (R8).  fp8_wgrad (with
    fp8_train only): the weight gradients on E4M3 operands as well (B5), each
    expert's runs of 128 rows counted from its first row."""
    if fp8_wgrad and not fp8_train:
        raise ValueError("layer_backward: fp8_wgrad needs fp8_train")
    if fp8_train:
        ffn_bwd = lambda *a: ffn_backward_fp8_train(*a, fp8_wgrad_products=fp8_wgrad)
    else:
        ffn_bwd = ffn_backward_fp8 if fp8_dgrad else ffn_backward
    u, e, G = _f64(u), _f64(e), _f64(grad_out)
    w13, w2 = _f64(w13), _f64(w2)
    T, d = u.shape
    r = route(u, e, b, K)
    du_ffn = np.zeros((T, d))
    dw13 = np.zeros_like(w13)
    dw2 = np.zeros_like(w2)
    dgate = np.zeros((T, K))

    # shared experts: gate 1 (R7), every token
    for j in range(Ns):
        dx, dw13[Nr + j], dw2[Nr + j], _ = ffn_bwd(u, w13[Nr + j], w2[Nr + j], G)
        du_ffn += dx

    # routed experts: the output gradient reaches FFN_i scaled by the gate;
    # the gate's own gradient is <dL/dout_t, FFN_i(u_t)>
    for i in range(Nr):
        t_sel, k_sel = np.nonzero(r.idx == i)
        if t_sel.size == 0:
            continue
        dy = r.gate[t_sel, k_sel][:, None] * G[t_sel]
        dx, dw13[i], dw2[i], y = ffn_bwd(u[t_sel], w13[i], w2[i], dy)
        np.add.at(du_ffn, t_sel, dx)
        dgate[t_sel, k_sel] = np.sum(G[t_sel] * y, axis=1)

    # gates g_k = s_k / S (R1): dL/ds_k = (dL/dg_k - sum_j g_j dL/dg_j) / S;
    # s = sigmoid(z): dz = ds * s (1 - s); z = u . e_i
    S = np.sum(r.score, axis=1, keepdims=True)
    ds = (dgate - np.sum(r.gate * dgate, axis=1, keepdims=True)) / S
    dz = ds * r.score * (1.0 - r.score)
    du_router = np.zeros((T, d))
    de = np.zeros_like(e)
    for k in range(K):
        du_router += dz[:, k:k + 1] * e[r.idx[:, k]]
        np.add.at(de, r.idx[:, k], dz[:, k:k + 1] * u)

    du = G + du_ffn + du_router         # the residual passes grad_out through
    return LayerGrads(du, de, dw13, dw2, dgate, dz, du_ffn, du_router)
