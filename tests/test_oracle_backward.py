"""Pins of the layer-backward oracle (oracle/backward.py), independent of it:
central finite differences of the oracle forward on a tiny layer, PyTorch
autograd in fp64 through a forward written here from the equations, and
closed forms."""
import numpy as np
import pytest
import torch

from oracle import backward as B
from oracle import moe as O

TINY = dict(T=5, d=12, Nr=5, Ns=1, I=6, K=2)


def tiny_inputs(seed, T, d, Nr, Ns, I, K, scale=1.0):
    rng = np.random.default_rng(seed)
    E = Nr + Ns
    return dict(u=rng.standard_normal((T, d)),
                e=rng.standard_normal((Nr, d)) * scale / np.sqrt(d),
                b=rng.uniform(-0.05, 0.05, Nr),
                w13=rng.standard_normal((E, 2 * I, d)) / np.sqrt(d),
                w2=rng.standard_normal((E, d, I)) / np.sqrt(I),
                G=rng.standard_normal((T, d)))


def loss(p, Nr, Ns, K):
    out = O.layer_forward(p["u"], p["e"], p["b"], p["w13"], p["w2"], Nr, Ns, K).out
    return float(np.sum(p["G"] * out))


def fd_grad(p, name, Nr, Ns, K, eps=1e-6):
    """Central differences of L = sum(G * out) in every coordinate of p[name];
    a coordinate whose perturbation changes the selection is reported as NaN."""
    base_idx = O.route(p["u"], p["e"], p["b"], K).idx
    x = p[name]
    g = np.zeros_like(x)
    for j in np.ndindex(x.shape):
        old = x[j]
        x[j] = old + eps
        ip = O.route(p["u"], p["e"], p["b"], K).idx
        lp = loss(p, Nr, Ns, K)
        x[j] = old - eps
        im = O.route(p["u"], p["e"], p["b"], K).idx
        lm = loss(p, Nr, Ns, K)
        x[j] = old
        same = np.array_equal(ip, base_idx) and np.array_equal(im, base_idx)
        g[j] = (lp - lm) / (2 * eps) if same else np.nan
    return g


@pytest.mark.parametrize("seed", [0, 1])
def test_backward_matches_finite_differences(seed):
    c = TINY
    p = tiny_inputs(seed, **c)
    gr = B.layer_backward(p["u"], p["e"], p["b"], p["w13"], p["w2"], c["Nr"], c["Ns"], c["K"], p["G"])
    for name, got in [("u", gr.du), ("e", gr.de), ("w13", gr.dw13), ("w2", gr.dw2)]:
        want = fd_grad(p, name, c["Nr"], c["Ns"], c["K"])
        ok = np.isfinite(want)
        assert ok.mean() > 0.95, name
        np.testing.assert_allclose(got[ok], want[ok], rtol=1e-6, atol=1e-7, err_msg=name)


def test_bias_has_no_gradient():
    """The bias only moves the selection, which is piecewise constant (B1):
    away from ties the output does not depend on it at all."""
    c = TINY
    p = tiny_inputs(3, **c)
    g = fd_grad(p, "b", c["Nr"], c["Ns"], c["K"])
    ok = np.isfinite(g)
    assert ok.all() and np.all(g[ok] == 0.0)


def torch_forward(u, e, w13, w2, idx, Nr, Ns):
    """The layer forward from the equations, in torch, for a fixed selection
    idx (the top-K decision is not differentiable)."""
    T, d = u.shape
    I = w2.shape[2]
    s = torch.sigmoid(u @ e.T)                              # [T, Nr]
    sel = torch.gather(s, 1, idx)                           # [T, K]
    g = sel / sel.sum(dim=1, keepdim=True)
    out = u.clone()

    def ffn(x, j):
        ab = x @ w13[j].T
        return (torch.nn.functional.silu(ab[:, :I]) * ab[:, I:]) @ w2[j].T

    for j in range(Ns):
        out = out + ffn(u, Nr + j)
    for k in range(idx.shape[1]):
        ys = torch.stack([ffn(u[t:t + 1], int(idx[t, k]))[0] for t in range(T)])
        out = out + g[:, k:k + 1] * ys
    return out


def test_backward_matches_autograd():
    c = dict(T=24, d=32, Nr=12, Ns=1, I=16, K=4)
    p = tiny_inputs(7, **c)
    r = O.route(p["u"], p["e"], p["b"], c["K"])
    gr = B.layer_backward(p["u"], p["e"], p["b"], p["w13"], p["w2"], c["Nr"], c["Ns"], c["K"], p["G"])
    t = {k: torch.tensor(p[k], dtype=torch.float64, requires_grad=True) for k in ["u", "e", "w13", "w2"]}
    out = torch_forward(t["u"], t["e"], t["w13"], t["w2"], torch.tensor(r.idx, dtype=torch.long), c["Nr"], c["Ns"])
    (out * torch.tensor(p["G"])).sum().backward()
    for name, got in [("u", gr.du), ("e", gr.de), ("w13", gr.dw13), ("w2", gr.dw2)]:
        np.testing.assert_allclose(got, t[name].grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=name)


def test_zero_output_gradient_gives_zero():
    c = TINY
    p = tiny_inputs(4, **c)
    gr = B.layer_backward(p["u"], p["e"], p["b"], p["w13"], p["w2"], c["Nr"], c["Ns"], c["K"],
                          np.zeros_like(p["G"]))
    for a in (gr.du, gr.de, gr.dw13, gr.dw2, gr.dgate, gr.dz):
        assert np.all(a == 0.0)


def test_gate_gradient_sums_to_zero_over_a_token():
    """sum_k g_k = 1 for every token, so along the normalisation the score
    gradients ds_k = (dg_k - sum_j g_j dg_j) / S satisfy sum_k s_k ds_k = 0."""
    c = dict(T=16, d=24, Nr=8, Ns=1, I=8, K=3)
    p = tiny_inputs(5, **c)
    r = O.route(p["u"], p["e"], p["b"], c["K"])
    gr = B.layer_backward(p["u"], p["e"], p["b"], p["w13"], p["w2"], c["Nr"], c["Ns"], c["K"], p["G"])
    ds = gr.dz / (r.score * (1 - r.score))
    np.testing.assert_allclose(np.sum(r.score * ds, axis=1), 0.0, atol=1e-12)


# ------------------------------------------------------------------ FP8 --
# fp8_tile_matmul (reading B2) against what the E4M3 format and the tile
# scaling fix, without calling the oracle's quantiser from the test.

def _e4m3_grid_values(rng, shape):
    """Random finite E4M3FN values, decoded from the format's fields here:
    sign, 4-bit exponent (bias 7), 3-bit mantissa; exponent 15 with mantissa
    7 is NaN and left out, exponent 0 is subnormal."""
    e = rng.integers(0, 16, size=shape)
    m = rng.integers(0, 8, size=shape)
    m = np.where((e == 15) & (m == 7), 6, m)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.where(rng.integers(0, 2, size=shape) == 1, -mag, mag)


def _on_grid(rng, rows, cols, tile_rows, tile_cols, kmin=-4, kmax=4):
    """A matrix whose every tile holds E4M3 values times its own 2^k, with one
    entry of magnitude 448 * 2^k, so that the tile's scale is 2^k and every
    entry is a code times the scale."""
    x = _e4m3_grid_values(rng, (rows, cols))
    for r0 in range(0, rows, tile_rows):
        for c0 in range(0, cols, tile_cols):
            k = int(rng.integers(kmin, kmax + 1))
            t = x[r0:r0 + tile_rows, c0:c0 + tile_cols]
            t[rng.integers(0, t.shape[0]), rng.integers(0, t.shape[1])] = 448.0 * (1 if rng.random() < .5 else -1)
            x[r0:r0 + tile_rows, c0:c0 + tile_cols] = t * 2.0 ** k
    return x


def test_fp8_tile_matmul_is_exact_on_the_grid():
    """Operands that the tile quantisation represents exactly give exactly
    the fp64 product.  Each 1x128 tile of g and each 128x128 block of w has
    its own exponent, so tiles taken along the wrong axis, or of the wrong
    size, would mix exponents and round the smaller entries."""
    rng = np.random.default_rng(5)
    g = _on_grid(rng, 48, 384, 1, 128)
    w = _on_grid(rng, 384, 256, 128, 128)
    assert np.array_equal(B.fp8_tile_matmul(g, w), g @ w)
    # the identity is exact in 128x128 blocks, so g comes back unchanged
    assert np.array_equal(B.fp8_tile_matmul(g, np.eye(384)), g)
    # tiles whose scale changes inside a 128x128 block are not exact
    w_bad = w.copy()
    w_bad[:, :128] = _on_grid(rng, 384, 128, 1, 128)  # scales vary inside a 128x128 block
    assert not np.array_equal(B.fp8_tile_matmul(g, w_bad), g @ w_bad)


def test_fp8_tile_matmul_error_within_the_rounding_bound():
    """Random operands: every entry is off by at most half an E4M3 step of
    its tile (relative 2^-4 for normal codes, 2^-10 of the scale below
    2^-6), so each product entry is within sum |g| e_w + e_g |w| + e_g e_w."""
    rng = np.random.default_rng(6)
    g = rng.standard_normal((40, 256)) * np.exp(rng.standard_normal((40, 1)))
    g = g.astype(np.float32).astype(np.float64)        # the operand must be exact in fp32
    w = rng.standard_normal((256, 384)) / 16
    got = B.fp8_tile_matmul(g, w)
    want = g @ w

    def step_bound(x, tile_rows, tile_cols):
        rows, cols = x.shape
        t = np.abs(x).reshape(rows // tile_rows, tile_rows, cols // tile_cols, tile_cols).max(axis=(1, 3))
        s = 2.0 ** np.ceil(np.log2(t / 448.0))          # the smallest 2^k with amax <= 448 * 2^k
        s = np.repeat(np.repeat(s, tile_rows, 0), tile_cols, 1)
        return np.maximum(np.abs(x) * 2.0 ** -4, s * 2.0 ** -10)

    eg, ew = step_bound(g, 1, 128), step_bound(w, 128, 128)
    bound = np.abs(g) @ ew + eg @ np.abs(w) + eg @ ew
    assert np.all(np.abs(got - want) <= bound * (1 + 1e-12) + 1e-300)
    assert np.linalg.norm(got - want) / np.linalg.norm(want) < 0.05


def test_fp8_ffn_backward_weight_gradients_and_closeness():
    """ffn_backward_fp8 keeps the weight gradient of W2 unquantised (equal to
    ffn_backward's), and its input gradient stays within the E4M3 error of
    the exact one."""
    rng = np.random.default_rng(7)
    n, d, I = 64, 256, 128
    x = rng.standard_normal((n, d))
    w13 = rng.standard_normal((2 * I, d)) / np.sqrt(d)
    w2 = rng.standard_normal((d, I)) / np.sqrt(I)
    dy = rng.standard_normal((n, d))
    dx8, dw13_8, dw2_8, y8 = B.ffn_backward_fp8(x, w13, w2, dy)
    dx, dw13, dw2, y = B.ffn_backward(x, w13, w2, dy)
    assert np.array_equal(dw2_8, dw2) and np.array_equal(y8, y)
    rel = lambda a, b: np.linalg.norm(a - b) / np.linalg.norm(b)
    assert rel(dx8, dx) < 0.06 and rel(dw13_8, dw13) < 0.06
    assert rel(dx8, dx) > 1e-4  # the quantisation did happen


def test_fp8_layer_backward_switch():
    """layer_backward(fp8_dgrad=True) changes only what flows through the
    expert input gradients: the gate and score gradients and dW2 are those of
    the exact backward."""
    p = tiny_inputs(3, T=6, d=256, Nr=4, Ns=1, I=128, K=2)
    g = B.layer_backward(p["u"], p["e"], p["b"], p["w13"], p["w2"], 4, 1, 2, p["G"])
    g8 = B.layer_backward(p["u"], p["e"], p["b"], p["w13"], p["w2"], 4, 1, 2, p["G"], fp8_dgrad=True)
    assert np.array_equal(g8.dgate, g.dgate) and np.array_equal(g8.dz, g.dz) and np.array_equal(g8.dw2, g.dw2)
    assert np.array_equal(g8.du_router, g.du_router) and np.array_equal(g8.de, g.de)
    assert not np.array_equal(g8.du_ffn, g.du_ffn)
    assert np.linalg.norm(g8.du - g.du) / np.linalg.norm(g.du) < 0.05


def test_fp8_train_step_forward_is_the_fp8_forward():
    """The forward inside ffn_backward_fp8_train is the FP8 forward oracle
    (x and h in 1x128 tiles, R8), and the layer gradients of the FP8 training
    step use its outputs for the gate gradients."""
    p = tiny_inputs(4, T=6, d=256, Nr=4, Ns=1, I=128, K=2)
    w13q = np.stack([O.quantize_activations(w) for w in p["w13"]])   # any fixed weights will do here
    w2q = np.stack([O.quantize_activations(w) for w in p["w2"]])
    f = O.layer_forward(p["u"], p["e"], p["b"], w13q, w2q, 4, 1, 2, x_quant=True, h_quant=True)
    g = B.layer_backward(p["u"], p["e"], p["b"], w13q, w2q, 4, 1, 2, p["G"], fp8_train=True)
    dgate = np.einsum("td,tkd->tk", p["G"], f.y_routed)
    assert np.allclose(g.dgate, dgate, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------- exact pins --
# The FP8 backward variants against fp64 PyTorch autograd.  The readings are
# built into the autograd graph with three devices of its own, none of which
# restates the oracle's derivative formulas:
#   st_q(t)     value Q(t), gradient the identity (a straight-through
#               quantiser of the forward, B3);
#   GradQ       value t, gradient Q(bf16(dL/dt)) (the gradient operand of an
#               E4M3 input-gradient product, B2 and B4);
#   at_bf16(t)  value bf16(t), gradient the identity, so that autograd's own
#               derivative of the SwiGLU is taken at the stored bf16
#               pre-activations (B4) while the forward value stays exact.
# A product whose two gradients differ (dW from the unquantised gradient, dX
# from the quantised one times the E4M3 weight Wq) is split as
# X.detach() W^T + GradQ(X Wq^T) - (X Wq^T).detach(): its value is X W^T,
# autograd sends dL/dY to dW and Q(bf16(dL/dY)) Wq to dX.

def _q_tiles(a: np.ndarray, rows: int = 1) -> np.ndarray:
    from oracle.e4m3 import dequantize_tiles, quantize_tiles
    return dequantize_tiles(*quantize_tiles(a.astype(np.float32), rows, 128), rows, 128)


def _bf16(a: np.ndarray) -> np.ndarray:
    """torch's own bf16 rounding (independent of oracle.backward.round_bf16)."""
    return torch.from_numpy(np.asarray(a, dtype=np.float64)).float().to(torch.bfloat16).double().numpy()


class GradQ(torch.autograd.Function):
    @staticmethod
    def forward(ctx, t):
        return t.view_as(t)

    @staticmethod
    def backward(ctx, g):
        return torch.from_numpy(_q_tiles(_bf16(g.numpy())))


def st_q(t):
    return t + (torch.from_numpy(_q_tiles(t.detach().numpy())) - t).detach()


def at_bf16(t):
    return t + (torch.from_numpy(_bf16(t.detach().numpy())) - t).detach()


def _split_product(x, w, wq):
    return x.detach() @ w.T + GradQ.apply(x @ wq.T) - (x @ wq.T).detach()


def _autograd_ffn(x, w13, w2, dy, train: bool):
    """(dx, dW13, dW2, y) of one expert by autograd; train: the FP8 training
    step (forward quantisers st_q on x and h), else the bf16 forward."""
    I = w2.shape[1]
    xt = torch.tensor(x, requires_grad=True)
    W13 = torch.tensor(w13, requires_grad=True)
    W2 = torch.tensor(w2, requires_grad=True)
    W13q = torch.from_numpy(_q_tiles(w13, 128))   # the E4M3 weights of the dgrad products
    W2q = torch.from_numpy(_q_tiles(w2, 128))
    xin = st_q(xt) if train else xt
    ab = _split_product(xin, W13, W13q)
    a, b = ab[:, :I], ab[:, I:]
    h_val = (a * torch.sigmoid(a) * b).detach()
    if train:
        h_val = torch.from_numpy(_q_tiles(h_val.numpy()))
    ar, br = at_bf16(a), at_bf16(b)
    h_r = ar * torch.sigmoid(ar) * br
    h = h_val + (h_r - h_r.detach())      # value h (Q(h) in training); gradient at bf16(a), bf16(b)
    y = _split_product(h, W2, W2q)
    (y * torch.from_numpy(dy)).sum().backward()
    return xt.grad.numpy(), W13.grad.numpy(), W2.grad.numpy(), y.detach().numpy()


def _assert_same(got, want, name):
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-13 * np.abs(want).max(), err_msg=name)


@pytest.mark.parametrize("seed", [8, 9])
def test_fp8_train_step_gradients_equal_autograd(seed):
    """ffn_backward_fp8_train: forward Q(x), Q(h) (R8); quantisers straight
    through (B3: dW13 = [da | db]^T Q(x), dW2 = dy^T Q(h)); E4M3 input-gradient
    products (B2) of bf16 gradients; SwiGLU backward at the bf16
    pre-activations (B4).  Equal to fp64 autograd of that graph."""
    rng = np.random.default_rng(seed)
    n, d, I = 16, 256, 128
    x = _bf16(rng.standard_normal((n, d)))
    w13q = O.quantize_activations(rng.standard_normal((2 * I, d)) / 16)   # E4M3 values, any fixed tiling
    w2q = O.quantize_activations(rng.standard_normal((d, I)) / 16)
    w13q, w2q = _q_tiles(w13q, 128), _q_tiles(w2q, 128)                  # on the 128x128-block grid
    dy = _bf16(rng.standard_normal((n, d)) * 0.3)
    dx, dw13, dw2, y = B.ffn_backward_fp8_train(x, w13q, w2q, dy)
    gx, g13, g2, yt = _autograd_ffn(x, w13q, w2q, dy, train=True)
    np.testing.assert_allclose(y, yt, rtol=1e-12, atol=1e-12)
    _assert_same(dw2, g2, "dW2")
    _assert_same(dw13, g13, "dW13")
    _assert_same(dx, gx, "dx")


def test_fp8_dgrad_gradients_equal_autograd():
    """ffn_backward_fp8 (bf16 forward, E4M3 input-gradient products on the
    weights' 128x128 blocks): the same graph without the forward
    quantisers."""
    rng = np.random.default_rng(10)
    n, d, I = 24, 256, 128
    x = _bf16(rng.standard_normal((n, d)))
    w13 = _bf16(rng.standard_normal((2 * I, d)) / 16)
    w2 = _bf16(rng.standard_normal((d, I)) / 16)
    dy = _bf16(rng.standard_normal((n, d)) * 0.3)
    dx, dw13, dw2, y = B.ffn_backward_fp8(x, w13, w2, dy)
    gx, g13, g2, yt = _autograd_ffn(x, w13, w2, dy, train=False)
    np.testing.assert_allclose(y, yt, rtol=1e-12, atol=1e-12)
    _assert_same(dw2, g2, "dW2")
    _assert_same(dw13, g13, "dW13")
    _assert_same(dx, gx, "dx")


def test_fp8_train_step_plausible_mistakes_fail_the_pin():
    """Each reading of the FP8 training step is visible to the autograd pin:
    the unquantised x in dW13, quantising from fp32 instead of bf16, and the
    SwiGLU backward at the fp64 pre-activations all move the gradients by
    more than its tolerance."""
    rng = np.random.default_rng(11)
    n, d, I = 16, 256, 128
    x = _bf16(rng.standard_normal((n, d)))
    w13q = _q_tiles(O.quantize_activations(rng.standard_normal((2 * I, d)) / 16), 128)
    w2q = _q_tiles(O.quantize_activations(rng.standard_normal((d, I)) / 16), 128)
    dy = _bf16(rng.standard_normal((n, d)) * 0.3)
    gx, g13, g2, _ = _autograd_ffn(x, w13q, w2q, dy, train=True)
    xq = _q_tiles(x)
    ab = xq @ w13q.T
    a, b = ab[:, :I], ab[:, I:]
    dh = _q_tiles(_bf16(dy)) @ w2q
    far = lambda got, want: np.max(np.abs(got - want)) > 1e-6 * np.abs(want).max()
    # dW13 from the unquantised rows
    ar, br = _bf16(a), _bf16(b)
    dab = np.concatenate([dh * br * B.silu_grad(ar), dh * B.silu(ar)], axis=1)
    assert far(dab.T @ x, g13) and not far(dab.T @ xq, g13)
    # the SwiGLU backward at the fp64 pre-activations
    dab64 = np.concatenate([dh * b * B.silu_grad(a), dh * B.silu(a)], axis=1)
    assert far(dab64.T @ xq, g13)
    # [da | db] quantised from fp32 instead of bf16
    assert far(_q_tiles(dab) @ w13q, gx) and not far(_q_tiles(_bf16(dab)) @ w13q, gx)


def test_round_bf16_matches_torch_and_hand_cases():
    """round_bf16 against torch's bf16 cast (an independent routine) over
    normal, subnormal and tie values, and hand-worked ties: 1 + 2^-8 sits
    halfway between 1 and 1 + 2^-7 and goes to the even 1; 1 + 3*2^-8 sits
    halfway between 1 + 2^-7 and 1 + 2^-6 and goes to the even 1 + 2^-6."""
    rng = np.random.default_rng(12)
    x = np.concatenate([rng.standard_normal(20000) * np.exp2(rng.integers(-140, 120, 20000)),
                        (1 + rng.integers(0, 2 ** 16, 4000) * 2.0 ** -16) * np.exp2(rng.integers(-130, 100, 4000)),
                        (rng.integers(0, 2 ** 8, 4000) * 2 + 1) * 2.0 ** -8])
    x = x.astype(np.float32).astype(np.float64)
    want = torch.from_numpy(x).float().to(torch.bfloat16).double().numpy()
    assert np.array_equal(B.round_bf16(x), want)
    assert B.round_bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0
    assert B.round_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6
    assert B.round_bf16(np.array([-(1 + 3 * 2.0 ** -8)]))[0] == -(1 + 2.0 ** -6)
    assert B.round_bf16(np.array([1 + 2.0 ** -8 + 2.0 ** -20]))[0] == 1 + 2.0 ** -7


# ------------------------------------------------- E4M3 weight gradients --
# Reading B5: both operands of a weight gradient in E4M3 runs of 128 rows
# (the token axis) per column.  The pins below use a quantiser written here
# by exhaustive search over the format's values, not the oracle's codec.

def _e4m3_magnitudes() -> np.ndarray:
    """Every finite non-negative E4M3FN value, indexed by its 7-bit code,
    from the fields: exponent code >> 3 (bias 7, 0 subnormal), mantissa
    code & 7; code 127 is NaN."""
    return np.array([(c & 7) / 8.0 * 2.0 ** -6 if c >> 3 == 0 else (1 + (c & 7) / 8.0) * 2.0 ** ((c >> 3) - 7)
                     for c in range(127)])


_MAGS = _e4m3_magnitudes()


def _search_scale(amax: float) -> float:
    if amax == 0.0:
        return 1.0
    k = -126
    while amax > 448.0 * 2.0 ** k:
        k += 1
    return 2.0 ** k


def _nearest_e4m3(v: np.ndarray) -> np.ndarray:
    """Each |v| <= 448 to the nearest E4M3 value by exhaustive search; of two
    equally near values the one with the even code (mantissa bit 0 clear)."""
    dist = np.abs(np.abs(v)[:, None] - _MAGS[None, :])
    best = dist.min(axis=1, keepdims=True)
    tie_ok = (dist == best) & (np.arange(127)[None, :] % 2 == 0)
    only = (dist == best).sum(axis=1) == 1
    code = np.where(only, np.argmin(dist, axis=1), np.argmax(tie_ok, axis=1))
    return np.copysign(_MAGS[code], v)


def _search_token_runs(m: np.ndarray) -> np.ndarray:
    """Runs of 128 rows per column, each scaled by its own searched power of
    two, rounded by exhaustive search, decoded."""
    m = np.asarray(m, dtype=np.float64)
    out = np.zeros_like(m)
    for c in range(m.shape[1]):
        for r0 in range(0, m.shape[0], 128):
            run = m[r0:r0 + 128, c]
            s = _search_scale(float(np.abs(run).max()))
            out[r0:r0 + 128, c] = _nearest_e4m3(run / s) * s
    return out


def test_token_runs_match_exhaustive_search():
    """quantize_token_runs against the searched quantiser: 300 rows (runs of
    128, 128 and 44), columns of very different magnitude, exact zeros, a
    zero column, and values halfway between two E4M3 values of their run."""
    rng = np.random.default_rng(20)
    m = rng.standard_normal((300, 7)) * np.exp2(rng.integers(-20, 20, (1, 7)))
    m[:, 3] = 0.0
    m[5:9, 1] = 0.0
    m[128, 2] = 448.0 * 2.0 ** -3          # run 2 of column 2: scale 2^-3
    m[129:140, 2] = np.array([1.0625, 1.1875, 3.125, 0.5 + 2.0 ** -5, 2.0 ** -9 * 1.5, 2.0 ** -9 * 0.5, 13.5, 26.0,
                              -1.0625, -3.125, 200.0]) * 2.0 ** -3   # midpoints at that scale (26: on the grid)
    m = m.astype(np.float32).astype(np.float64)
    got = B.quantize_token_runs(m)
    want = _search_token_runs(m)
    assert np.array_equal(got, want)
    assert np.all(got[:, 3] == 0.0)
    # ties went to the even neighbour (mantissa field even): 1.0625 -> 1,
    # 1.1875 -> 1.25, 3.125 -> 3, 0.53125 -> 0.5, 1.5 * 2^-9 -> 2^-8,
    # 0.5 * 2^-9 -> 0, 13.5 -> 14, 200 -> 192
    assert list(got[129:140, 2] * 8) == [1.0, 1.25, 3.0, 0.5, 2.0 ** -8, 0.0, 14.0, 26.0, -1.0, -3.0, 192.0]
    assert B.quantize_token_runs(np.zeros((0, 5))).shape == (0, 5)


def _on_grid_runs(rng, rows, cols, kmin=-6, kmax=6):
    """Every run of 128 rows of every column holds E4M3 values times its own
    2^k and one entry of magnitude 448 * 2^k: the run's scale is 2^k and the
    quantiser is the identity on it."""
    x = _e4m3_grid_values(rng, (rows, cols))
    for c in range(cols):
        for r0 in range(0, rows, 128):
            run = x[r0:r0 + 128, c]
            run[rng.integers(0, run.size)] = 448.0 if rng.random() < .5 else -448.0
            x[r0:r0 + 128, c] = run * 2.0 ** int(rng.integers(kmin, kmax + 1))
    return x


def test_fp8_wgrad_is_exact_on_the_grid():
    """Operands on the grid of their runs give exactly the fp64 product.  The
    exponent changes from run to run and from column to column, so runs cut
    along the columns, of another length, or not restarted at row 0 would mix
    exponents and round the smaller entries."""
    rng = np.random.default_rng(21)
    a = _on_grid_runs(rng, 300, 40)
    b = _on_grid_runs(rng, 300, 24)
    assert np.array_equal(B.fp8_wgrad(a, b), a.T @ b)
    # one run shifted by a row: its scale no longer holds for the row that moved in
    shifted = np.concatenate([np.zeros((1, 40)), a[:-1]])
    shifted[0] = a[-1]
    assert not np.array_equal(B.quantize_token_runs(shifted), shifted)


def test_fp8_wgrad_error_within_the_rounding_bound():
    """Random operands (fp32-exact, per-row outliers): each entry is off by
    at most half an E4M3 step of its run, so each product entry is within
    |a|^T e_b + e_a^T |b| + e_a^T e_b."""
    rng = np.random.default_rng(22)
    a = (rng.standard_normal((333, 48)) * np.exp(2 * rng.standard_normal((333, 1)))).astype(np.float32).astype(
        np.float64)
    b = (rng.standard_normal((333, 40)) / 16).astype(np.float32).astype(np.float64)
    got = B.fp8_wgrad(a, b)
    want = a.T @ b

    def step_bound(x):
        e = np.zeros_like(x)
        for c in range(x.shape[1]):
            for r0 in range(0, x.shape[0], 128):
                run = x[r0:r0 + 128, c]
                s = _search_scale(float(np.abs(run).max()))
                e[r0:r0 + 128, c] = np.maximum(np.abs(run) * 2.0 ** -4, s * 2.0 ** -10)
        return e

    ea, eb = step_bound(a), step_bound(b)
    bound = np.abs(a).T @ eb + ea.T @ np.abs(b) + ea.T @ eb
    assert np.all(np.abs(got - want) <= bound * (1 + 1e-12) + 1e-300)
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    assert 1e-4 < rel < 0.05


class GradQRuns(torch.autograd.Function):
    """value t, gradient R(bf16(dL/dt)): the gradient operand of an E4M3
    weight-gradient product, in runs of 128 rows (B5, B4)."""
    @staticmethod
    def forward(ctx, t):
        return t.view_as(t)

    @staticmethod
    def backward(ctx, g):
        return torch.from_numpy(_search_token_runs(_bf16(g.numpy())))


def _split_product_w8(x, w, wq):
    """Value x wq^T; dW = R(bf16(dY))^T R(x), dX = Q(bf16(dY)) wq."""
    xr = torch.from_numpy(_search_token_runs(x.detach().numpy()))
    p1 = GradQRuns.apply(xr @ w.T)
    return GradQ.apply(x @ wq.T) + p1 - p1.detach()


def _autograd_ffn_w8(x, w13, w2, dy):
    """_autograd_ffn(train=True) with both weight gradients on E4M3 runs."""
    I = w2.shape[1]
    xt = torch.tensor(x, requires_grad=True)
    W13 = torch.tensor(w13, requires_grad=True)
    W2 = torch.tensor(w2, requires_grad=True)
    W13q = torch.from_numpy(_q_tiles(w13, 128))
    W2q = torch.from_numpy(_q_tiles(w2, 128))
    ab = _split_product_w8(st_q(xt), W13, W13q)
    a, b = ab[:, :I], ab[:, I:]
    h_val = torch.from_numpy(_q_tiles((a * torch.sigmoid(a) * b).detach().numpy()))
    ar, br = at_bf16(a), at_bf16(b)
    h_r = ar * torch.sigmoid(ar) * br
    h = h_val + (h_r - h_r.detach())
    y = _split_product_w8(h, W2, W2q)
    (y * torch.from_numpy(dy)).sum().backward()
    return xt.grad.numpy(), W13.grad.numpy(), W2.grad.numpy(), y.detach().numpy()


@pytest.mark.parametrize("n", [200, 77])
def test_fp8_wgrad_train_step_equals_autograd(n):
    """ffn_backward_fp8_train(fp8_wgrad_products=True) against fp64 autograd
    of the training step's graph with both weight-gradient products on runs of
    128 rows (B5): dW2 = R(bf16(dy))^T R(Q(h)), dW13 = R(bf16([da | db]))^T
    R(Q(x)); dx and y as without (B2-B4)."""
    rng = np.random.default_rng(23 + n)
    d, I = 256, 128
    x = _bf16(rng.standard_normal((n, d)))
    w13q = _q_tiles(O.quantize_activations(rng.standard_normal((2 * I, d)) / 16), 128)
    w2q = _q_tiles(O.quantize_activations(rng.standard_normal((d, I)) / 16), 128)
    dy = _bf16(rng.standard_normal((n, d)) * 0.3 * np.exp(rng.standard_normal((n, 1))))
    dx, dw13, dw2, y = B.ffn_backward_fp8_train(x, w13q, w2q, dy, fp8_wgrad_products=True)
    gx, g13, g2, yt = _autograd_ffn_w8(x, w13q, w2q, dy)
    np.testing.assert_allclose(y, yt, rtol=1e-12, atol=1e-12)
    _assert_same(dw2, g2, "dW2")
    _assert_same(dw13, g13, "dW13")
    _assert_same(dx, gx, "dx")
    # the quantisation of the weight-gradient operands did happen
    dx0, dw13_0, dw2_0, _ = B.ffn_backward_fp8_train(x, w13q, w2q, dy)
    far = lambda p, q: np.max(np.abs(p - q)) > 1e-6 * np.abs(q).max()
    assert far(dw2, dw2_0) and far(dw13, dw13_0) and np.array_equal(dx, dx0)


def test_fp8_wgrad_plausible_mistakes_fail_the_pin():
    """Runs of 128 along the columns instead of the rows, and the gradient
    operand quantised from fp32 instead of bf16, both move dW2 past the
    autograd pin's tolerance."""
    rng = np.random.default_rng(24)
    n, d, I = 200, 256, 128
    dy = rng.standard_normal((n, d)) * 0.3 * np.exp(rng.standard_normal((n, 1)))
    h = _q_tiles(rng.standard_normal((n, I)) * np.exp(rng.standard_normal((n, 1))))
    want = _search_token_runs(_bf16(dy)).T @ _search_token_runs(h)
    assert np.array_equal(B.fp8_wgrad(B.round_bf16(dy), h), want)
    far = lambda p, q: np.max(np.abs(p - q)) > 1e-6 * np.abs(q).max()
    along_cols = _q_tiles(_bf16(dy)).T @ _q_tiles(h)
    assert far(along_cols, want)
    from_f32 = _search_token_runs(dy.astype(np.float32).astype(np.float64)).T @ _search_token_runs(h)
    assert far(from_f32, want)


def test_fp8_wgrad_layer_switch():
    """layer_backward(fp8_train, fp8_wgrad) changes dW13 and dW2 only; each
    expert's runs start at its own first row (an expert with more than 128
    rows checked against the single-expert function); fp8_wgrad alone is
    refused."""
    p = tiny_inputs(25, T=300, d=256, Nr=2, Ns=1, I=128, K=1)
    w13q = np.stack([_q_tiles(O.quantize_activations(w), 128) for w in p["w13"]])
    w2q = np.stack([_q_tiles(O.quantize_activations(w), 128) for w in p["w2"]])
    g = B.layer_backward(p["u"], p["e"], p["b"], w13q, w2q, 2, 1, 1, p["G"], fp8_train=True)
    g8 = B.layer_backward(p["u"], p["e"], p["b"], w13q, w2q, 2, 1, 1, p["G"], fp8_train=True, fp8_wgrad=True)
    for name in ("du", "de", "dgate", "dz", "du_ffn", "du_router"):
        assert np.array_equal(getattr(g8, name), getattr(g, name)), name
    assert not np.array_equal(g8.dw13, g.dw13) and not np.array_equal(g8.dw2, g.dw2)
    r = O.route(p["u"], p["e"], p["b"], 1)
    for i in range(2):
        t_sel = np.nonzero(r.idx[:, 0] == i)[0]
        if t_sel.size > 128:
            dy = r.gate[t_sel, 0][:, None] * p["G"][t_sel]
            _, dw13, dw2, _ = B.ffn_backward_fp8_train(p["u"][t_sel], w13q[i], w2q[i], dy, fp8_wgrad_products=True)
            assert np.array_equal(g8.dw13[i], dw13) and np.array_equal(g8.dw2[i], dw2)
            break
    else:
        pytest.fail("no expert with more than 128 rows")
    with pytest.raises(ValueError):
        B.layer_backward(p["u"], p["e"], p["b"], w13q, w2q, 2, 1, 1, p["G"], fp8_wgrad=True)
