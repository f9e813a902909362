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
    w = rng.standard_normal((256, 384)) / 16
    got = B.fp8_tile_matmul(g, w)
    want = g @ w

    def step_bound(x, tile_rows, tile_cols):
        rows, cols = x.shape
        t = np.abs(x).reshape(rows // tile_rows, tile_rows, cols // tile_cols, tile_cols).max(axis=(1, 3))
        s = 2.0 ** np.ceil(np.log2(t / 448.0))          # the smallest 2^k with amax <= 448 * 2^k
        s = np.repeat(np.repeat(s, tile_rows, 0), tile_cols, 1)
        return np.maximum(np.abs(x) * 2.0 ** -4, s * 2.0 ** -10)

    eg, ew = step_bound(g.astype(np.float32).astype(np.float64), 1, 128), step_bound(w, 128, 128)
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


def test_fp8_train_step_straight_through_gradients():
    """With quantisers treated as the identity (B3) the FP8 training step's
    gradients equal the fp64 autograd gradients of the same function in which
    each quantiser's output is a constant offset added to its input: checked
    here by torch autograd with Q(z) = z + (Q(z) - z).detach()."""
    rng = np.random.default_rng(8)
    n, d, I = 16, 256, 128
    x = rng.standard_normal((n, d))
    w13q = O.quantize_activations(rng.standard_normal((2 * I, d)) / 16)
    w2q = O.quantize_activations(rng.standard_normal((d, I)) / 16)
    dy = rng.standard_normal((n, d))
    dx, dw13, dw2, y = B.ffn_backward_fp8_train(x, w13q, w2q, dy)

    def q(t):   # forward value of the oracle's quantiser, gradient of the identity
        return t + (torch.from_numpy(O.quantize_activations(t.detach().numpy().astype(np.float32))) - t).detach()

    xt = torch.tensor(x, requires_grad=True)
    W13 = torch.tensor(w13q, requires_grad=True)
    W2 = torch.tensor(w2q, requires_grad=True)
    ab = q(xt) @ W13.T
    a, b = ab[:, :I], ab[:, I:]
    h = q(a * torch.sigmoid(a) * b)
    yt = h @ W2.T
    assert np.allclose(yt.detach().numpy(), y, rtol=1e-12, atol=1e-12)
    (yt * torch.from_numpy(dy)).sum().backward()
    # dW2 and the exact dW13 of this function (through Q(x)) vs the oracle's
    assert np.allclose(W2.grad.numpy(), dw2, rtol=1e-10, atol=1e-10)
    # the oracle's dW13 reads the unquantised x (B3) and its dx quantises the
    # gradients (B2): both differ from straight-through autograd by E4M3 error only
    rel = lambda u_, v: np.linalg.norm(u_ - v) / np.linalg.norm(v)
    assert rel(dw13, W13.grad.numpy()) < 0.05
    assert rel(dx, xt.grad.numpy()) < 0.08
