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
