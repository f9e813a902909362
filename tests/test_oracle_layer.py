"""Pins of the oracle's SwiGLU experts, combine and full layer.

Independent checks: a pure-Python loop evaluation of the FFN and of the whole
layer on tiny shapes, and closed forms (identical routed experts give
u + FFN_s(u) + FFN_r(u) for any routing; W_up = 0 gives u; an FP8 input that
already sits on the E4M3 grid with unit scales is left unchanged).
"""
import math

import numpy as np
import pytest

from oracle import e4m3, moe


def _silu(a):
    return a / (1.0 + math.exp(-a))


def _loop_ffn(x_row, w13, w2):
    I = w2.shape[1]
    d = x_row.shape[0]
    h = []
    for i in range(I):
        a = sum(w13[i, j] * x_row[j] for j in range(d))
        up = sum(w13[I + i, j] * x_row[j] for j in range(d))
        h.append(_silu(a) * up)
    return [sum(w2[o, i] * h[i] for i in range(I)) for o in range(d)]


def test_swiglu_matches_python_loops():
    rng = np.random.default_rng(1)
    d, I, R = 5, 3, 4
    x = rng.normal(size=(R, d))
    w13 = rng.normal(size=(2 * I, d))
    w2 = rng.normal(size=(d, I))
    y, h = moe.swiglu_ffn(x, w13, w2)
    for r in range(R):
        np.testing.assert_allclose(y[r], _loop_ffn(x[r], w13, w2), rtol=1e-12, atol=1e-14)


def test_silu_values():
    a = np.array([0.0, 30.0, -30.0, 1.0])
    h = a * moe.sigmoid(a)
    assert h[0] == 0.0 and abs(h[1] - 30.0) < 1e-9 and abs(h[2]) < 1e-11
    assert abs(h[3] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15


def _tiny(rng, T=12, d=6, Nr=5, Ns=2, I=4, K=2):
    u = rng.normal(size=(T, d))
    e = rng.normal(size=(Nr, d)) / math.sqrt(d)
    b = rng.uniform(-0.05, 0.05, Nr).astype(np.float32)
    w13 = rng.normal(size=(Nr + Ns, 2 * I, d)) / math.sqrt(d)
    w2 = rng.normal(size=(Nr + Ns, d, I)) / math.sqrt(d)
    return u, e, b, w13, w2, Nr, Ns, K


def test_layer_matches_python_loops():
    rng = np.random.default_rng(2)
    u, e, b, w13, w2, Nr, Ns, K = _tiny(rng)
    out = moe.layer_forward(u, e, b, w13, w2, Nr, Ns, K)
    T, d = u.shape
    for t in range(T):
        s = [1 / (1 + math.exp(-sum(u[t, j] * e[i, j] for j in range(d)))) for i in range(Nr)]
        v = [s[i] + float(b[i]) for i in range(Nr)]
        sel = sorted(range(Nr), key=lambda i: (-v[i], i))[:K]
        den = sum(s[i] for i in sel)
        want = list(u[t])
        for j in range(Ns):
            yj = _loop_ffn(u[t], w13[Nr + j], w2[Nr + j])
            want = [a + c for a, c in zip(want, yj)]
        for i in sel:
            yi = _loop_ffn(u[t], w13[i], w2[i])
            want = [a + s[i] / den * c for a, c in zip(want, yi)]
        np.testing.assert_allclose(out.out[t], want, rtol=1e-12, atol=1e-13)
        assert out.routing.idx[t].tolist() == sel


def test_identical_routed_experts_closed_form():
    rng = np.random.default_rng(3)
    u, e, b, w13, w2, Nr, Ns, K = _tiny(rng, T=40, Nr=8, K=3)
    w13[:Nr] = w13[0]
    w2[:Nr] = w2[0]
    want = u.copy()
    for j in range(Ns):
        want += moe.swiglu_ffn(u, w13[Nr + j], w2[Nr + j])[0]
    want += moe.swiglu_ffn(u, w13[0], w2[0])[0]
    for bias in (b, np.zeros_like(b), rng.uniform(-1, 1, Nr).astype(np.float32)):
        out = moe.layer_forward(u, e, bias, w13, w2, Nr, Ns, K)
        np.testing.assert_allclose(out.out, want, rtol=1e-12, atol=1e-12)


def test_zero_up_projection_gives_residual():
    rng = np.random.default_rng(4)
    u, e, b, w13, w2, Nr, Ns, K = _tiny(rng)
    I = w2.shape[2]
    w13[:, I:] = 0.0
    out = moe.layer_forward(u, e, b, w13, w2, Nr, Ns, K)
    assert np.array_equal(out.out, u)


def test_combine_terms_and_flags():
    rng = np.random.default_rng(5)
    u, e, b, w13, w2, Nr, Ns, K = _tiny(rng)
    lo = moe.layer_forward(u, e, b, w13, w2, Nr, Ns, K)
    full = moe.combine(u, lo.y_shared, lo.y_routed, lo.routing.gate)
    np.testing.assert_allclose(full, lo.out, rtol=1e-14, atol=1e-14)
    parts = (moe.combine(u, lo.y_shared, lo.y_routed, lo.routing.gate, shared=False, routed=False)
             + moe.combine(u, lo.y_shared, lo.y_routed, lo.routing.gate, residual=False, routed=False)
             + moe.combine(u, lo.y_shared, lo.y_routed, lo.routing.gate, residual=False, shared=False))
    np.testing.assert_allclose(parts, full, rtol=1e-13, atol=1e-13)
    assert np.array_equal(moe.combine(u, lo.y_shared, lo.y_routed, lo.routing.gate, shared=False, routed=False), u)


def test_fp8_input_on_grid_is_unchanged():
    """x_quant is the identity when every 1x128 tile has amax 448 and all
    values are E4M3 values: the scale is 1 and every code is exact."""
    rng = np.random.default_rng(6)
    T, d = 8, 256
    codes = rng.integers(0, 0x7F, (T, d)).astype(np.uint8) | (rng.integers(0, 2, (T, d)).astype(np.uint8) << 7)
    u = e4m3.e4m3_decode(codes)
    u[:, 0] = 448.0
    u[:, 128] = -448.0
    np.testing.assert_array_equal(moe.quantize_activations(u), u)


def test_fp8_layer_error_is_bounded_by_quantisation():
    rng = np.random.default_rng(7)
    T, d, Nr, Ns, I, K = 16, 256, 4, 1, 128, 2
    u = rng.normal(size=(T, d)).astype(np.float32).astype(np.float64)
    e = rng.normal(size=(Nr, d)) / 16
    b = np.zeros(Nr, np.float32)
    w13 = rng.normal(size=(Nr + Ns, 2 * I, d)) / 16
    w2 = rng.normal(size=(Nr + Ns, d, I)) / 16
    exact = moe.layer_forward(u, e, b, w13, w2, Nr, Ns, K)
    q = moe.layer_forward(u, e, b, w13, w2, Nr, Ns, K, x_quant=True, h_quant=True)
    assert np.array_equal(exact.routing.idx, q.routing.idx)          # router unquantised
    ffn_exact = exact.out - u
    ffn_q = q.out - u
    rel = np.linalg.norm(ffn_q - ffn_exact) / np.linalg.norm(ffn_exact)
    assert 1e-3 < rel < 0.08


@pytest.mark.parametrize("tile_m,tile_rows", [(1, 4), (4, 8), (8, 8), (16, 64)])
def test_layout_matches_python_construction(tile_m, tile_rows):
    rng = np.random.default_rng(tile_m)
    T, Nr, Ns, K = 37, 9, 2, 3
    idx = np.stack([rng.choice(Nr, K, replace=False) for _ in range(T)]).astype(np.int32)
    idx[:, 0] = np.where(rng.random(T) < 0.5, 4, idx[:, 0])          # skew: expert 4 is common
    idx = np.stack([row if len(set(row)) == K else rng.choice(Nr, K, replace=False) for row in idx])
    lay = moe.permute_layout(idx, Nr, Ns, tile_m, tile_rows)
    rows, offs, inv, tiles = [], [], {}, []
    for seg in range(Nr + Ns):
        offs.append(len(rows))
        start = len(rows)
        for t in range(T):
            if seg >= Nr:
                rows.append(t)
            else:
                for k in range(K):
                    if idx[t, k] == seg:
                        inv[(t, k)] = len(rows)
                        rows.append(t)
        while (len(rows) - start) % tile_m:
            rows.append(-1)
        r0 = start
        while r0 < len(rows):
            n = min(tile_rows, len(rows) - r0)
            tiles.append([seg, r0, n, sum(1 for r in rows[r0:r0 + n] if r >= 0)])   # token rows of the tile
            r0 += n
    offs.append(len(rows))
    assert lay.seg_offset.tolist() == offs
    P = offs[-1]
    assert lay.row_token[:P].tolist() == rows
    assert np.all(lay.row_token[P:] == -1)
    assert len(lay.row_token) == moe.permuted_rows_max(T, K, Nr, Ns, tile_m)
    assert all(lay.inv_row[t, k] == inv[(t, k)] for t in range(T) for k in range(K))
    assert lay.tile_map.tolist() == tiles and lay.n_tiles == len(tiles)


def test_expert_rows_in_layout_equal_layer_terms():
    rng = np.random.default_rng(8)
    u, e, b, w13, w2, Nr, Ns, K = _tiny(rng, T=20)
    lo = moe.layer_forward(u, e, b, w13, w2, Nr, Ns, K)
    lay = moe.permute_layout(lo.routing.idx, Nr, Ns, 4, 8)
    y = moe.expert_rows(u, w13, w2, lay, Nr, Ns)
    T = u.shape[0]
    for t in range(T):
        for k in range(K):
            np.testing.assert_allclose(y[lay.inv_row[t, k]], lo.y_routed[t, k], rtol=1e-13, atol=1e-14)
        for j in range(Ns):
            np.testing.assert_allclose(y[lay.seg_offset[Nr + j] + t], lo.y_shared[j, t], rtol=1e-13, atol=1e-14)
    pad = lay.row_token[: lay.seg_offset[-1]] < 0
    assert np.all(y[pad] == 0)
