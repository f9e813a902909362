"""Plain fp64 CPU oracle of the DeepSeekMoE layer forward (test infrastructure).

THIS IS TEST INFRASTRUCTURE.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it.  It shares no code, header, table
or constant generator with the HIP library, and the product path never calls
it.  It is slow on purpose: every step is the plain definition, in fp64,
with NumPy primitives (matmul, sort) as the only library help.

Sources (web pages about the DeepSeek-V3 Technical Report)
----------------------------------------------------------
[RG-MoE]  "DeepSeek-V3 Technical Report" reading guide (xyznot.com; Turkish
          edition "Okuma rehberi", French edition "Guide de lecture"), Method
          section 2, "DeepSeekMoE with auxiliary-loss-free balancing".  It
          prints: the layer output h'_t = u_t + sum over shared experts of
          FFN^(s)(u_t) + sum over routed experts of g_{i,t} FFN^(r)_i(u_t)
          (the "combine equation"); the affinity s_{i,t} = Sigmoid(u_t^T e_i)
          and the sentence that the gates g are obtained by normalising g'
          (the "affinity sentence"); g'_{i,t} = s_{i,t} when s_{i,t} + b_i is
          among the Topk of {s_{j,t} + b_j}, else 0 (the "gate equation"); and
          the end-of-step update b_i <- b_i - gamma for an overloaded expert,
          b_i <- b_i + gamma for an underloaded one, gamma = 0.001 (the
          "bias rule").
[RG-Key]  same page, section "Key ideas": 1 shared + 256 routed experts with 8
          active; FP8 with 1x128 activation tiles and 128x128 weight blocks.
[Blog-MoE] "DeepSeek 알고 아는 척 좀 해보자 – 단편: 671B 파라미터의 괴물,
          DeepSeek-V3" (machineindeep.tistory.com), section "DeepSeekMoE &
          load balancing": shared plus routed experts, each token activates
          its top-K routed experts, and no token is dropped.

Readings where the pages leave a step open (each used below):
  R1 gate normalisation: g = g' / sum_j g'_j over the selected experts.
  R2 top-K order and ties: experts ordered by (s+b descending, index
     ascending); an exact tie goes to the lower index.
  R3 "overloaded/underloaded": compare the load c_i with the mean T*K/N_r by
     the exact integer test N_r*c_i vs T*K; equal means unchanged.
  R4 "end of the step": loads come from the tokens of this forward, routed
     with the pre-update bias; one update per step.
  R5 bias precision: b is fp32 state; the update is one fp32 add.
  R6 FFN form: SwiGLU, FFN(x) = W_down (SiLU(W_gate x) * (W_up x)),
     SiLU(a) = a * sigmoid(a), no biases; W13 holds gate rows then up rows.
  R7 shared experts carry gate 1; the output includes the residual u_t.
  R8 FP8 (when used): u is quantised once per token in 1x128 tiles, h in
     1x128 tiles after it is rounded to fp32, weights come as 128x128-block
     codes and scales; the router stays fp32 (here fp64).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .e4m3 import dequantize_tiles, quantize_tiles

GAMMA = 0.001   # [RG-MoE] bias rule


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# Routing: affinity, selection, gates, loads
# --------------------------------------------------------------------------

def sigmoid(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def affinity(u: np.ndarray, e: np.ndarray) -> np.ndarray:
    """s_{i,t} = Sigmoid(u_t . e_i) for every token and routed expert
    ([RG-MoE] affinity sentence).  u [T, d], e [N_r, d] -> s [T, N_r]."""
    return sigmoid(_f64(u) @ _f64(e).T)


@dataclass
class Routing:
    idx: np.ndarray        # [T, K] int32, ordered by (s+b desc, index asc)   (R2)
    gate: np.ndarray       # [T, K] fp64, g = s / sum of selected s          (R1)
    score: np.ndarray      # [T, K] fp64, s of the selected experts
    load: np.ndarray       # [N_r] int64, tokens that selected each expert
    s: np.ndarray          # [T, N_r] fp64 affinities
    v: np.ndarray          # [T, N_r] fp64 selection keys s + b
    boundary_gap: np.ndarray  # [T] v_(K) - v_(K+1) (inf when K == N_r)
    inner_gap: np.ndarray     # [T, K-1] v_(k) - v_(k+1) inside the selection


def route(u: np.ndarray, e: np.ndarray, b: np.ndarray, K: int) -> Routing:
    """Sigmoid routing with a bias that steers selection but not the gate.

    [RG-MoE] affinity sentence and gate equation: the selection uses s + b,
    the kept value g' is s itself; gates are g'/sum g' (R1)."""
    s = affinity(u, e)
    Nr = s.shape[1]
    if not 1 <= K <= Nr:
        raise ValueError("K out of range")
    v = s + _f64(b)[None, :]
    order = np.argsort(-v, axis=1, kind="stable")
    idx = order[:, :K]
    score = np.take_along_axis(s, idx, axis=1)
    gate = score / score.sum(axis=1, keepdims=True)
    load = np.bincount(idx.ravel(), minlength=Nr).astype(np.int64)
    vs = np.take_along_axis(v, order, axis=1)
    boundary = vs[:, K - 1] - vs[:, K] if K < Nr else np.full(s.shape[0], np.inf)
    inner = vs[:, : K - 1] - vs[:, 1:K]
    return Routing(idx.astype(np.int32), gate, score, load, s, v, boundary, inner)


def bias_update(b: np.ndarray, load: np.ndarray, T: int, K: int, gamma: float = GAMMA) -> np.ndarray:
    """End-of-step bias rule ([RG-MoE] bias rule, readings R3-R5).

    Expert i is overloaded when N_r*c_i > T*K (load above the mean T*K/N_r):
    b_i <- b_i - gamma; underloaded when N_r*c_i < T*K: b_i <- b_i + gamma;
    unchanged on equality.  b and gamma are fp32, the add is one fp32 add."""
    b32 = np.asarray(b, dtype=np.float32)
    g32 = np.float32(gamma)
    load = np.asarray(load, dtype=np.int64)
    Nr = load.shape[0]
    mean_x_nr = np.int64(T) * np.int64(K)
    out = b32.copy()
    over = Nr * load > mean_x_nr
    under = Nr * load < mean_x_nr
    out[over] = b32[over] - g32
    out[under] = b32[under] + g32
    return out


# --------------------------------------------------------------------------
# Expert FFN and the layer
# --------------------------------------------------------------------------

def swiglu_ffn(x: np.ndarray, w13: np.ndarray, w2: np.ndarray, h_quant: bool = False):
    """One expert FFN on rows x (reading R6).

    x [R, d]; w13 [2I, d] (gate rows 0..I-1, then up rows I..2I-1);
    w2 [d, I].  Returns (y [R, d], h [R, I]).  With h_quant the hidden state
    is rounded to fp32 and passed through 1x128 E4M3 quantisation (R8)."""
    x, w13, w2 = _f64(x), _f64(w13), _f64(w2)
    I = w2.shape[1]
    a = x @ w13[:I].T
    up = x @ w13[I:].T
    h = a * sigmoid(a) * up
    if h_quant:
        codes, sc = quantize_tiles(h.astype(np.float32), 1, 128)
        h = dequantize_tiles(codes, sc, 1, 128)
    return h @ w2.T, h


@dataclass
class LayerOut:
    out: np.ndarray          # [T, d] h'_t
    routing: Routing
    y_routed: np.ndarray     # [T, K, d] ungated FFN^(r)_{idx[t,k]}(u_t)
    y_shared: np.ndarray     # [Ns, T, d] FFN^(s)_j(u_t)
    new_bias: np.ndarray     # [N_r] fp32 after one bias rule application


def quantize_activations(u: np.ndarray) -> np.ndarray:
    """u as the FP8 path sees it: 1x128 tiles, E4M3 codes times fp32 scale (R8)."""
    codes, sc = quantize_tiles(np.asarray(u, dtype=np.float32), 1, 128)
    return dequantize_tiles(codes, sc, 1, 128)


def layer_forward(u, e, b, w13, w2, Nr: int, Ns: int, K: int,
                  x_quant: bool = False, h_quant: bool = False,
                  gamma: float = GAMMA) -> LayerOut:
    """DeepSeekMoE layer forward ([RG-MoE] combine equation).

    u [T, d]: token hidden states (stored values, widened exactly).
    e [N_r, d] centroids, b [N_r] bias (fp32 values).
    w13 [N_r+N_s, 2I, d], w2 [N_r+N_s, d, I]: experts 0..N_r-1 routed,
    N_r..N_r+N_s-1 shared; values as stored (fp8 weights already decoded as
    code x block scale).
    x_quant / h_quant select the FP8 activation quantisation points (R8).
    The router always sees the unquantised u (R8).
    """
    u = _f64(u)
    T, d = u.shape
    r = route(u, e, b, K)
    x = quantize_activations(u) if x_quant else u

    y_shared = np.zeros((Ns, T, d))
    for j in range(Ns):
        y_shared[j], _ = swiglu_ffn(x, w13[Nr + j], w2[Nr + j], h_quant)

    y_routed = np.zeros((T, K, d))
    for i in range(Nr):
        t_sel, k_sel = np.nonzero(r.idx == i)
        if t_sel.size:
            y_routed[t_sel, k_sel], _ = swiglu_ffn(x[t_sel], w13[i], w2[i], h_quant)

    out = u + y_shared.sum(axis=0) + np.einsum("tk,tkd->td", r.gate, y_routed)
    return LayerOut(out, r, y_routed, y_shared, bias_update(b, r.load, T, K, gamma))


def combine(u, y_shared, y_routed, gate, residual=True, shared=True, routed=True):
    """h'_t = u_t + sum_j y_shared[j, t] + sum_k gate[t,k] * y_routed[t,k]
    ([RG-MoE] combine equation); the flags drop a term for component checks."""
    u = _f64(u)
    out = np.zeros_like(u)
    if residual:
        out += u
    if shared:
        out += _f64(y_shared).sum(axis=0)
    if routed:
        out += np.einsum("tk,tkd->td", _f64(gate), _f64(y_routed))
    return out


# --------------------------------------------------------------------------
# Expert-contiguous layout (the stable counting sort the GPU path builds)
# --------------------------------------------------------------------------

@dataclass
class Layout:
    seg_offset: np.ndarray   # [N_r+N_s+1] int32, first padded row of each segment
    row_token: np.ndarray    # [P_max] int32, token of each row, -1 for padding
    inv_row: np.ndarray      # [T, K] int32, row holding (t, k)
    tile_map: np.ndarray     # [n_tiles, 4] int32: segment, first row, rows, token rows
    n_tiles: int


def permuted_rows_max(T: int, K: int, Nr: int, Ns: int, tile_m: int) -> int:
    """Upper bound on padded rows: all real rows plus tile_m-1 padding rows
    for every segment."""
    return T * K + Ns * T + (Nr + Ns) * (tile_m - 1)


def permute_layout(idx: np.ndarray, Nr: int, Ns: int, tile_m: int, tile_rows: int) -> Layout:
    """Definition of the expert-contiguous layout.

    Segment i < N_r holds the rows (t, k) with idx[t, k] == i in increasing t
    (a stable counting sort by expert); segment N_r + j holds every token t in
    order for shared expert j (gate 1, reading R7).  Each segment is padded
    with -1 rows to a multiple of tile_m; no token is dropped ([Blog-MoE]),
    so a segment may hold all T tokens.  The tile map cuts every segment, in
    segment order, into row tiles of tile_rows rows (the last one shorter).
    """
    idx = np.asarray(idx)
    T, K = idx.shape
    P_max = permuted_rows_max(T, K, Nr, Ns, tile_m)
    row_token = np.full(P_max, -1, dtype=np.int32)
    inv_row = np.full((T, K), -1, dtype=np.int32)
    seg_offset = np.zeros(Nr + Ns + 1, dtype=np.int32)
    tiles = []
    pos = 0
    for seg in range(Nr + Ns):
        seg_offset[seg] = pos
        if seg < Nr:
            t_sel, k_sel = np.nonzero(idx == seg)     # row-major: t ascending
        else:
            t_sel, k_sel = np.arange(T), None
        n = t_sel.size
        row_token[pos:pos + n] = t_sel
        if k_sel is not None:
            inv_row[t_sel, k_sel] = pos + np.arange(n)
        padded = -(-n // tile_m) * tile_m
        for r0 in range(0, padded, tile_rows):
            tiles.append((seg, pos + r0, min(tile_rows, padded - r0), max(0, min(tile_rows, n - r0))))
        pos += padded
    seg_offset[Nr + Ns] = pos
    tile_map = np.array(tiles, dtype=np.int32).reshape(-1, 4)
    return Layout(seg_offset, row_token, inv_row, tile_map, len(tiles))


def expert_rows(x: np.ndarray, w13, w2, layout: Layout, Nr: int, Ns: int, h_quant: bool = False):
    """y[row] = FFN_{segment(row)}(x[row_token[row]]) for every real row, 0 for
    padding rows: the ungated expert outputs in the permuted layout."""
    x = _f64(x)
    d = x.shape[1]
    P = layout.seg_offset[-1]
    y = np.zeros((P, d))
    for seg in range(Nr + Ns):
        r0, r1 = layout.seg_offset[seg], layout.seg_offset[seg + 1]
        toks = layout.row_token[r0:r1]
        real = toks >= 0
        if real.any():
            y[r0:r1][real], _ = swiglu_ffn(x[toks[real]], w13[seg], w2[seg], h_quant)
    return y
