"""Parity at the full V3 sizes, in the launch configuration the benchmark
times (MoeLayer with tile_m = 32 on the full T, d = 7168, 256 routed + 1
shared experts, I = 2048, top-8).

Compared against the fp64 oracle on the same seeded inputs:
- the routing of every token (fp64 logits for all T x 256 pairs), the loads
  and the bias rule of the first step;
- v3_prefill_bf16 (T = 8192) and v3_decode_fp8w (T = 128): the expert
  output y of every row of every expert, and the whole output h'_t of every
  token, with its FFN part (h'_t - u_t) on its own;
- v3_prefill_fp8 (T = 16384): h'_t and its FFN part for 1024 tokens spread
  over the batch, and the rows of the most loaded, a median and the shared
  expert (every 37th row, every tile boundary);
- the two multi-step workloads: 10 steps of the bias rule with a fresh u per
  step, teacher-forced (each GPU step starts from the oracle's bias):
  routing and loads at every step; the new bias is, bit for bit, the bias
  rule on the GPU's loads, and the oracle's wherever the loads agree (a
  near-tie token moves one assignment between two experts).
Each token is compared where its selection equals the oracle's (a token at a
near-tie may legitimately select another expert).  The E4M3 workloads'
weights are quantised by the oracle's own 128x128 quantiser, expert by
expert, in a pool of host threads.
"""
import concurrent.futures as cf
import os

import numpy as np
import pytest
import torch

import sparse_expert_routing_sigmoid_amd as M
import workloads as W
from moe_testutil import check_routing, f64_of, np_of, rel_l2
from oracle import e4m3 as OE
from oracle import moe as O

pytestmark = pytest.mark.gpu

TILE_M = 32
TOL = {"v3_prefill_bf16": 1e-2, "v3_decode_fp8w": 1e-2, "v3_prefill_fp8": 3e-2}
# tokens whose output is compared (None = all) and experts whose rows are
# compared ("all", or the most loaded / shared / median sample)
TOKENS = {"v3_prefill_bf16": None, "v3_decode_fp8w": None, "v3_prefill_fp8": 1024}
ROWS = {"v3_prefill_bf16": "all", "v3_decode_fp8w": "all", "v3_prefill_fp8": "sample"}
HOST_THREADS = max(1, min(16, os.cpu_count() or 1))


def oracle_weights(cfg, w13, w2, i):
    """Expert i's weights as the oracle sees them: widened bf16, or the
    oracle's own 128x128 E4M3 quantisation of the fp32 values, decoded."""
    a13 = w13[i].to("cpu", torch.float32).numpy()
    a2 = w2[i].to("cpu", torch.float32).numpy()
    if cfg.weights == "e4m3":
        deq = lambda m: OE.dequantize_tiles(*OE.quantize_tiles(m, 128, 128), 128, 128)
        return deq(a13), deq(a2)
    return a13.astype(np.float64), a2.astype(np.float64)


def sample_rows(r0, r1, every):
    """Rows r0..r1-1 sampled every `every`, plus the first and last row of
    each 256-row tile of the segment."""
    rows = set(range(r0, r1, every))
    for t0 in range(r0, r1, M.MOE_TILE_ROWS):
        rows.update({t0, min(t0 + M.MOE_TILE_ROWS, r1) - 1})
    return np.array(sorted(rows))


class FullRun:
    """One forward + bias rule of a full-size layer on the GPU, the oracle's
    routing of every token, and (on first use) the oracle's expert outputs."""

    def __init__(self, name):
        cfg = self.cfg = W.CONFIGS[name]
        print(f"[fullsize] {name}: T={cfg.T} d={cfg.d} E={cfg.E} I={cfg.I} K={cfg.K}", flush=True)
        self.u = W.make_tokens(cfg, 0, "cuda")
        self.e = W.make_centroids(cfg, "cuda")
        self.b = W.make_bias(cfg, "cuda")
        self.w13, self.w2 = W.make_expert_weights(cfg, "cuda")
        if cfg.weights == "e4m3":
            weights = M.quantize_weights(self.w13, self.w2)
        else:
            weights = M.ExpertWeights(M.MOE_BF16, self.w13, self.w2)
        self.layer = M.MoeLayer(cfg.T, cfg.d, cfg.Nr, cfg.Ns, cfg.I, cfg.K, W.TORCH_DTYPE[cfg.act], weights,
                                x_fp8=cfg.x_fp8, tile_m=TILE_M)
        self.out = self.layer.forward(self.u, self.e, self.b)
        self.bias = self.b.clone()
        self.layer.update_bias(self.bias, cfg.gamma)
        torch.cuda.synchronize()
        self.u64 = f64_of(self.u)
        self.routing = O.route(self.u64, f64_of(self.e), f64_of(self.b), cfg.K)
        self._ffn = None

    def checked_tokens(self):
        """Tokens whose output is compared: all, or an even spread."""
        n = TOKENS[self.cfg.name]
        return np.arange(self.cfg.T) if n is None else np.linspace(0, self.cfg.T - 1, n).astype(np.int64)

    def checked_rows(self):
        """{expert: permuted rows of the GPU layout whose y is compared}."""
        cfg, layer = self.cfg, self.layer
        seg, row_token = np_of(layer.seg_offset), np_of(layer.row_token)
        if ROWS[cfg.name] == "all":
            experts, every = range(cfg.E), 1
        else:
            order = np.argsort(np_of(layer.expert_load), kind="stable")
            experts, every = [int(order[-1]), int(order[len(order) // 2])] + list(range(cfg.Nr, cfg.E)), 37
        rows = {}
        for i in experts:
            r = sample_rows(int(seg[i]), int(seg[i + 1]), every)
            r = r[row_token[r] >= 0] if r.size else r
            if r.size:
                rows[int(i)] = r
        return rows

    def ffn(self):
        """{expert: (tokens, oracle FFN_i of their FFN input rows)} over the
        tokens every comparison needs: the checked tokens' oracle-selected
        experts and shared experts, and the tokens of the checked rows."""
        if self._ffn is not None:
            return self._ffn
        cfg, r = self.cfg, self.routing
        toks = self.checked_tokens()
        need = {i: set() for i in range(cfg.E)}
        for i in range(cfg.Nr, cfg.E):
            need[i].update(toks.tolist())
        sel = r.idx[toks]
        for t, row in zip(toks.tolist(), sel):
            for i in row.tolist():
                need[i].add(t)
        row_token = np_of(self.layer.row_token)
        self.rows = self.checked_rows()
        for i, rows in self.rows.items():
            need[i].update(row_token[rows].tolist())
        # FFN inputs of every token needed: u, or u through its 1x128 E4M3
        # tiles (a tile lies within a row, so a subset of rows quantises alike)
        all_t = np.array(sorted(set().union(*need.values())), dtype=np.int64)
        x_all = O.quantize_activations(self.u64[all_t]) if cfg.x_fp8 else self.u64[all_t]

        def task(i):
            ts = np.array(sorted(need[i]), dtype=np.int64)
            if ts.size == 0:
                return i, ts, None
            w13_i, w2_i = oracle_weights(cfg, self.w13, self.w2, i)
            y, _ = O.swiglu_ffn(x_all[np.searchsorted(all_t, ts)], w13_i, w2_i, h_quant=cfg.x_fp8)
            return i, ts, y

        experts = [i for i in range(cfg.E) if need[i]]
        out = {}
        if cfg.weights == "e4m3":
            # the oracle's quantiser is NumPy, which leaves the GIL while it
            # works: one BLAS thread per pool thread
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=1), cf.ThreadPoolExecutor(HOST_THREADS) as ex:
                for n, (i, ts, y) in enumerate(ex.map(task, experts)):
                    out[i] = (ts, y)
                    if n % 64 == 63:
                        print(f"[fullsize] {cfg.name}: oracle experts {n + 1}/{len(experts)}", flush=True)
        else:
            for i in experts:
                i, ts, y = task(i)
                out[i] = (ts, y)
        self._ffn = out
        return out


@pytest.fixture(scope="module", params=list(TOL))
def full(request):
    run = FullRun(request.param)
    yield run
    del run
    torch.cuda.empty_cache()


def _y_of(ffn, i, tokens):
    ts, y = ffn[i]
    pos = np.searchsorted(ts, tokens)
    assert np.array_equal(ts[pos], tokens)
    return y[pos]


def check_bias(b_gpu, b_old, gpu_load, r, cfg):
    """The GPU's new bias is the bias rule applied to its own loads, bit for
    bit, and equals the oracle's wherever the two loads agree (a near-tie
    moves one assignment between two experts).  Returns the experts whose
    loads differ."""
    mine = O.bias_update(b_old, gpu_load, cfg.T, cfg.K, cfg.gamma)
    want = O.bias_update(b_old, r.load, cfg.T, cfg.K, cfg.gamma)
    assert np.array_equal(b_gpu.view(np.uint32), mine.view(np.uint32))
    same = gpu_load == r.load
    assert np.array_equal(b_gpu[same].view(np.uint32), want[same].view(np.uint32))
    return np.nonzero(~same)[0]


def test_routing_loads_and_bias_at_full_size(full):
    cfg, layer, r = full.cfg, full.layer, full.routing
    _, tied = check_routing(np_of(layer.topk_idx), np_of(layer.topk_gate), np_of(layer.expert_load), r, cfg.Nr)
    moved = check_bias(np_of(full.bias), np_of(full.b), np_of(layer.expert_load), r, cfg)
    print(f"[fullsize] {cfg.name}: {len(tied)} near-tie tokens, loads differ at experts {moved.tolist()}", flush=True)


@pytest.mark.timeout(900)
def test_expert_rows_at_full_size(full):
    """y of every row of every expert (bf16 prefill, decode), or of sampled
    rows of the most loaded, a median and the shared expert (FP8 prefill):
    each expert's rows within the tolerance, and all of them together."""
    cfg, layer = full.cfg, full.layer
    ffn = full.ffn()
    row_token = np_of(layer.row_token)
    num = den = 0.0
    worst = (0.0, -1)
    for i, rows in full.rows.items():
        want = _y_of(ffn, i, row_token[rows])
        got = f64_of(layer.y[torch.from_numpy(rows).cuda()])
        assert np.all(np.isfinite(got)), i
        err = rel_l2(got, want)
        num += float(np.sum((got - want) ** 2))
        den += float(np.sum(want ** 2))
        worst = max(worst, (err, i))
        assert err <= TOL[cfg.name], (i, len(rows), err)
    total = float(np.sqrt(num / den))
    print(f"[fullsize] {cfg.name}: y of {sum(len(v) for v in full.rows.values())} rows over "
          f"{len(full.rows)} experts: rel L2 {total:.2e}, worst expert {worst[1]} at {worst[0]:.2e}", flush=True)
    assert total <= TOL[cfg.name]


@pytest.mark.timeout(900)
def test_token_outputs_at_full_size(full):
    """h'_t of every checked token whose selection equals the oracle's, from
    the oracle's expert outputs and gates; the FFN part on its own as well,
    over all of them together and token by token."""
    cfg, layer, r = full.cfg, full.layer, full.routing
    ffn = full.ffn()
    toks = full.checked_tokens()
    toks = toks[np.all(np_of(layer.topk_idx)[toks] == r.idx[toks], axis=1)]
    n = len(toks)
    y_shared = np.stack([_y_of(ffn, i, toks) for i in range(cfg.Nr, cfg.E)])
    y_routed = np.zeros((n, cfg.K, cfg.d))
    for k in range(cfg.K):
        for i in np.unique(r.idx[toks, k]).tolist():
            m = r.idx[toks, k] == i
            y_routed[m, k] = _y_of(ffn, i, toks[m])
    u_t = full.u64[toks]
    want = O.combine(u_t, y_shared, y_routed, r.gate[toks])
    got = f64_of(full.out[torch.from_numpy(toks).cuda()])
    err, err_ffn = rel_l2(got, want), rel_l2(got - u_t, want - u_t)
    per_tok = np.linalg.norm((got - u_t) - (want - u_t), axis=1) / np.linalg.norm(want - u_t, axis=1)
    print(f"[fullsize] {cfg.name}: {n} of {cfg.T} tokens: rel L2 {err:.2e}, FFN part {err_ffn:.2e}, "
          f"worst token FFN part {per_tok.max():.2e} (median {np.median(per_tok):.2e})", flush=True)
    assert n >= 0.99 * len(full.checked_tokens())
    assert err <= TOL[cfg.name] and err_ffn <= TOL[cfg.name]
    assert per_tok.max() <= 3 * TOL[cfg.name]


@pytest.mark.timeout(300)
def test_bias_trajectory_teacher_forced(full):
    """Ten steps of the bias rule, a fresh u each step, each GPU step started
    from the oracle's bias: routing, loads and the new bias every step (runs
    last: it overwrites the layer's buffers)."""
    cfg, layer = full.cfg, full.layer
    if cfg.steps < 2:
        pytest.skip("single-step workload")
    e64 = f64_of(full.e)
    b = np_of(full.b).astype(np.float32)
    for s in range(cfg.steps):
        u = W.make_tokens(cfg, s, "cuda")
        b_gpu = torch.from_numpy(b.copy()).cuda()
        layer.forward(u, full.e, b_gpu)
        layer.update_bias(b_gpu, cfg.gamma)
        torch.cuda.synchronize()
        r = O.route(f64_of(u), e64, b, cfg.K)
        _, tied = check_routing(np_of(layer.topk_idx), np_of(layer.topk_gate), np_of(layer.expert_load), r, cfg.Nr)
        moved = check_bias(np_of(b_gpu), b, np_of(layer.expert_load), r, cfg)
        b = O.bias_update(b, r.load, cfg.T, cfg.K, cfg.gamma)
        print(f"[fullsize] {cfg.name} step {s}: max load {int(r.load.max())}, near-ties {len(tied)}, "
              f"loads differ at {moved.tolist()}, |b|max {np.abs(b).max():.4f}", flush=True)
