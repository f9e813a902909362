"""Parity at the full V3 sizes, in the launch configuration the benchmark
times (MoeLayer with tile_m = 32 on the full T, d = 7168, 256 routed + 1
shared experts, I = 2048, top-8).

The oracle cannot run the whole layer at this size in seconds, so it checks
what it can compute exactly: the routing of every token (fp64 logits for all
T x 256 pairs), the loads and the bias rule; every row of three experts'
segments sampled along the segment (the most loaded expert, a median one
and the shared expert, tile boundaries included); and the full output of a
few tokens, each computed from only the experts it selects.
"""
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
    """One forward + bias rule of a full-size layer on the GPU, and the
    oracle's routing of every token."""

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

    def x_of(self, tokens):
        """FFN input rows of `tokens`: u, or u through the 1x128 E4M3 tiles
        (tiles lie within a row, so a subset of rows quantises alike)."""
        return O.quantize_activations(self.u64[tokens]) if self.cfg.x_fp8 else self.u64[tokens]


TOL = {"v3_prefill_bf16": 1e-2, "v3_decode_fp8w": 1e-2, "v3_prefill_fp8": 3e-2}
# experts whose rows are checked / tokens whose whole output is checked;
# fewer for the E4M3 layers, where the oracle quantises each expert itself
SIZES = {"v3_prefill_bf16": (3, 4), "v3_decode_fp8w": (3, 2), "v3_prefill_fp8": (3, 2)}


@pytest.fixture(scope="module", params=list(TOL))
def full(request):
    run = FullRun(request.param)
    yield run
    del run
    torch.cuda.empty_cache()


def test_routing_loads_and_bias_at_full_size(full):
    cfg, layer, r = full.cfg, full.layer, full.routing
    _, tied = check_routing(np_of(layer.topk_idx), np_of(layer.topk_gate), np_of(layer.expert_load), r, cfg.Nr)
    if not tied:
        want_b = O.bias_update(np_of(full.b), r.load, cfg.T, cfg.K, cfg.gamma)
        assert np.array_equal(np_of(full.bias).view(np.uint32), want_b.view(np.uint32))


def test_expert_rows_at_full_size(full):
    """Rows of the most loaded expert, the shared expert and a median one:
    all rows of a segment of up to 256 rows, else every 37th row with every
    tile boundary included."""
    cfg, layer = full.cfg, full.layer
    n_exp, _ = SIZES[cfg.name]
    seg = np_of(layer.seg_offset)
    row_token = np_of(layer.row_token)
    order = np.argsort(np_of(layer.expert_load), kind="stable")
    experts = [int(order[-1]), cfg.Nr, int(order[len(order) // 2])][:n_exp]
    for i in experts:
        r0, r1 = int(seg[i]), int(seg[i + 1])
        rows = sample_rows(r0, r1, 1 if r1 - r0 <= 256 else 37)
        rows = rows[row_token[rows] >= 0]
        w13_i, w2_i = oracle_weights(cfg, full.w13, full.w2, i)
        want, _ = O.swiglu_ffn(full.x_of(row_token[rows]), w13_i, w2_i, h_quant=cfg.x_fp8)
        got = f64_of(layer.y[torch.from_numpy(rows).cuda()])
        err = rel_l2(got, want)
        print(f"[fullsize] {cfg.name}: expert {i}, {len(rows)} of {seg[i + 1] - seg[i]} rows, rel L2 {err:.2e}",
              flush=True)
        assert np.all(np.isfinite(got)) and err <= TOL[cfg.name], (i, err)


def test_token_outputs_at_full_size(full):
    """The whole output h'_t of a few tokens routed alike on both sides, from
    only the experts each selects; the FFN part on its own as well."""
    cfg, layer, r = full.cfg, full.layer, full.routing
    _, n_tok = SIZES[cfg.name]
    bad_or_tied = np.any(np_of(layer.topk_idx) != r.idx, axis=1)
    cand = np.nonzero(~bad_or_tied)[0]
    toks = cand[np.linspace(0, len(cand) - 1, n_tok).astype(int)]
    y_shared = np.zeros((cfg.Ns, len(toks), cfg.d))
    y_routed = np.zeros((len(toks), cfg.K, cfg.d))
    for i in sorted(set(r.idx[toks].ravel().tolist()) | set(range(cfg.Nr, cfg.E))):
        w13_i, w2_i = oracle_weights(cfg, full.w13, full.w2, i)
        if i >= cfg.Nr:
            y_shared[i - cfg.Nr], _ = O.swiglu_ffn(full.x_of(toks), w13_i, w2_i, h_quant=cfg.x_fp8)
        else:
            ts, ks = np.nonzero(r.idx[toks] == i)
            y_routed[ts, ks], _ = O.swiglu_ffn(full.x_of(toks[ts]), w13_i, w2_i, h_quant=cfg.x_fp8)
    u_t = full.u64[toks]
    want = O.combine(u_t, y_shared, y_routed, r.gate[toks])
    got = f64_of(full.out[torch.from_numpy(toks).cuda()])
    err, err_ffn = rel_l2(got, want), rel_l2(got - u_t, want - u_t)
    print(f"[fullsize] {cfg.name}: tokens {toks.tolist()}: rel L2 {err:.2e}, FFN part {err_ffn:.2e}", flush=True)
    assert err <= TOL[cfg.name] and err_ffn <= TOL[cfg.name]
