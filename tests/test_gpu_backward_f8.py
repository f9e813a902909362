"""E4M3 weight gradients (reading B5 of the backward oracle): the token-axis
quantiser fp8_quantize_runs bit for bit against the oracle's E4M3 codec, the
weight-gradient kernel against oracle.backward.fp8_wgrad on the GPU's own
operands (to fp32 accumulation order), and the whole E4M3 training step with
moe_expert_gemm_backward_f8 against layer_backward(fp8_train=True,
fp8_wgrad=True).

Layouts come from the oracle's permute_layout on seeded selections (skewed
loads: empty experts, experts of one row, experts of several 128-row runs,
tile_m 32 and 1); padding rows of the inputs hold NaN, which the quantiser
must read as zeros."""
import numpy as np
import pytest
import torch

import sparse_expert_routing_sigmoid_amd as M
import workloads as W
from moe_testutil import check_routing, f64_of, np_of, rel_l2
from oracle import backward as OB
from oracle import moe as O
from oracle.e4m3 import dequantize_tiles, e4m3_decode, quantize_tiles

pytestmark = pytest.mark.gpu

TOL8, TOL, MIRROR = 3e-2, 1e-2, 5e-3


def skewed_selection(T, K, Nr, seed):
    """[T, K] distinct experts per token with Zipf-like loads; the last
    quarter of the experts is never chosen."""
    rng = np.random.default_rng(seed)
    live = max(K, Nr - Nr // 4)
    p = 1.0 / np.arange(1, live + 1) ** 1.1
    p /= p.sum()
    return np.stack([rng.choice(live, size=K, replace=False, p=p) for _ in range(T)]).astype(np.int32)


def oracle_runs(src_rows, seg_offset, row_token, n_seg):
    """Expected codes [P, C] (0 on padding rows) and scales [runs, C] of
    fp8_quantize_runs, from the oracle's E4M3 tile quantiser on each
    segment's rows, zero-padded to whole runs of 128."""
    P, C = row_token.shape[0], src_rows.shape[1]
    codes = np.zeros((P, C), dtype=np.uint8)
    scales = []
    for s in range(n_seg):
        a, b = seg_offset[s], seg_offset[s + 1]
        if b == a:
            continue
        n = -(-(b - a) // 128) * 128
        m = np.zeros((n, C))
        live = row_token[a:b] >= 0
        m[:b - a][live] = src_rows[a:b][live]
        q, sc = quantize_tiles(m, 128, 1)
        codes[a:b] = q[:b - a]
        scales.append(sc)
    return codes, (np.concatenate(scales) if scales else np.zeros((0, C), np.float32))


@pytest.mark.parametrize("T,K,Nr,Ns,C,tile_m,gather,dtype", [
    (300, 4, 16, 1, 256, 32, False, torch.bfloat16),
    (300, 4, 16, 1, 384, 32, True, torch.bfloat16),      # a half 256-column chunk
    (1000, 6, 24, 2, 512, 1, True, torch.float32),       # no row padding; segments of many runs
    (5, 2, 8, 1, 128, 32, False, torch.float32),
    (0, 2, 8, 1, 256, 32, True, torch.bfloat16),         # no tokens: every segment empty
])
def test_quantize_runs_bit_exact(T, K, Nr, Ns, C, tile_m, gather, dtype):
    print(f"fp8_quantize_runs T={T} K={K} Nr={Nr} Ns={Ns} C={C} tile_m={tile_m} gather={gather} {dtype}", flush=True)
    idx = skewed_selection(T, K, Nr, 40 + T) if T else np.zeros((0, K), np.int32)
    lay = O.permute_layout(idx, Nr, Ns, tile_m, 256)
    P, n_seg = lay.row_token.shape[0], Nr + Ns
    rng = np.random.default_rng(41)
    rows = T if gather else P
    x = rng.standard_normal((rows, C)) * np.exp2(rng.integers(-8, 8, (rows, 1))) * np.exp2(rng.integers(-4, 4, (1, C)))
    x = torch.from_numpy(x).to(dtype)
    if not gather:
        x[torch.from_numpy(lay.row_token < 0)] = float("nan")   # padding rows: never read as values
    xd = x.cuda()
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    so, rt = dev(lay.seg_offset), dev(lay.row_token)
    runs_max = M.fp8_quantize_runs_max(P, n_seg)
    q = torch.full((P, C), 0xAB, dtype=torch.uint8, device="cuda")
    sc = torch.full((max(runs_max, 1), C), -1.0, dtype=torch.float32, device="cuda")
    ro = torch.full((n_seg + 1,), -7, dtype=torch.int32, device="cuda")
    M.fp8_quantize_runs(xd, rt, gather, so, P, ro, q, sc)
    torch.cuda.synchronize()
    xs = f64_of(x)
    if gather:
        src = xs[np.maximum(lay.row_token, 0)] if rows else np.zeros((P, C))
    else:
        src = xs
    want_q, want_s = oracle_runs(src, lay.seg_offset, lay.row_token, n_seg)
    lens = np.diff(lay.seg_offset)
    want_ro = np.concatenate([[0], np.cumsum(-(-lens // 128))]).astype(np.int32)
    assert np.array_equal(np_of(ro), want_ro)
    runs = int(want_ro[-1])
    assert runs <= runs_max
    used = lay.seg_offset[-1]
    assert np.array_equal(np_of(q)[:used], want_q[:used])
    assert np.all(np_of(q)[used:] == 0xAB)                  # rows past the last segment untouched
    assert np.array_equal(np_of(sc)[:runs].view(np.uint32), want_s.astype(np.float32).view(np.uint32))


def train_layer(cfg, grad_dtype, wgrad_fp8=True):
    w13, w2 = W.make_expert_weights(cfg, "cuda")
    w8 = M.quantize_weights(w13, w2)
    layer = M.MoeLayer(cfg.T, cfg.d, cfg.Nr, cfg.Ns, cfg.I, cfg.K, torch.bfloat16, w8, x_fp8=True, tile_m=32,
                       train=True, grad_dtype=grad_dtype, wgrad_fp8=wgrad_fp8)
    u, e, b = W.make_tokens(cfg, 0, "cuda"), W.make_centroids(cfg, "cuda"), W.make_bias(cfg, "cuda")
    return layer, w13, w2, u, e, b


def oracle_weights(w13, w2):
    deq = lambda w: dequantize_tiles(*quantize_tiles(w.astype(np.float32), 128, 128), 128, 128)
    return np.stack([deq(x) for x in f64_of(w13)]), np.stack([deq(x) for x in f64_of(w2)])


BASE = W.CONFIGS["mid_bf16"]
CASES = {
    "small": BASE.with_(T=256, d=512, Nr=16, Ns=1, I=256, K=4),
    # experts of 200+ rows (two runs and more), an odd row count per run
    "long": BASE.with_(T=600, d=768, Nr=8, Ns=2, I=256, K=3),
    "mid": BASE.with_(T=1024, d=1024, Nr=32, Ns=2, I=512, K=6),
}


# The scaled matrix instruction sums each block of 32 K values (one E8M0
# scale block) in limited precision and adds the block sum to the fp32
# accumulator (see test_scaled_mfma_accumulation): per output element the
# error stays within BLOCK_ACC of sum |a b|, besides fp32 rounding.
BLOCK_ACC = 2.0 ** -9


def direct_f8_backward(cfg, grad_dtype, seed=110):
    """A bf16 training forward (its h and [a | b]), moe_combine_backward, then
    moe_expert_gemm_backward_f8 called directly (any I % 128 == 0).  Returns
    the layer, the dW tensors, the workspace and the input x."""
    w13, w2 = W.make_expert_weights(cfg, "cuda")
    w8 = M.quantize_weights(w13, w2)
    layer = M.MoeLayer(cfg.T, cfg.d, cfg.Nr, cfg.Ns, cfg.I, cfg.K, torch.bfloat16,
                       M.ExpertWeights(M.MOE_BF16, w13, w2), tile_m=32, train=True, grad_dtype=grad_dtype)
    u, e, b = W.make_tokens(cfg, 0, "cuda"), W.make_centroids(cfg, "cuda"), W.make_bias(cfg, "cuda")
    layer.forward(u, e, b)
    G = W.make_free((cfg.T, cfg.d), 1.0, seed, "cuda", torch.bfloat16)
    M.moe_combine_backward(G, layer.y, layer.inv_row, layer.topk_gate, layer.topk_score, layer.seg_offset,
                           cfg.Nr, cfg.Ns, layer.dy, layer.dgate, layer.dz, layer.dz_row)
    E = cfg.Nr + cfg.Ns
    ws = torch.empty((M.moe_gemm_backward_f8_workspace_bytes(cfg.T, cfg.K, cfg.Nr, cfg.Ns, cfg.d, cfg.I, 32),),
                     dtype=torch.uint8, device="cuda")
    dw13 = torch.full((E, 2 * cfg.I, cfg.d), float("nan"), dtype=grad_dtype, device="cuda")
    dw2 = torch.full((E, cfg.d, cfg.I), float("nan"), dtype=grad_dtype, device="cuda")
    M.moe_expert_gemm_backward_f8(u, w8, layer.h, layer.ab, layer.dy, cfg.T, cfg.K, cfg.Nr, cfg.Ns, cfg.d, cfg.I,
                                  32, layer.seg_offset, layer.row_token, layer.tile_map, layer.n_tiles, ws, layer.dx,
                                  dw13, dw2)
    torch.cuda.synchronize()
    return layer, dw13, dw2, ws, u


WG_CASES = dict(CASES)
# I % 256 == 128: h and dW2 end in half an N tile (the E4M3 forward needs
# I % 256 == 0, the backward call does not)
WG_CASES["ragged"] = BASE.with_(T=600, d=768, Nr=8, Ns=2, I=384, K=3)


@pytest.mark.parametrize("name", list(WG_CASES))
def test_wgrad8_equals_oracle_on_gpu_operands(name):
    """dW2_e = R(dy_e)^T R(h_e) and dW13_e = R([da | db]_e)^T R(x_e) from the
    GPU's own bf16 operands (dy and h as the layer keeps them, [da | db] at
    the head of the call's workspace, x = u at the rows' tokens) by
    oracle.backward.fp8_wgrad, expert by expert, fp32 and bf16 outputs."""
    cfg = WG_CASES[name]
    for gd in (torch.float32, torch.bfloat16):
        print(f"wgrad8 on GPU operands {name} {gd}: {cfg}", flush=True)
        layer, dw13, dw2, ws, u = direct_f8_backward(cfg, gd)
        P = layer.P_max
        so, rt = np_of(layer.seg_offset), np_of(layer.row_token)
        dab = f64_of(ws[:P * 2 * cfg.I * 2].view(torch.bfloat16).view(P, 2 * cfg.I))
        xs = f64_of(u)
        ops = {"dw2": (f64_of(layer.dy), f64_of(layer.h), f64_of(dw2)),
               "dw13": (dab, None, f64_of(dw13))}
        worst = 0.0
        for which, (A, B, got) in ops.items():
            for s in range(cfg.Nr + cfg.Ns):
                a, c = so[s], so[s + 1]
                live = np.nonzero(rt[a:c] >= 0)[0] + a
                if live.size == 0:
                    assert np.all(got[s] == 0.0), (which, s)
                    continue
                b_rows = B[live] if B is not None else xs[rt[live]]
                ra, rb = OB.quantize_token_runs(A[live]), OB.quantize_token_runs(b_rows)
                want = OB.fp8_wgrad(A[live], b_rows)
                sab = np.abs(ra).T @ np.abs(rb)
                bound = (BLOCK_ACC + (live.size + 4) * 2.0 ** -24) * sab
                if gd == torch.bfloat16:
                    bound = bound + np.abs(want) * 2.0 ** -8 * (1 + 1e-6)   # round to nearest bf16
                err = np.abs(got[s] - want)
                worst = max(worst, float((err / np.maximum(sab, 1e-300)).max()))
                assert np.all(err <= bound + 1e-30), (which, s, float((err - bound).max()))
        print(f"  max |error| / sum|ab| = {worst:.3g}", flush=True)


def test_scaled_mfma_accumulation():
    """The accumulation of the E4M3 products, probed through
    moe_expert_gemm_backward_f8 on one expert of 128 rows: dW2[0, n] =
    sum_k dy[k, 0] h[k, n] with dy[:, 0] = 1 and h[:, n] holding 256 and
    2^-8 (both exact in E4M3 at the run's scale 1).  Terms in different
    32-value blocks add exactly (the block sums are accumulated in fp32):
    64 x 256 + 64 x 2^-8 and 32 x 256 + 32 x 2^-8 come out exact.  Inside
    one block the small terms next to a large one lose low bits; the error
    stays within BLOCK_ACC of sum |a b|."""
    T, K, Nr, Ns, d, I, tm = 128, 1, 1, 0, 256, 256, 32
    lay = O.permute_layout(np.zeros((T, K), np.int32), Nr, Ns, tm, 256)
    P = M.moe_permute_rows(T, K, Nr, Ns, tm)
    assert P == lay.row_token.shape[0]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    tmap = torch.zeros((M.moe_permute_tiles_max(T, K, Nr, Ns, tm), 4), dtype=torch.int32, device="cuda")
    tmap[:lay.tile_map.shape[0]] = dev(lay.tile_map)
    g = torch.Generator().manual_seed(0)
    w8 = M.quantize_weights((torch.randn((1, 2 * I, d), generator=g) / 16).cuda(),
                            (torch.randn((1, d, I), generator=g) / 16).cuda())
    bf = dict(dtype=torch.bfloat16, device="cuda")
    dy, h, ab, x = (torch.zeros((P, d), **bf), torch.zeros((P, I), **bf), torch.zeros((P, 2 * I), **bf),
                    torch.zeros((T, d), **bf))
    big, small = 256.0, 2.0 ** -8
    dy[:128, 0] = 1.0
    h[:64, 0], h[64:128, 0] = big, small            # a block of each: exact
    h[:32, 1], h[32:64, 1] = big, small             # the two blocks of one instruction: exact
    h[0:64:2, 2], h[1:64:2, 2] = big, small         # mixed inside each block
    h[:128, 3], h[0, 3] = small, big                # one large term among small ones
    exact = np.array([64 * big + 64 * small, 32 * big + 32 * small, 32 * big + 32 * small, big + 127 * small])
    sab = np.array([64 * big + 64 * small, 32 * big + 32 * small, 32 * big + 32 * small, big + 127 * small])
    ws = torch.empty((M.moe_gemm_backward_f8_workspace_bytes(T, K, Nr, Ns, d, I, tm),), dtype=torch.uint8,
                     device="cuda")
    dw13 = torch.empty((1, 2 * I, d), device="cuda")
    dw2 = torch.empty((1, d, I), device="cuda")
    M.moe_expert_gemm_backward_f8(x, w8, h, ab, dy, T, K, Nr, Ns, d, I, tm, dev(lay.seg_offset), dev(lay.row_token),
                                  tmap, dev(np.array([lay.n_tiles], np.int32)), ws, torch.empty((P, d), **bf),
                                  dw13, dw2)
    torch.cuda.synchronize()
    got = f64_of(dw2[0, 0, :4])
    print(f"accumulation probe: got {got.tolist()}, exact {exact.tolist()}", flush=True)
    assert got[0] == exact[0] and got[1] == exact[1]
    assert np.all(np.abs(got - exact) <= BLOCK_ACC * sab)
    assert np.all(f64_of(dw2[0, 1:]) == 0.0) and np.all(f64_of(dw2[0, 0, 4:]) == 0.0)


@pytest.mark.parametrize("name", list(CASES))
def test_f8_training_step_matches_oracle(name):
    """The E4M3 training step with E4M3 weight gradients against
    layer_backward(fp8_train=True, fp8_wgrad=True)."""
    cfg = CASES[name]
    print(f"E4M3 training step, E4M3 wgrad {name}: {cfg}", flush=True)
    layer, w13, w2, u, e, b = train_layer(cfg, torch.float32)
    layer.forward(u, e, b)
    G = W.make_free((cfg.T, cfg.d), 1.0, 100, "cuda", torch.bfloat16)
    du, de, dw13, dw2 = layer.backward(G, u, e)
    torch.cuda.synchronize()
    u64, e64, b64, G64 = map(f64_of, (u, e, b, G))
    r = O.route(u64, e64, b64, cfg.K)
    ok, tied = check_routing(np_of(layer.topk_idx), np_of(layer.topk_gate), np_of(layer.expert_load), r, cfg.Nr)
    assert not tied, "seeded inputs hold a near-tie; the gradients would not be comparable"
    w13q, w2q = oracle_weights(w13, w2)
    gr = OB.layer_backward(u64, e64, b64, w13q, w2q, cfg.Nr, cfg.Ns, cfg.K, G64, fp8_train=True, fp8_wgrad=True)
    errs = {"du": rel_l2(f64_of(du), gr.du), "dw13": rel_l2(f64_of(dw13), gr.dw13),
            "dw2": rel_l2(f64_of(dw2), gr.dw2), "de": rel_l2(f64_of(de), gr.de),
            "dgate": rel_l2(f64_of(layer.dgate), gr.dgate), "dz": rel_l2(f64_of(layer.dz), gr.dz)}
    print(errs, flush=True)
    for k, v in errs.items():
        assert v <= (MIRROR if k in ("du", "dw13", "dw2") else TOL), (k, v)
    # the E4M3 weight gradients differ from the bf16 ones of reading B3
    plain = OB.layer_backward(u64, e64, b64, w13q, w2q, cfg.Nr, cfg.Ns, cfg.K, G64, fp8_train=True)
    assert rel_l2(f64_of(dw2), plain.dw2) > 5 * errs["dw2"]


def test_f8_backward_idle_experts_no_tokens_and_determinism():
    """Experts without rows get zero weight gradients; a step without tokens
    writes zeros; two backward calls give identical bits."""
    cfg = CASES["small"].with_(T=8, Nr=64, K=2)
    layer, w13, w2, u, e, b = train_layer(cfg, torch.bfloat16)
    for t in (layer.dw13, layer.dw2):
        t.fill_(float("nan"))
    layer.forward(u, e, b)
    G = W.make_free((cfg.T, cfg.d), 1.0, 102, "cuda", torch.bfloat16)
    first = [t.clone() for t in layer.backward(G, u, e)]
    second = layer.backward(G, u, e)
    torch.cuda.synchronize()
    for a, c in zip(first, second):
        assert torch.equal(a, c)
    idle = np.nonzero(np_of(layer.expert_load) == 0)[0]
    assert idle.size > 0
    assert torch.count_nonzero(first[2][idle]).item() == 0 and torch.count_nonzero(first[3][idle]).item() == 0
    w13q, w2q = oracle_weights(w13, w2)
    gr = OB.layer_backward(*map(f64_of, (u, e, b)), w13q, w2q, cfg.Nr, cfg.Ns, cfg.K, f64_of(G), fp8_train=True,
                           fp8_wgrad=True)
    # experts of one or two rows: each run's scale comes from one value, so a
    # code decided from a bf16 value one step off moves the product by a
    # whole E4M3 step; the E4M3 bound applies
    for name, got, want in (("dw13", first[2], gr.dw13), ("dw2", first[3], gr.dw2)):
        assert rel_l2(f64_of(got), want) <= TOL8, name

    cfg0 = CASES["small"].with_(T=0)
    layer, w13, w2, u, e, b = train_layer(cfg0, torch.bfloat16)
    for t in (layer.dw13, layer.dw2):
        t.fill_(float("nan"))
    layer.forward(u, e, b)
    du, de, dw13, dw2 = layer.backward(torch.empty((0, cfg0.d), dtype=torch.bfloat16, device="cuda"), u, e)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dw13).item() == 0 and torch.count_nonzero(dw2).item() == 0


def test_wgrad_fp8_needs_the_e4m3_training_path():
    cfg = CASES["small"]
    w13, w2 = W.make_expert_weights(cfg, "cuda")
    with pytest.raises(ValueError):
        M.MoeLayer(cfg.T, cfg.d, cfg.Nr, cfg.Ns, cfg.I, cfg.K, torch.bfloat16, M.ExpertWeights(M.MOE_BF16, w13, w2),
                   train=True, dgrad_weights=M.quantize_weights(w13, w2), wgrad_fp8=True)
