"""Benchmark of the DeepSeekMoE layer forward on one MI355X.

One step = one pass of the whole hot path over one batch of T tokens already
resident in HBM: moe_route -> moe_permute -> [fp8_quantize_tiles] ->
moe_expert_gemm -> moe_combine -> moe_bias_update (the bias carries over to
the next step, as in a training step).  W untimed warm-up steps, then exactly
K timed steps between two device synchronisations.  Prints one JSON line.

Workloads (synthetic, seeded; see workloads/):
  v3_prefill_bf16  T=8192, d=7168, 256 routed + 1 shared SwiGLU experts
                   (I=2048), top-8, bf16, Zipf-skewed loads (default)
  v3_prefill_fp8   T=16384, same layer, E4M3 activations and weights
  v3_decode_fp8w   T=128, same layer, E4M3 weights, bf16 activations
  mid_bf16, tiny_fp32  smaller layers

The roofline object describes the expert GEMM call (gate/up + SwiGLU, then
down), the dominant cost of the step, timed with HIP events on the stream it
is launched on.  The cpu_baseline object times the fp64 CPU oracle on a
bounded sample of the same workload.

--train times the training step instead (bf16 workloads): the forward with
its activations kept, the backward (combine/gate, expert GEMM dgrad and
wgrad, input and centroid gradients) for a seeded output gradient, and the
bias rule; its roofline object describes the expert GEMM backward call.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s at 256e/top-8 d7168; % MFMA peak (bf16/fp8), decode GB/s"
PEAK = {"bf16": 2.5e15, "fp8": 5.0e15, "f32": 157.3e12, "hbm": 8.0e12}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--config", default="v3_prefill_bf16")
    p.add_argument("--tile-m", type=int, default=32)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-tokens", type=int, default=0)
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target length of the oracle's timed CPU work (the sample is sized for it)")
    p.add_argument("--train", action="store_true",
                   help="time the training step instead: training forward + backward (bf16 workloads)")
    p.add_argument("--dgrad-fp8", action="store_true",
                   help="with --train: the backward's input-gradient products on E4M3 operands "
                        "(moe_expert_gemm_backward_w8; E4M3 weights prepared once at set-up)")
    p.add_argument("--wgrad-bf16", action="store_true",
                   help="with --train on an E4M3 workload: bf16 weight gradients (moe_expert_gemm_backward_w8) "
                        "instead of E4M3 ones (moe_expert_gemm_backward_f8)")
    p.add_argument("--fused-combine", action="store_true",
                   help="the expert GEMMs with the combine fused into the down projection (fp32 atomics, "
                        "moe_expert_gemm_combine) instead of moe_expert_gemm + moe_combine")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="only run a plain device copy of this many MiB (calibrates HBM byte counters) and exit")
    return p.parse_args()


# HBM traffic of one moe_expert_gemm call, from rocprofv3 --pmc FETCH_SIZE and
# WRITE_SIZE runs of this script (summed over the call's kernels, scaled by the
# factor the same counters give for a plain copy of known size).  Valid only
# for the kernel sources they were taken on: a changed source gives null.
TRAFFIC = {
    "v3_prefill_bf16": {"fetch_bytes": 36420200448, "write_bytes": 1359596134, "digest": "0cad120530f2390f"},
    "v3_prefill_fp8": {"fetch_bytes": 28308518912, "write_bytes": 2472101068, "digest": "0cad120530f2390f"},
    "v3_decode_fp8w": {"fetch_bytes": 11296614400, "write_bytes": 21416633, "digest": "07612974f52de25f"},
    # moe_expert_gemm_combine (--fused-combine): k_fused_prep + both phases
    "v3_prefill_bf16:fused": {"fetch_bytes": 37136534056, "write_bytes": 2653921382, "digest": "a14063dd68e34507",
                              "sources": ("gemm_mfma.hip", "elementwise.hip", "common.h")},
    "v3_prefill_fp8:fused": {"fetch_bytes": 28748369100, "write_bytes": 5060349440, "digest": "a14063dd68e34507",
                             "sources": ("gemm_mfma.hip", "elementwise.hip", "common.h")},
}

# HBM traffic of one backward expert GEMM call of the training step
# (moe_expert_gemm_backward / _w8 / _f8, with their quantisation passes),
# taken the same way from `--train` runs; keyed by workload, and for the
# E4M3 step with bf16 weight gradients by workload + ":bf16wgrad".
TRAIN_TRAFFIC = {
    "v3_prefill_bf16": {"fetch_bytes": 50803504256, "write_bytes": 24468564554, "digest": "eeb0641dc97e5494",
                        "sources": ("gemm_bwd.hip", "common.h")},
    "v3_train_fp8": {"fetch_bytes": 25938263722, "write_bytes": 27113556970, "digest": "76e3eec81c97cbbb",
                     "sources": ("gemm_bwd.hip", "elementwise.hip", "common.h")},
    "v3_train_fp8:bf16wgrad": {"fetch_bytes": 32813522133, "write_bytes": 25460402218, "digest": "76e3eec81c97cbbb",
                               "sources": ("gemm_bwd.hip", "elementwise.hip", "common.h")},
}

# Source files of the kernels each workload's expert GEMM runs.
GEMM_SOURCES = {"v3_decode_fp8w": ("gemm_w8.hip", "common.h")}
DEFAULT_GEMM_SOURCES = ("gemm_mfma.hip", "common.h")


def gemm_source_digest(workload, sources=None):
    import hashlib
    h = hashlib.sha256()
    for f in sources or GEMM_SOURCES.get(workload, DEFAULT_GEMM_SOURCES):
        with open(os.path.join(ROOT, "sparse_expert_routing_sigmoid_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def copy_probe(mib):
    """A plain device-to-device copy of `mib` MiB, launched 3 times: the
    reference for scaling FETCH_SIZE / WRITE_SIZE to bytes."""
    import torch
    n = mib * (1 << 20)
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "launches": 3}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}): the layer is built and measured on one "
              "GPU; multi-GPU expert parallelism is not part of this build.", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
        return
    import numpy as np
    import torch

    import sparse_expert_routing_sigmoid_amd as M
    import workloads as W

    cfg = W.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    if args.train:
        train_main(args, cfg, dev, stream)
        return

    # ---- inputs, resident in HBM before timing
    e = W.make_centroids(cfg, dev)
    bias0 = W.make_bias(cfg, dev)
    n_u = min(max(args.steps, 1), 10)
    us = [W.make_tokens(cfg, s, dev) for s in range(n_u)]
    w13, w2 = W.make_expert_weights(cfg, dev)
    if cfg.weights == "e4m3":
        weights = M.quantize_weights(w13, w2)
        del w13, w2
    else:
        weights = M.ExpertWeights(M.MOE_F32 if cfg.weights == "f32" else M.MOE_BF16, w13, w2)
    layer = M.MoeLayer(cfg.T, cfg.d, cfg.Nr, cfg.Ns, cfg.I, cfg.K, W.TORCH_DTYPE[cfg.act], weights,
                       x_fp8=cfg.x_fp8, tile_m=args.tile_m, device=dev, fused_combine=args.fused_combine)
    torch.cuda.synchronize()

    bias = bias0.clone()
    gemm_events = []
    step_events = []

    def step(s, timed):
        u = us[s % n_u]
        if timed:
            sv0 = torch.cuda.Event(enable_timing=True)
            sv0.record(stream)
        layer.route(u, e, bias)
        layer.permute()
        if timed:
            ev0 = torch.cuda.Event(enable_timing=True)
            ev1 = torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
        if args.fused_combine:
            layer.experts_combine(u)
        else:
            layer.experts(u)
        if timed:
            ev1.record(stream)
            gemm_events.append((ev0, ev1))
        if not args.fused_combine:
            layer.combine(u)
        layer.update_bias(bias, cfg.gamma)
        if timed:
            sv1 = torch.cuda.Event(enable_timing=True)
            sv1.record(stream)
            step_events.append((sv0, sv1))

    for s in range(args.warmup):
        step(s, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(s, True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / max(args.steps, 1)
    gemm_ms = float(np.mean([a.elapsed_time(b) for a, b in gemm_events])) if gemm_events else float("nan")
    step_ms = np.array([a.elapsed_time(b) for a, b in step_events])

    # ---- algorithmic work of one step
    loads = layer.expert_load.cpu().numpy().astype(np.int64)
    rows = int(cfg.T * cfg.K + cfg.T * cfg.Ns)
    gemm_flops = 6.0 * cfg.d * cfg.I * rows
    touched = int((loads > 0).sum()) + cfg.Ns
    wbytes_per_expert = 3 * cfg.I * cfg.d * (1 if cfg.weights == "e4m3" else (4 if cfg.weights == "f32" else 2))
    if cfg.weights == "e4m3":
        wbytes_per_expert += 4 * (2 * cfg.I // 128) * (cfg.d // 128) + 4 * (cfg.d // 128) * (cfg.I // 128)
    act_b = 4 if cfg.act == "f32" else 2
    x_b = 1 if cfg.x_fp8 else act_b
    # weights of touched experts, the gathered activations read once per row set, h and y unexcluded
    gemm_bytes = touched * wbytes_per_expert + cfg.T * cfg.d * x_b
    layer_bytes = touched * wbytes_per_expert + cfg.Nr * cfg.d * 4 + 2 * cfg.T * cfg.d * act_b
    dtype = {"bf16": "bf16", "f32": "f32", "e4m3": "fp8"}[cfg.weights] if not cfg.x_fp8 else "fp8"
    if cfg.weights == "e4m3" and not cfg.x_fp8:
        bound, peak, unit = "hbm", PEAK["hbm"], "GB/s"
        achieved = gemm_bytes / (gemm_ms * 1e-3)
        roof = {"bound": bound, "achieved": achieved / 1e9, "peak": peak / 1e9, "unit": unit,
                "frac": achieved / peak}
        dtype = "bf16"   # E4M3 weights are widened exactly to bf16 for the MFMAs
    else:
        mfma_peak = PEAK["fp8" if cfg.x_fp8 else ("f32" if cfg.weights == "f32" else "bf16")]
        achieved = gemm_flops / (gemm_ms * 1e-3)
        roof = {"bound": "mfma", "achieved": achieved / 1e12, "peak": mfma_peak / 1e12, "unit": "TFLOP/s",
                "frac": achieved / mfma_peak}
    tr = TRAFFIC.get(cfg.name + (":fused" if args.fused_combine else ""))
    digest = gemm_source_digest(cfg.name, tr.get("sources") if tr else None)
    roof["traffic"] = (tr["fetch_bytes"] + tr["write_bytes"]) / 1e9 if tr and tr["digest"] == digest else None
    roof["traffic_unit"] = "GB per launch"
    roof["kernel_digest"] = digest
    roof["kernel"] = ("moe_expert_gemm call: k_ffn_w8a16 phase A (gate/up + SwiGLU), then phase B (down), "
                      "each launched on the two halves of the tile map"
                      if cfg.weights == "e4m3" and not cfg.x_fp8 else
                      "moe_expert_gemm_combine call: k_fused_prep + k_ffn_schedule + k_ffn_persistent phase A "
                      "(gate/up + SwiGLU) + phase B (down, combine fused: fp32 atomics into the layer output)"
                      if args.fused_combine else
                      "moe_expert_gemm call: k_ffn_schedule + k_ffn_persistent phase A (gate/up + SwiGLU) + phase B (down)")
    roof["units_per_launch"] = {"rows": rows, "flops": gemm_flops, "algorithmic_bytes": gemm_bytes}
    roof["avg_launch_ms"] = gemm_ms

    tokens_s = cfg.T / (ms_step * 1e-3)
    layer_time = ms_step * 1e-3
    out = {
        "metric": METRIC,
        "value": tokens_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded; random-init expert weights and centroids of the V3 MoE-layer shape)",
        "config": {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "Nr": cfg.Nr, "Ns": cfg.Ns, "I": cfg.I,
                   "K": cfg.K, "routing": cfg.routing, "weights": cfg.weights, "x_fp8": cfg.x_fp8,
                   "tile_m": args.tile_m, "bias_update": "every step", "parallelism": "single GPU",
                   "combine": "fused into the down projection (fp32 atomics)" if args.fused_combine else
                   "moe_combine (deterministic)"},
        "layer": {"tflops": gemm_flops / layer_time / 1e12,
                  "mfma_frac": gemm_flops / layer_time / (PEAK["fp8"] if cfg.x_fp8 else PEAK["bf16"]),
                  "hbm_gbs": layer_bytes / layer_time / 1e9, "hbm_frac": layer_bytes / layer_time / PEAK["hbm"],
                  "experts_touched": touched, "max_load": int(loads.max()), "mean_load": float(loads.mean()),
                  "last_step_load_slope": load_fit_exponent(loads),
                  "padded_rows": int(layer.seg_offset[-1].item())},
        "step_ms": {"median": float(np.median(step_ms)), "p10": float(np.percentile(step_ms, 10)),
                    "p90": float(np.percentile(step_ms, 90)), "timer": "HIP events per step on the stream"},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, layer, us[0], e, bias0, weights, args.cpu_sample_tokens,
                                           args.cpu_seconds)
    print(json.dumps(out), flush=True)


def load_fit_exponent(loads):
    """Least-squares slope of log(load) against log(rank) over the experts
    with a nonzero load, sorted by load (a Zipf law of exponent s gives -s).
    Reported for the last timed step: the bias rule, applied after every
    step, flattens the skew of the first step (slope -1.1 at T = 8192 with
    b = 0) as the steps go on."""
    import numpy as np
    x = np.sort(loads[loads > 0])[::-1].astype(np.float64)
    if x.size < 2:
        return None
    return float(np.polyfit(np.log(np.arange(1, x.size + 1)), np.log(x), 1)[0])


def host_info():
    """CPU model and the BLAS NumPy uses, for the oracle timing."""
    from threadpoolctl import threadpool_info
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = [f"{p.get('internal_api')} ({p.get('num_threads')} threads)" for p in threadpool_info()
            if p.get("user_api") == "blas"]
    return {"cpu_model": model, "blas": ", ".join(blas) or None}


def cpu_baseline(cfg, layer, u, e, b, weights, sample_tokens, seconds):
    """Time the fp64 oracle on the first S tokens of step 0: routing, the
    routed + shared SwiGLU experts of each sampled token, and the combine.
    S is sized so that the FFN work takes about `seconds` at the host's fp64
    matrix-product rate (measured here first); weight conversion to fp64 is
    input preparation and is not timed."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    from oracle import e4m3 as OE
    from oracle import moe as O

    if not sample_tokens:
        a = np.ones((256, cfg.d))
        w = np.ones((cfg.d, cfg.I))
        t1 = time.perf_counter()
        a @ w
        rate = 2.0 * 256 * cfg.d * cfg.I / max(time.perf_counter() - t1, 1e-6)
        per_token = 6.0 * cfg.d * cfg.I * (cfg.K + cfg.Ns)
        sample_tokens = int(seconds * rate / per_token)
    S = max(16, min(sample_tokens, cfg.T))
    f64 = lambda t: t.detach().to("cpu", torch.float64).numpy()
    u_s = f64(u[:S])
    e_h = f64(e)
    b_h = f64(b)
    t_route = time.perf_counter()
    r = O.route(u_s, e_h, b_h, cfg.K)
    t_route = time.perf_counter() - t_route
    x = O.quantize_activations(u_s) if cfg.x_fp8 else u_s
    need = sorted(set(r.idx.ravel().tolist()) | set(range(cfg.Nr, cfg.Nr + cfg.Ns)))

    def expert_w(i):
        if weights.w_t == 2:   # E4M3 codes + 128x128 block scales
            w13 = OE.dequantize_tiles(weights.w13[i].cpu().numpy(), weights.w13_scale[i].cpu().numpy(), 128, 128)
            w2 = OE.dequantize_tiles(weights.w2[i].cpu().numpy(), weights.w2_scale[i].cpu().numpy(), 128, 128)
            return w13, w2
        return f64(weights.w13[i]), f64(weights.w2[i])

    t_ffn = 0.0
    y_routed = np.zeros((S, cfg.K, cfg.d))
    y_shared = np.zeros((cfg.Ns, S, cfg.d))
    for i in need:
        w13, w2 = expert_w(i)
        t1 = time.perf_counter()
        if i >= cfg.Nr:
            y_shared[i - cfg.Nr], _ = O.swiglu_ffn(x, w13, w2, h_quant=cfg.x_fp8)
        else:
            ts, ks = np.nonzero(r.idx == i)
            y_routed[ts, ks], _ = O.swiglu_ffn(x[ts], w13, w2, h_quant=cfg.x_fp8)
        t_ffn += time.perf_counter() - t1
    t1 = time.perf_counter()
    O.combine(u_s, y_shared, y_routed, r.gate)
    t_comb = time.perf_counter() - t1
    total = t_route + t_ffn + t_comb
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": S / total, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {S} of {cfg.T} tokens of step 0: fp64 routing over all {cfg.Nr} experts, "
                      f"{cfg.K} routed + {cfg.Ns} shared SwiGLU experts per token, combine; "
                      f"{len(need)} experts touched; weight conversion to fp64 not timed",
            "seconds": total, "host_cpus": os.cpu_count(), **host_info()}


TRAIN_METRIC = "MoE-layer training step (forward + backward) tokens/s at 256e/top-8 d7168"


def train_main(args, cfg, dev, stream):
    """One training step = the forward of main() with the activations kept
    (moe_expert_gemm_train) + moe_combine_backward -> moe_expert_gemm_backward
    -> moe_route_backward for a seeded bf16 dL/dh' + the bias rule.  The
    roofline object describes the moe_expert_gemm_backward call (dgrad and
    wgrad of both expert projections, 12 d I flops per row).  On an E4M3
    workload (x_fp8, E4M3 weights) the step is the FP8 one:
    moe_expert_gemm_train_w8, Q(u) decoded for the gate/up weight gradient,
    and moe_expert_gemm_backward_f8 (every backward product on E4M3
    operands; --wgrad-bf16: moe_expert_gemm_backward_w8)."""
    import numpy as np
    import torch

    import sparse_expert_routing_sigmoid_amd as M
    import workloads as W

    fp8_step = cfg.x_fp8 and cfg.weights == "e4m3"
    if not fp8_step and (cfg.weights != "bf16" or cfg.act != "bf16" or cfg.x_fp8):
        print(f"--train needs a bf16 or an E4M3 workload (got {cfg.name})", file=sys.stderr)
        sys.exit(2)
    e = W.make_centroids(cfg, dev)
    bias0 = W.make_bias(cfg, dev)
    n_u = min(max(args.steps, 1), 4)
    us = [W.make_tokens(cfg, s, dev) for s in range(n_u)]
    gs = [W.make_free((cfg.T, cfg.d), 1.0, 100 + s, dev, torch.bfloat16) for s in range(n_u)]
    w13, w2 = W.make_expert_weights(cfg, dev)
    # E4M3 weights: quantised once per optimizer step, outside the layer step
    w8 = M.quantize_weights(w13, w2) if (args.dgrad_fp8 or fp8_step) else None
    wgrad8 = fp8_step and not args.wgrad_bf16
    if fp8_step:
        layer = M.MoeLayer(cfg.T, cfg.d, cfg.Nr, cfg.Ns, cfg.I, cfg.K, torch.bfloat16, w8, x_fp8=True,
                           tile_m=args.tile_m, device=dev, train=True, grad_dtype=torch.bfloat16,
                           wgrad_fp8=wgrad8)
    else:
        layer = M.MoeLayer(cfg.T, cfg.d, cfg.Nr, cfg.Ns, cfg.I, cfg.K, torch.bfloat16,
                           M.ExpertWeights(M.MOE_BF16, w13, w2), tile_m=args.tile_m, device=dev, train=True,
                           grad_dtype=torch.bfloat16, dgrad_weights=w8)
    torch.cuda.synchronize()
    bias = bias0.clone()
    bwd_events = []

    def step(s, timed):
        u, G = us[s % n_u], gs[s % n_u]
        layer.forward(u, e, bias)
        M.moe_combine_backward(G, layer.y, layer.inv_row, layer.topk_gate, layer.topk_score, layer.seg_offset,
                               cfg.Nr, cfg.Ns, layer.dy, layer.dgate, layer.dz, layer.dz_row)
        x = u
        if fp8_step:   # the gate/up weight gradient takes the Q(u) the forward multiplied
            M.fp8_dequantize_tiles(layer.xq, layer.xs, 1, layer.xdq)
            x = layer.xdq
        if timed:
            ev0 = torch.cuda.Event(enable_timing=True)
            ev1 = torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
        if w8 is None:
            M.moe_expert_gemm_backward(u, w13, w2, layer.h, layer.ab, layer.dy, cfg.T, cfg.K, cfg.Nr, cfg.Ns, cfg.d,
                                       cfg.I, args.tile_m, layer.seg_offset, layer.row_token, layer.tile_map,
                                       layer.n_tiles, layer.bwd_ws, layer.dx, layer.dw13, layer.dw2)
        else:
            bwd = M.moe_expert_gemm_backward_f8 if wgrad8 else M.moe_expert_gemm_backward_w8
            bwd(x, w8, layer.h, layer.ab, layer.dy, cfg.T, cfg.K, cfg.Nr, cfg.Ns, cfg.d, cfg.I, args.tile_m,
                layer.seg_offset, layer.row_token, layer.tile_map, layer.n_tiles, layer.bwd_ws, layer.dx, layer.dw13,
                layer.dw2)
        if timed:
            ev1.record(stream)
            bwd_events.append((ev0, ev1))
        M.moe_route_backward(G, layer.dx, u, e, layer.topk_idx, layer.inv_row, layer.dz, layer.dz_row,
                             layer.seg_offset, layer.row_token, cfg.Nr, cfg.Ns, layer.du, layer.de)
        layer.update_bias(bias, cfg.gamma)

    for s in range(args.warmup):
        step(s, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(s, True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / max(args.steps, 1)
    bwd_ms = float(np.mean([a.elapsed_time(b) for a, b in bwd_events]))
    rows = int(cfg.T * cfg.K + cfg.T * cfg.Ns)
    bwd_flops = 12.0 * cfg.d * cfg.I * rows
    step_flops = 18.0 * cfg.d * cfg.I * rows
    if not fp8_step:
        step_peak = PEAK["bf16"]
    elif wgrad8:
        step_peak = PEAK["fp8"]
    else:   # the weight gradients (6 of the 18 d I flops per row) in bf16
        step_peak = step_flops / (12.0 / 18 * step_flops / PEAK["fp8"] + 6.0 / 18 * step_flops / PEAK["bf16"])
    loads = layer.expert_load.cpu().numpy().astype(np.int64)
    achieved = bwd_flops / (bwd_ms * 1e-3)
    if w8 is None:
        peak = PEAK["bf16"]
        kernels = ("moe_expert_gemm_backward call: k_dgrad (down + SwiGLU backward), k_dgrad (gate/up), "
                   "k_wgrad (down), k_wgrad (gate/up)")
    elif wgrad8:
        peak = PEAK["fp8"]
        kernels = ("moe_expert_gemm_backward_f8 call: k_run_offsets, k_quant_runs (dy: runs and 1x128 tiles), "
                   "k_dgrad8 (down + SwiGLU backward), k_quant_runs ([da|db]: runs and 1x128 tiles), k_dgrad8 "
                   "(gate/up), k_quant_runs (h), k_quant_runs (gathered x), k_wgrad_deal, k_wgrad8 (down), "
                   "k_wgrad8 (gate/up); every product E4M3")
    else:
        # half the flops (the input-gradient products) at the E4M3 peak, half
        # (the weight gradients) at the bf16 peak: the call's time at peak
        # gives its effective peak rate
        peak = bwd_flops / (0.5 * bwd_flops / PEAK["fp8"] + 0.5 * bwd_flops / PEAK["bf16"])
        kernels = ("moe_expert_gemm_backward_w8 call: k_quant_1x128 (dy), k_dgrad8 (down + SwiGLU backward), "
                   "k_quant_1x128 ([da|db]), k_dgrad8 (gate/up), k_wgrad (down), k_wgrad (gate/up); peak = the "
                   "call's flops over their time at the E4M3 (dgrad) and bf16 (wgrad) peaks")
    tkey = cfg.name + (":bf16wgrad" if fp8_step and not wgrad8 else "")
    tt = TRAIN_TRAFFIC.get(tkey) if (w8 is not None) == fp8_step else None
    traffic = None
    if tt and gemm_source_digest(cfg.name, tt["sources"]) == tt["digest"]:
        traffic = (tt["fetch_bytes"] + tt["write_bytes"]) / 1e9
    roof = {"bound": "mfma", "achieved": achieved / 1e12, "peak": peak / 1e12, "unit": "TFLOP/s",
            "frac": achieved / peak, "traffic": traffic, "traffic_unit": "GB per call", "kernel": kernels,
            "units_per_launch": {"rows": rows, "flops": bwd_flops}, "avg_launch_ms": bwd_ms}
    out = {
        "metric": TRAIN_METRIC,
        "value": cfg.T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("e4m3" if wgrad8 else "e4m3 + bf16 wgrad") if fp8_step else (
            "bf16" if w8 is None else "bf16 + e4m3 dgrad"),
        "data": "synthetic (seeded; random-init expert weights and centroids, seeded bf16 output gradients)",
        "config": {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "Nr": cfg.Nr, "Ns": cfg.Ns, "I": cfg.I,
                   "K": cfg.K, "routing": cfg.routing, "weights": cfg.weights, "tile_m": args.tile_m,
                   "step": "training forward + backward + bias rule" + (
                       ("; E4M3 forward and every backward product (weight gradients on runs of 128 tokens)"
                        if wgrad8 else "; E4M3 forward and backward input-gradient products, bf16 weight gradients")
                       + " (weights quantised once per optimizer step, not in the step)" if fp8_step else
                       "; backward input-gradient products on E4M3 (weights quantised once at set-up, "
                       "not in the step)" if w8 is not None else ""), "grad_dtype": "bf16",
                   "parallelism": "single GPU"},
        "layer": {"tflops": step_flops / (ms_step * 1e-3) / 1e12,
                  "mfma_frac": step_flops / (ms_step * 1e-3) / step_peak,
                  "max_load": int(loads.max()), "mean_load": float(loads.mean())},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_train(cfg, us[0], gs[0], e, bias0, w13, w2, args.cpu_seconds,
                                                 fp8=("train8" if wgrad8 else "train") if fp8_step else
                                                 w8 is not None)
    print(json.dumps(out), flush=True)


def cpu_baseline_train(cfg, u, G, e, b, w13, w2, seconds, fp8=False):
    """Time the fp64 backward oracle's expert FFN backward (oracle/backward.py
    ffn_backward, the dominant part of the layer backward) on the first S
    tokens: for every expert their rows select, dx, dW13, dW2 of those rows.
    S is sized for about `seconds` of work; weight conversion not timed."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    from oracle import backward as OB
    from oracle import moe as O

    a = np.ones((256, cfg.d))
    w = np.ones((cfg.d, cfg.I))
    t1 = time.perf_counter()
    a @ w
    rate = 2.0 * 256 * cfg.d * cfg.I / max(time.perf_counter() - t1, 1e-6)
    per_token = 18.0 * cfg.d * cfg.I * (cfg.K + cfg.Ns)
    S = max(16, min(int(seconds * rate / per_token), cfg.T))
    f64 = lambda t: t.detach().to("cpu", torch.float64).numpy()
    u_s, G_s = f64(u[:S]), f64(G[:S])
    r = O.route(u_s, f64(e), f64(b), cfg.K)
    need = sorted(set(r.idx.ravel().tolist()) | set(range(cfg.Nr, cfg.Nr + cfg.Ns)))
    total = 0.0
    # (FP8 training step: the weights go in as stored; quantising them
    # belongs to the optimizer step, and the timed work does not depend on
    # their values)
    print(f"cpu baseline: {S} tokens, {len(need)} experts", file=sys.stderr, flush=True)
    for i in need:
        w13_i, w2_i = f64(w13[i]), f64(w2[i])
        if i >= cfg.Nr:
            x, dy = u_s, G_s
        else:
            ts, ks = np.nonzero(r.idx == i)
            x, dy = u_s[ts], r.gate[ts, ks][:, None] * G_s[ts]
        t1 = time.perf_counter()
        if fp8 in ("train", "train8"):
            OB.ffn_backward_fp8_train(x, w13_i, w2_i, dy, fp8_wgrad_products=fp8 == "train8")
        else:
            (OB.ffn_backward_fp8 if fp8 else OB.ffn_backward)(x, w13_i, w2_i, dy)
        total += time.perf_counter() - t1
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": S / total, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {S} of {cfg.T} tokens of step 0: fp64 SwiGLU FFN backward"
                      f"{' of the FP8 training step' if fp8 == 'train' else ' of the FP8 training step with E4M3 weight gradients' if fp8 == 'train8' else ' with E4M3 input-gradient products' if fp8 else ''}"
                      f" (forward recomputed, "
                      f"dx, dW13, dW2) of the {cfg.K} routed + {cfg.Ns} shared experts of each token, "
                      f"{len(need)} experts touched; routing, gate and centroid gradients not timed",
            "seconds": total, "host_cpus": os.cpu_count(), **host_info()}


if __name__ == "__main__":
    main()
