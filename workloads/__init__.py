"""Seeded synthetic workloads for the DeepSeekMoE layer forward.

This module only draws random inputs of the right shape, dtype and value
distribution.  It holds none of the layer's arithmetic (no routing, no FFN,
no quantisation): both the CPU oracle and the GPU path receive the tensors it
makes, and nothing else is shared between them.

Shapes follow the DeepSeek-V3 MoE layer as the pages describe it (1 shared +
256 routed experts, 8 active, hidden size 7168) plus two smaller layers for
parity work.  Every tensor is drawn with a torch.Generator seeded from
(1234, config id, stream id, step) on the device it is made on, in fp32, and
then rounded (round-to-nearest-even) to its storage dtype; the rounded tensor
is the ground truth for both sides.

Streams: 0 = u, 1 = centroids e, 2 = W13, 3 = W2, 5 = initial bias,
6 = expert rank permutation (Zipf skew), 7 = free test data.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass

import torch

SEED_BASE = 1234

# Zipf skew of the expert loads (V3-scale prefill): centroid norms scale as
# r^-ZIPF_BETA for expert rank r.  The value was fitted so that the measured
# per-step load histogram has a least-squares log-log slope near -1.1.
ZIPF_BETA = 0.30


@dataclass(frozen=True)
class LayerConfig:
    name: str
    cfg_id: int
    T: int           # tokens per step
    d: int           # hidden size
    Nr: int          # routed experts
    Ns: int          # shared experts
    I: int           # expert intermediate size
    K: int           # routed experts per token
    act: str         # storage dtype of u and of the layer output: "f32" | "bf16"
    weights: str     # storage of W13/W2: "f32" | "bf16" | "e4m3" (128x128 blocks)
    x_fp8: bool      # expert-GEMM activations quantised to E4M3 in 1x128 tiles
    routing: str     # "iid" (all experts alike) | "zipf" (skewed centroid norms)
    bias_init: str   # "zero" | "uniform" (U(-0.01, 0.01))
    steps: int       # forward steps with the bias rule between them
    gamma: float = 0.001

    @property
    def E(self) -> int:
        return self.Nr + self.Ns

    def with_(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)

    def ffn_flops(self) -> int:
        """Expert FFN flops on real rows: 6*d*I per row (gate+up 4dI, down 2dI)."""
        return 6 * self.d * self.I * self.T * (self.K + self.Ns)


CONFIGS = {
    "tiny_fp32": LayerConfig("tiny_fp32", 0, T=64, d=256, Nr=16, Ns=1, I=128, K=4,
                             act="f32", weights="f32", x_fp8=False, routing="iid",
                             bias_init="zero", steps=1),
    "mid_bf16": LayerConfig("mid_bf16", 1, T=4096, d=2048, Nr=64, Ns=2, I=1408, K=6,
                            act="bf16", weights="bf16", x_fp8=False, routing="iid",
                            bias_init="uniform", steps=1),
    "v3_prefill_bf16": LayerConfig("v3_prefill_bf16", 2, T=8192, d=7168, Nr=256, Ns=1, I=2048, K=8,
                                   act="bf16", weights="bf16", x_fp8=False, routing="zipf",
                                   bias_init="zero", steps=10),
    "v3_decode_fp8w": LayerConfig("v3_decode_fp8w", 3, T=128, d=7168, Nr=256, Ns=1, I=2048, K=8,
                                  act="bf16", weights="e4m3", x_fp8=False, routing="iid",
                                  bias_init="zero", steps=1),
    "v3_prefill_fp8": LayerConfig("v3_prefill_fp8", 4, T=16384, d=7168, Nr=256, Ns=1, I=2048, K=8,
                                  act="bf16", weights="e4m3", x_fp8=True, routing="zipf",
                                  bias_init="zero", steps=10),
    # the v3_prefill_bf16 layer (same seeds: same tokens, centroids and weight
    # draws) run on the E4M3 path, at the size the training step fits in
    # 32-bit buffer offsets; a training workload only
    "v3_train_fp8": LayerConfig("v3_train_fp8", 2, T=8192, d=7168, Nr=256, Ns=1, I=2048, K=8,
                                act="bf16", weights="e4m3", x_fp8=True, routing="zipf",
                                bias_init="zero", steps=10),
}

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def generator(cfg_id: int, stream: int, step: int, device) -> torch.Generator:
    """A torch.Generator on `device` seeded from (1234, cfg_id, stream, step)."""
    g = torch.Generator(device=device)
    key = ((SEED_BASE * 1_000_003 + cfg_id) * 1_000_003 + stream) * 1_000_003 + step
    g.manual_seed(key % (2 ** 63 - 1))
    return g


def normal(shape, std: float, g: torch.Generator, device, dtype=torch.float32) -> torch.Tensor:
    """N(0, std^2) drawn in fp32, rounded once to `dtype`."""
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def make_tokens(cfg: LayerConfig, step: int, device) -> torch.Tensor:
    """u ~ N(0, 1), [T, d], in the activation storage dtype (fresh per step)."""
    return normal((cfg.T, cfg.d), 1.0, generator(cfg.cfg_id, 0, step, device), device,
                  TORCH_DTYPE[cfg.act])


def expert_ranks(cfg: LayerConfig) -> torch.Tensor:
    """Seeded permutation of ranks 1..N_r, so heavy experts are spread over indices."""
    g = generator(cfg.cfg_id, 6, 0, "cpu")
    return torch.randperm(cfg.Nr, generator=g) + 1


def make_centroids(cfg: LayerConfig, device) -> torch.Tensor:
    """e_i ~ N(0, I/d) fp32 [N_r, d]; for "zipf" routing row i is scaled by
    r_i^-ZIPF_BETA, r_i the expert's seeded rank."""
    e = normal((cfg.Nr, cfg.d), 1.0 / math.sqrt(cfg.d), generator(cfg.cfg_id, 1, 0, device), device)
    if cfg.routing == "zipf":
        r = expert_ranks(cfg).to(torch.float64)
        scale = (r ** (-ZIPF_BETA)).to(torch.float32).to(device)
        e.mul_(scale[:, None])
    return e


def make_bias(cfg: LayerConfig, device) -> torch.Tensor:
    """Initial routing bias [N_r] fp32: zeros or U(-0.01, 0.01)."""
    if cfg.bias_init == "zero":
        return torch.zeros(cfg.Nr, dtype=torch.float32, device=device)
    g = generator(cfg.cfg_id, 5, 0, device)
    return (torch.rand(cfg.Nr, generator=g, device=device, dtype=torch.float32) * 0.02 - 0.01)


def make_expert_weights(cfg: LayerConfig, device, experts=None):
    """W13 [E, 2I, d] and W2 [E, d, I], entries N(0, 1/d).

    Experts 0..N_r-1 are routed, N_r..N_r+N_s-1 shared.  Each expert is drawn
    from its own generator, so any subset (`experts`, a list of expert ids)
    can be regenerated alone with identical values.  Storage: fp32 or bf16 as
    configured; for "e4m3" weights the fp32 values are returned and the
    caller quantises them in 128x128 blocks on its own side.
    Returns (w13, w2) with a leading dim of len(experts) (all by default).
    """
    store = torch.float32 if cfg.weights in ("f32", "e4m3") else torch.bfloat16
    ids = list(range(cfg.E)) if experts is None else list(experts)
    std = 1.0 / math.sqrt(cfg.d)
    w13 = torch.empty((len(ids), 2 * cfg.I, cfg.d), dtype=store, device=device)
    w2 = torch.empty((len(ids), cfg.d, cfg.I), dtype=store, device=device)
    for n, i in enumerate(ids):
        w13[n] = normal((2 * cfg.I, cfg.d), std, generator(cfg.cfg_id, 2, i, device), device, store)
        w2[n] = normal((cfg.d, cfg.I), std, generator(cfg.cfg_id, 3, i, device), device, store)
    return w13, w2


def make_free(shape, std: float, seed: int, device, dtype=torch.float32) -> torch.Tensor:
    """Free seeded test data (stream 7), e.g. synthetic expert outputs."""
    return normal(shape, std, generator(99, 7, seed, device), device, dtype)


def to_f64(x: torch.Tensor):
    """Exact widening of a stored tensor to an fp64 NumPy array."""
    return x.detach().to("cpu", torch.float64).numpy()
