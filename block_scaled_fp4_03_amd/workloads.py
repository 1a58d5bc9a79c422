"""Seeded synthetic inputs for the NVFP4 MoE workloads.

This module only draws random numbers; it holds none of the pipeline's
arithmetic (no quantisation, routing or GEMM).  It is the one place both the
GPU library's callers and the CPU oracle's callers take their inputs from.

Workloads (hidden 7168, expert intermediate 3072, 384 experts, top-6 are the
DeepSeek-V4 MoE shapes named on the pages):

=========  ==================================================================
tiny       T=16, H=256, I=128, E=8, top-2; logits N(0,1); x N(0,1) -> bf16;
           weights N(0, 0.02^2).
shared     shared expert (one group, no routing), T=128, H=7168, I=3072; x
           N(0,1) with floor(0.001*T*H) positions (random permutation) scaled
           by 20, then bf16.
decode     routed layer, T=256, E=384, top-6, logits N(0,1).
prefill    routed layer, T=8192, E=384, top-6; logits N(0,1) plus a
           per-expert bias -1.1*ln(rank_e), rank a random permutation of
           1..384, so expert popularity follows Zipf(1.1).
mla        MLA projections, T=4096: x1 [T,7168] through the fused q_a+kv
           weight [1536+512, 7168]; x2 [T,1536] through q_b [65536, 1536].
attn_out   attention output path, T=4096: all heads' outputs x [T, 128*512]
           N(0,1) -> bf16 through wo_a [1024, 65536] (FP8 weights), then
           wo_b [7168, 1024] (NVFP4 weights).
=========  ==================================================================

Draw order.  Every tensor has its own torch generator seeded from the batch
seed and a tag, so tensors can be drawn independently and in any order:
x -> seed*10+1, logits -> seed*10+2, expert-rank permutation -> seed*10+3,
outlier positions -> seed*10+4, mla x2 -> seed*10+5, attention outputs ->
seed*10+6.  Weights: one generator
per (expert, projection), seed*1_000_003 + 3*e + p with p = 0 (gate_up),
1 (down), 2 (extra projections), 3 (wo_a), 4 (wo_b; the attention output
workload has no experts); weights of the full-size routed workloads are
drawn on the GPU (torch's Philox generator) because 384 experts are 25e9
values; the rows the oracle needs are copied back to the host.
The measured batch uses seed 0, the warmup batch that sets the activation
global scales uses seed 1.
"""
from dataclasses import dataclass, field
import math

import torch

WEIGHT_STD = 0.02


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "moe", "shared" or "mla"
    T: int
    H: int = 7168
    I: int = 3072
    E: int = 1
    k: int = 1
    zipf: float = 0.0         # exponent of the per-expert popularity bias, 0 = none
    outlier_frac: float = 0.0
    outlier_mult: float = 20.0
    # MLA shapes
    n_qa: int = 1536
    n_kv: int = 512
    q_lora: int = 1536
    n_qb: int = 128 * 512
    o_lora: int = 1024
    weights_on_device: bool = False
    warmup_tokens: int = 0    # tokens in the warmup batch (0: same T as the workload)

    def flops(self):
        """Algorithmic multiply-adds x2 of the GEMMs of one pass."""
        if self.kind == "moe":
            return 6.0 * self.T * self.k * self.H * self.I
        if self.kind == "shared":
            return 6.0 * self.T * self.H * self.I
        if self.kind == "attn_out":
            return 2.0 * self.T * (self.n_qb * self.o_lora + self.o_lora * self.H)
        return 2.0 * self.T * (self.H * (self.n_qa + self.n_kv) + self.q_lora * self.n_qb)


WORKLOADS = {
    "tiny": Workload("tiny", "moe", T=16, H=256, I=128, E=8, k=2),
    "shared": Workload("shared", "shared", T=128, outlier_frac=0.001),
    "decode": Workload("decode", "moe", T=256, E=384, k=6, weights_on_device=True),
    "prefill": Workload("prefill", "moe", T=8192, E=384, k=6, zipf=1.1, weights_on_device=True),
    "mla": Workload("mla", "mla", T=4096),
    "attn_out": Workload("attn_out", "attn_out", T=4096, warmup_tokens=64),
}


def _gen(seed, device="cpu"):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def activations(T, H, seed, outlier_frac=0.0, outlier_mult=20.0, tag=1):
    """x ~ N(0,1) [T, H] float32, optional outliers, rounded to bf16 and
    returned as float32 holding bf16 values."""
    x = torch.randn(T, H, generator=_gen(seed * 10 + tag), dtype=torch.float32)
    n_out = int(math.floor(outlier_frac * T * H))
    if n_out:
        pos = torch.randperm(T * H, generator=_gen(seed * 10 + 4))[:n_out]
        x.view(-1)[pos] *= outlier_mult
    return x.to(torch.bfloat16).to(torch.float32)


def router_logits(T, E, seed, zipf=0.0):
    """Router logits [T, E] float32: N(0,1), plus -zipf*ln(rank_e) if zipf."""
    logits = torch.randn(T, E, generator=_gen(seed * 10 + 2), dtype=torch.float32)
    if zipf:
        rank = torch.randperm(E, generator=_gen(seed * 10 + 3)).to(torch.float64) + 1.0
        logits = logits + (-zipf * torch.log(rank)).to(torch.float32)[None, :]
    return logits


def expert_seed(seed, e, p):
    return seed * 1_000_003 + 3 * e + p


def weight(N, K, seed, device="cpu"):
    """One weight matrix [N, K] float32 ~ N(0, 0.02^2) from its own generator."""
    g = _gen(seed, device)
    return torch.randn(N, K, generator=g, dtype=torch.float32, device=device) * WEIGHT_STD


def moe_gate_up(wl, e, seed=0, device="cpu"):
    """Stacked gate_up weight of expert e, [2I, H]: rows [0, I) gate, [I, 2I) up."""
    return weight(2 * wl.I, wl.H, expert_seed(seed, e, 0), device)


def moe_down(wl, e, seed=0, device="cpu"):
    """Down weight of expert e, [H, I]."""
    return weight(wl.H, wl.I, expert_seed(seed, e, 1), device)


def mla_weights(wl, seed=0, device="cpu"):
    """(fused q_a+kv [n_qa+n_kv, H], q_b [n_qb, q_lora])."""
    w1 = weight(wl.n_qa + wl.n_kv, wl.H, expert_seed(seed, 0, 0), device)
    w2 = weight(wl.n_qb, wl.q_lora, expert_seed(seed, 0, 1), device)
    return w1, w2


def attn_out_weights(wl, seed=0, device="cpu"):
    """(wo_a [o_lora, 128*512], wo_b [H, o_lora]) float32."""
    return (weight(wl.o_lora, wl.n_qb, expert_seed(seed, 0, 3), device),
            weight(wl.H, wl.o_lora, expert_seed(seed, 0, 4), device))


def batch(wl, seed=0, tokens=None):
    """The activations (and logits) of one batch: dict of float32 CPU tensors."""
    T = wl.T if tokens is None else tokens
    if wl.kind == "attn_out":
        return {"x": activations(T, wl.n_qb, seed, tag=6)}
    out = {"x": activations(T, wl.H, seed, wl.outlier_frac, wl.outlier_mult)}
    if wl.kind == "moe":
        out["logits"] = router_logits(T, wl.E, seed, wl.zipf)
    if wl.kind == "mla":
        out["x2"] = activations(T, wl.q_lora, seed, tag=5)
    return out


def warmup_batch(wl):
    """The warmup batch (seed 1) whose amax sets the activation global scales."""
    return batch(wl, seed=1, tokens=wl.warmup_tokens or None)
