"""Seeded synthetic inputs for the routing path.

This module only draws random numbers and shapes them; it holds none of the
routing arithmetic, so the GPU library and the CPU oracle can both be fed
from it without sharing any part of the method.

Five workloads (shapes of the router page's Args, the moe_finalize page's
Args, and the usual Mixtral / DeepSeek-V3 MoE layer sizes):

  tiny     T=64    E=8   G=1 TG=1 K=2 scale 1.0  H=128  down/out fp32
  mixtral  T=4096  E=8   G=1 TG=1 K=2 scale 1.0  H=4096 down/out bf16
  dsv3     T=8192  E=256 G=8 TG=4 K=8 scale 2.5  H=7168 down/out bf16
  decode   T=128   E=256 G=8 TG=4 K=8 scale 2.5  H=7168 down/out bf16
  skewed   T=65536 E=256 G=8 TG=4 K=8 scale 2.5  H=7168 down/out bf16

Recipe (seed S = 0 everywhere, one generator per tensor):
  logits   N(0, 1) [T, E], CPU generator seeded S;
           skewed adds 3 * (e + 1) ** -1.2 to expert e's logit (an
           un-normalised Zipf(1.2) rank weight, expert 0 hottest);
  scores   softmax over E of the logits (E = 8 workloads) or sigmoid
           (E = 256 workloads), fp32 on the CPU;
  bias     zeros (E = 8) or N(0, 0.01) (std 0.01), CPU generator seeded S+1;
  down     N(0, 1) [T*K, H] drawn in fp32 by a generator seeded S+2 on the
           requested device (in row blocks, so huge tensors need little
           temporary memory), then rounded to the workload's dtype.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    E: int
    n_groups: int
    topk_group: int
    K: int
    norm_weights: bool
    scale: float
    score_fn: str  # "softmax" | "sigmoid"
    bias: str  # "zero" | "normal"
    H: int
    down_dtype: torch.dtype
    out_dtype: torch.dtype
    skew: bool = False
    seed: int = 0

    @property
    def N(self) -> int:
        return self.T * self.K

    def with_tokens(self, T: int) -> "Workload":
        return replace(self, T=T)

    def describe(self) -> str:
        dt = {torch.float32: "f32", torch.bfloat16: "bf16"}
        return ("%s T=%d E=%d G=%d TG=%d K=%d H=%d down=%s out=%s scale=%g"
                % (self.name, self.T, self.E, self.n_groups, self.topk_group, self.K, self.H,
                   dt[self.down_dtype], dt[self.out_dtype], self.scale))


WORKLOADS = {
    "tiny": Workload("tiny", 64, 8, 1, 1, 2, True, 1.0, "softmax", "zero", 128,
                     torch.float32, torch.float32),
    "mixtral": Workload("mixtral", 4096, 8, 1, 1, 2, True, 1.0, "softmax", "zero", 4096,
                        torch.bfloat16, torch.bfloat16),
    "dsv3": Workload("dsv3", 8192, 256, 8, 4, 8, True, 2.5, "sigmoid", "normal", 7168,
                     torch.bfloat16, torch.bfloat16),
    "decode": Workload("decode", 128, 256, 8, 4, 8, True, 2.5, "sigmoid", "normal", 7168,
                       torch.bfloat16, torch.bfloat16),
    "skewed": Workload("skewed", 65536, 256, 8, 4, 8, True, 2.5, "sigmoid", "normal", 7168,
                       torch.bfloat16, torch.bfloat16, skew=True),
}


def make_logits(w: Workload) -> torch.Tensor:
    """Router logits [T, E] fp32 on the CPU (the scores are a function of them)."""
    g = torch.Generator().manual_seed(w.seed)
    logits = torch.randn(w.T, w.E, generator=g, dtype=torch.float32)
    if w.skew:
        rank = torch.arange(1, w.E + 1, dtype=torch.float64)
        logits = logits + (3.0 * rank.pow(-1.2)).to(torch.float32)
    return logits.contiguous()


def make_scores(w: Workload) -> torch.Tensor:
    """Routing scores [T, E] fp32 on the CPU."""
    logits = make_logits(w)
    if w.score_fn == "softmax":
        return torch.softmax(logits, dim=-1).contiguous()
    return torch.sigmoid(logits).contiguous()


def make_bias(w: Workload) -> torch.Tensor:
    """Per-expert selection bias [E] fp32 on the CPU."""
    if w.bias == "zero":
        return torch.zeros(w.E, dtype=torch.float32)
    g = torch.Generator().manual_seed(w.seed + 1)
    return (torch.randn(w.E, generator=g, dtype=torch.float32) * 0.01).contiguous()


def make_down(w: Workload, device="cpu", rows_per_block: int = 8192) -> torch.Tensor:
    """Expert outputs [T*K, H] in the workload's dtype on `device`."""
    n, h = w.N, w.H
    out = torch.empty(n, h, dtype=w.down_dtype, device=device)
    g = torch.Generator(device=device).manual_seed(w.seed + 2)
    for r0 in range(0, n, rows_per_block):
        r1 = min(n, r0 + rows_per_block)
        blk = torch.randn(r1 - r0, h, generator=g, dtype=torch.float32, device=device)
        out[r0:r1].copy_(blk)
        del blk
    return out


def random_scores(T: int, E: int, seed: int, levels: int = 0) -> torch.Tensor:
    """Scores in (0, 1) for property and parity tests. levels > 0 quantises to
    `levels` distinct values so that exact ties are frequent."""
    g = torch.Generator().manual_seed(seed)
    if levels > 0:
        q = torch.randint(1, levels + 1, (T, E), generator=g)
        return (q.to(torch.float32) / float(levels + 1)).contiguous()
    return torch.sigmoid(torch.randn(T, E, generator=g, dtype=torch.float32)).contiguous()


def random_bias(E: int, seed: int, std: float = 0.01, levels: int = 0) -> torch.Tensor:
    g = torch.Generator().manual_seed(seed)
    if levels > 0:
        q = torch.randint(0, levels, (E,), generator=g)
        return (q.to(torch.float32) / float(4 * levels)).contiguous()
    return (torch.randn(E, generator=g, dtype=torch.float32) * std).contiguous()


def random_ids(N: int, E: int, seed: int, skew: float = 0.0) -> torch.Tensor:
    """Flat expert ids [N] int32; skew > 0 draws from a Zipf(skew)-like pmf."""
    g = torch.Generator().manual_seed(seed)
    if skew > 0.0 and N > 0:
        p = torch.arange(1, E + 1, dtype=torch.float64).pow(-skew)
        return torch.multinomial(p / p.sum(), N, replacement=True, generator=g).to(torch.int32)
    return torch.randint(0, E, (N,), generator=g, dtype=torch.int32)


def random_permutation(N: int, seed: int) -> torch.Tensor:
    g = torch.Generator().manual_seed(seed)
    return torch.randperm(N, generator=g).to(torch.int32)
