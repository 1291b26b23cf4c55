"""Seeded synthetic inputs for causal attention.

This module draws random tensors and nothing else: it holds none of the
attention arithmetic, and it is the only code shared by the HIP-path tests,
the CPU oracle tests, the smoke check and the benchmark.

The workloads are the layer shapes of the CS336 model-size table (d_model /
n_heads: 768/12 -> D=64, 1024/16 -> D=64, 2560/32 -> D=80) and the largest
point of the handout's FlashAttention-2 benchmark sweep (B=1, causal,
S=65536, D=128).  Inputs are i.i.d. standard normal, as the pages' benchmarks
use random tensors; one workload scales Q and K by 2 to make the softmax
peaky.
"""
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "f32" or "bf16"
    B: int
    H: int
    S: int
    D: int
    seed: int
    qk_mult: float = 1.0
    causal: bool = True

    @property
    def scale(self) -> float:
        return 1.0 / (self.D ** 0.5)

    @property
    def shape(self):
        return (self.B, self.H, self.S, self.D)

    def causal_pairs(self) -> int:
        """Exact number of (query, key) pairs the causal mask allows."""
        if self.causal:
            return self.B * self.H * self.S * (self.S + 1) // 2
        return self.B * self.H * self.S * self.S


WORKLOADS = {
    w.name: w for w in [
        Workload("f32_b1h2_s128_d64", "f32", 1, 2, 128, 64, seed=1),
        Workload("bf16_b4h12_s512_d64", "bf16", 4, 12, 512, 64, seed=2),
        Workload("bf16_b4h16_s2048_d64_peaky", "bf16", 4, 16, 2048, 64, seed=3, qk_mult=2.0),
        Workload("bf16_b1h32_s16000_d80", "bf16", 1, 32, 16000, 80, seed=4),
        Workload("bf16_b1h16_s65536_d128", "bf16", 1, 16, 65536, 128, seed=5),
    ]
}

#: seed for the sampled heads and rows of the long workloads
ROW_SAMPLE_SEED = 1005

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def make_inputs(B, H, S, D, dtype="bf16", seed=0, qk_mult=1.0):
    """Q, K, V, dO of shape [B, H, S, D] in ``dtype`` (CPU tensors).

    Drawn as fp32 N(0,1) from ``torch.Generator('cpu').manual_seed(seed)`` in
    the order Q, K, V, dO; Q and K are multiplied by ``qk_mult``; then cast
    (round-to-nearest-even) to the storage dtype.
    """
    g = torch.Generator("cpu").manual_seed(int(seed))
    out = []
    for name in ("q", "k", "v", "do"):
        x = torch.randn((B, H, S, D), generator=g, dtype=torch.float32)
        if name in ("q", "k") and qk_mult != 1.0:
            x.mul_(qk_mult)
        out.append(x.to(TORCH_DTYPE[dtype]))
    return tuple(out)


def workload_inputs(w: Workload):
    return make_inputs(w.B, w.H, w.S, w.D, w.dtype, w.seed, w.qk_mult)


def sample_head_rows(n_heads, S, heads=4, per_head=64, seed=ROW_SAMPLE_SEED):
    """Seeded rows of a few heads: [(head, sorted rows)], `heads` distinct heads with
    `per_head` distinct rows each.  Every head's rows hold the ends of the sequence
    (0, 1, S-2, S-1), the edges of 32-, 256- and 512-row tiles at the start, the
    last 256-row tile edge, and random rows for the rest."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    hs = torch.randperm(n_heads, generator=g)[:min(heads, n_heads)].tolist()
    last = (S - 1) // 256 * 256
    fixed = [0, 1, 31, 32, 255, 256, 511, 512, last - 1, last, S - 2, S - 1]
    out = []
    for h in sorted(hs):
        rows = {r for r in fixed if 0 <= r < S}
        want = min(per_head, S)
        while len(rows) < want:
            rows.update(torch.randint(0, S, (want - len(rows),), generator=g).tolist())
        out.append((int(h), sorted(rows)))
    return out
