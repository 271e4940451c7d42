"""Seeded synthetic workloads for the token-pruned ViT pack -> attend -> unpack path.

This module only *generates inputs*: per-image keep masks and padded q/k/v
activations with the shapes, value distributions and pruning mixes of the
workloads on the pages (DeiT-Ti/S/B token grids of 197 = CLS + 14x14 patches,
577 = CLS + 24x24 patches at 384 px; head_dim 64).  It holds no step of the
method's arithmetic (no prefix sum, no gather, no softmax), so both the CPU
oracle tests and the HIP path can draw from it without sharing any of the
computation they are checked on.

Citations (pages on "Dispatch-Aware Ragged Attention for Pruned Vision
Transformers", arXiv 2604.15408):
  [Abstract]  the paper abstract (thelatestinai.com and mlsanity.com pages):
              ViT sequences of at most 197 tokens, 224 px and 384 px inputs,
              80 % token pruning, serving batch sizes 1-4.
  [FA2]       radpulse.milrad-way.com write-up, section on FlashAttention-2's
              62 us dispatch ceiling: DeiT-Base, 80 % pruning takes an image
              from 197 to about 39 tokens, batch 32.
  [Pipeline]  same write-up, section on the integrated packing pipeline:
              pruning-method agnostic (Threshold-l2, DynamicViT, EViT), batch
              sizes 32 and 512.

Every random draw comes from a `torch.Generator` seeded explicitly, so a
workload is a pure function of (config, seed).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
HEAD_DIM = 64
SCALE = 1.0 / math.sqrt(HEAD_DIM)  # 0.125, exact in every dtype

# Default seeds of the five named workloads.
SEEDS = {"tiny": 1, "deit_s": 2, "deit_b_sweep": 3, "deit_b_384": 4, "large_batch": 5}
SWEEP_B = (1, 2, 4)
SWEEP_P = (0.0, 0.25, 0.5, 0.8)


@dataclass
class Workload:
    """One batch: padded q/k/v [B, N, H, D] in `dtype`, keep mask uint8 [B, N]."""

    name: str
    B: int
    N: int
    H: int
    D: int
    dtype: str
    keep: torch.Tensor
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    scale: float = SCALE
    seed: int = 0
    meta: dict = field(default_factory=dict)
    # padded row indices b * N + n scaled as outliers (384 px workload), else None
    outlier_positions: torch.Tensor | None = None

    @property
    def row_elems(self) -> int:
        return self.H * self.D

    @property
    def kept_counts(self) -> list[int]:
        return [int(x) for x in (self.keep != 0).sum(dim=1).tolist()]

    @property
    def total_kept(self) -> int:
        return int((self.keep != 0).sum().item())

    def describe(self) -> dict:
        c = self.kept_counts
        return {
            "workload": self.name, "B": self.B, "N": self.N, "H": self.H,
            "head_dim": self.D, "dtype": self.dtype, "seed": self.seed,
            "total_tokens": sum(c), "max_seqlen": max(c) if c else 0,
            **self.meta,
        }


# --------------------------------------------------------------------------
# building blocks
# --------------------------------------------------------------------------
def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _normal(g: torch.Generator, shape, std: float = 1.0) -> torch.Tensor:
    x = torch.randn(shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x


def _cast(x: torch.Tensor, dtype: str) -> torch.Tensor:
    """float32 -> storage dtype (torch rounds to nearest even)."""
    return x.to(DTYPES[dtype]).contiguous()


def _round_half_up(x: float) -> int:
    return int(math.floor(x + 0.5))


def mask_from_counts(g: torch.Generator, N: int, counts) -> torch.Tensor:
    """CLS (position 0) kept; count-1 patches kept at uniformly random positions."""
    B = len(counts)
    keep = torch.zeros((B, N), dtype=torch.uint8)
    for b, c in enumerate(counts):
        c = int(c)
        if c <= 0:
            continue
        keep[b, 0] = 1
        if c > 1:
            pos = torch.randperm(N - 1, generator=g)[: c - 1] + 1
            keep[b, pos] = 1
    return keep


def mask_bernoulli(g: torch.Generator, B: int, N: int, p_keep: float) -> torch.Tensor:
    """CLS kept; every patch kept independently with probability p_keep."""
    u = torch.rand((B, N - 1), generator=g, dtype=torch.float64)
    keep = torch.ones((B, N), dtype=torch.uint8)
    keep[:, 1:] = (u < p_keep).to(torch.uint8)
    return keep


def mask_threshold_l2(g: torch.Generator, B: int, N: int, qlo=0.2, qhi=0.8):
    """Threshold-l2-shaped mask: per-token scores ~ N(0,1), each image keeps the
    patches whose score exceeds that image's own quantile, the quantile level
    drawn uniformly in [qlo, qhi]; CLS always kept.  Quantiles use linear
    interpolation between order statistics (torch's default)."""
    scores = torch.randn((B, N - 1), generator=g, dtype=torch.float64)
    levels = qlo + (qhi - qlo) * torch.rand((B,), generator=g, dtype=torch.float64)
    thr = torch.stack([torch.quantile(scores[b], levels[b]) for b in range(B)])
    keep = torch.ones((B, N), dtype=torch.uint8)
    keep[:, 1:] = (scores > thr[:, None]).to(torch.uint8)
    return keep, levels


def _qkv(g, B, N, H, D, dtype, std=1.0):
    shape = (B, N, H, D)
    return tuple(_cast(_normal(g, shape, std), dtype) for _ in range(3))


# --------------------------------------------------------------------------
# the named workloads
# --------------------------------------------------------------------------
def tiny(seed: int | None = None) -> Workload:
    """B=4, N=197, H=3 (DeiT-Ti), fp32; CLS kept, each patch kept w.p. 0.5."""
    seed = SEEDS["tiny"] if seed is None else seed
    g = _gen(seed)
    B, N, H = 4, 197, 3
    keep = mask_bernoulli(g, B, N, 0.5)
    q, k, v = _qkv(g, B, N, H, HEAD_DIM, "f32")
    return Workload("tiny", B, N, H, HEAD_DIM, "f32", keep, q, k, v, seed=seed,
                    meta={"mask": "cls+bernoulli(0.5)"})


def deit_s(seed: int | None = None, B: int = 32) -> Workload:
    """DeiT-S shape, 80 % pruning: B=32, N=197, H=6, fp16; per-image kept count
    uniform in {30..48} including CLS, kept patch positions a random subset."""
    seed = SEEDS["deit_s"] if seed is None else seed
    g = _gen(seed)
    N, H = 197, 6
    counts = torch.randint(30, 49, (B,), generator=g).tolist()
    keep = mask_from_counts(g, N, counts)
    q, k, v = _qkv(g, B, N, H, HEAD_DIM, "f16")
    return Workload("deit_s_80pct", B, N, H, HEAD_DIM, "f16", keep, q, k, v, seed=seed,
                    meta={"mask": "k~U{30..48} incl CLS", "prune": 0.8})


def sweep_kept_count(p: float) -> int:
    """Nominal kept count incl. CLS at pruning rate p of the 196 patches."""
    return _round_half_up((1.0 - p) * 196) + 1


def deit_b_sweep(B: int, p: float, seed: int | None = None,
                 exact_unpruned: bool = False) -> Workload:
    """DeiT-B serving sweep point: N=197, H=12, bf16, batch B in {1,2,4}, pruning
    rate p; kept count = nominal * (1+u), u ~ U[-0.1, 0.1], clamped to [1, 197].
    `exact_unpruned` keeps every token (no jitter)."""
    if seed is None:
        p_idx = SWEEP_P.index(p) if p in SWEEP_P else 9
        seed = 3000 + 10 * B + p_idx
    g = _gen(seed)
    N, H = 197, 12
    k0 = sweep_kept_count(p)
    if exact_unpruned:
        counts = [N] * B
    else:
        u = (torch.rand((B,), generator=g, dtype=torch.float64) * 0.2 - 0.1).tolist()
        counts = [min(N, max(1, _round_half_up(k0 * (1.0 + x)))) for x in u]
    keep = mask_from_counts(g, N, counts)
    q, k, v = _qkv(g, B, N, H, HEAD_DIM, "bf16")
    tag = "unpruned_exact" if exact_unpruned else f"p{int(round(p * 100))}"
    return Workload(f"deit_b_sweep_B{B}_{tag}", B, N, H, HEAD_DIM, "bf16", keep, q, k, v,
                    seed=seed, meta={"prune": 0.0 if exact_unpruned else p, "k0": k0})


def deit_b_384(seed: int | None = None, B: int = 64) -> Workload:
    """DeiT-B at 384 px: B=64, N=577, H=12, bf16, 50 % pruning (kept count
    uniform in {230..347} incl. CLS); q/k/v ~ N(0, 0.5^2) with 1 % of the padded
    token rows (the same positions in q, k and v) scaled by 8."""
    seed = SEEDS["deit_b_384"] if seed is None else seed
    g = _gen(seed)
    N, H = 577, 12
    counts = torch.randint(230, 348, (B,), generator=g).tolist()
    keep = mask_from_counts(g, N, counts)
    n_out = _round_half_up(0.01 * B * N)
    rows = torch.randperm(B * N, generator=g)[:n_out]
    qkv = []
    for _ in range(3):
        x = _normal(g, (B, N, H, HEAD_DIM), 0.5).view(B * N, H, HEAD_DIM)
        x[rows] *= 8.0
        qkv.append(_cast(x.view(B, N, H, HEAD_DIM), "bf16"))
    return Workload("deit_b_384_50pct", B, N, H, HEAD_DIM, "bf16", keep, *qkv, seed=seed,
                    meta={"prune": 0.5, "outlier_rows": n_out, "std": 0.5},
                    outlier_positions=rows.sort().values)


def large_batch(seed: int | None = None, B: int = 512) -> Workload:
    """Large-batch throughput: B=512, N=197, H=6, bf16; q, k and v are each a
    padded [B, 197, 384] activation ~ N(0,1); keep mask from a Threshold-l2-shaped
    rule (per-image quantile level uniform in [0.2, 0.8]), CLS forced kept."""
    seed = SEEDS["large_batch"] if seed is None else seed
    g = _gen(seed)
    N, H = 197, 6
    keep, _levels = mask_threshold_l2(g, B, N)
    q, k, v = _qkv(g, B, N, H, HEAD_DIM, "bf16")
    return Workload("large_batch_threshold_l2", B, N, H, HEAD_DIM, "bf16", keep, q, k, v,
                    seed=seed, meta={"mask": "threshold-l2 quantile U[0.2,0.8]"})


def custom(B: int, N: int, H: int, dtype: str, keep: torch.Tensor | None = None,
           p_keep: float = 0.5, std: float = 1.0, seed: int = 0, D: int = HEAD_DIM,
           scale: float = SCALE, name: str = "custom") -> Workload:
    """Free-form workload for tests: given keep mask (or CLS + Bernoulli(p_keep))."""
    g = _gen(seed)
    if keep is None:
        keep = mask_bernoulli(g, B, N, p_keep)
    keep = keep.to(torch.uint8).contiguous()
    assert keep.shape == (B, N)
    q, k, v = _qkv(g, B, N, H, D, dtype, std)
    return Workload(name, B, N, H, D, dtype, keep, q, k, v, scale=scale, seed=seed)


def by_name(name: str, **kw) -> Workload:
    table = {"tiny": tiny, "deit_s": deit_s, "deit_b_384": deit_b_384,
             "large_batch": large_batch}
    if name in table:
        return table[name](**kw)
    if name == "deit_b_sweep":
        return deit_b_sweep(**kw)
    raise KeyError(name)


def sweep_points():
    """(B, p, exact_unpruned) for every DeiT-B serving-sweep point."""
    pts = [(B, p, False) for B in SWEEP_B for p in SWEEP_P]
    pts += [(B, 0.0, True) for B in SWEEP_B]
    return pts
