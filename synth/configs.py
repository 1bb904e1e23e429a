"""Workload shapes for one draft-tree build + verify cycle.

Each workload is a batch of independent sequences with the tree knobs of
the pages (top-k, depth, budget N, expand threshold) and the attention
shape of the target model.  Sources for the knobs: EAGLE-2 summary page
App. A (N = 60 draft tokens at 7B/8B, depth 6, 10 expansion nodes);
EAGLE notes, "EAGLE 2 / 方法" Expand stage (threshold 0.1 with k = 2,
N = 8); explainer "Watch the Budget Being Spent" (context sharpness about
2.5 for predictable text and about 0.8 for open-ended text).

This module holds shapes and seeds only; no step of the method.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    vocab: int
    topk: int
    depth: int
    budget_n: int
    threshold: float
    logits_dtype: str                  # "f32" or "bf16"
    sharpness: tuple                   # per-sequence s, len == batch
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    prefix_cap: int
    prefix_range: tuple                # (lo, hi) inclusive; lo == hi: fixed
    qkv_dtype: str
    seed: int
    note: str = field(default="", compare=False)

    @property
    def T(self) -> int:
        return self.budget_n + 1

    @property
    def W(self) -> int:
        return (self.T + 63) // 64

    @property
    def pool_cap(self) -> int:
        return self.topk + (self.depth - 1) * self.topk * self.topk

    @property
    def G(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        if "batch" in kw and "sharpness" not in kw:
            s = self.sharpness
            d["sharpness"] = tuple(s[i % len(s)] for i in range(kw["batch"]))
        return Workload(**d)


def _uniform(b, s):
    return tuple([s] * b)


WORKLOADS = {
    # fp32 correctness case with the threshold rule switched on.
    "tiny": Workload(
        "tiny", batch=1, vocab=1024, topk=2, depth=3, budget_n=8,
        threshold=0.1, logits_dtype="f32", sharpness=_uniform(1, 1.5),
        n_q_heads=1, n_kv_heads=1, head_dim=64, prefix_cap=64,
        prefix_range=(64, 64), qkv_dtype="f32", seed=0),
    "vicuna7b_flat": Workload(
        "vicuna7b_flat", batch=1, vocab=32000, topk=10, depth=6, budget_n=60,
        threshold=0.0, logits_dtype="bf16", sharpness=_uniform(1, 0.8),
        n_q_heads=32, n_kv_heads=32, head_dim=128, prefix_cap=1024,
        prefix_range=(1024, 1024), qkv_dtype="bf16", seed=1),
    "vicuna7b_sharp": Workload(
        "vicuna7b_sharp", batch=1, vocab=32000, topk=10, depth=6, budget_n=60,
        threshold=0.0, logits_dtype="bf16", sharpness=_uniform(1, 2.5),
        n_q_heads=32, n_kv_heads=32, head_dim=128, prefix_cap=1024,
        prefix_range=(1024, 1024), qkv_dtype="bf16", seed=2),
    # The headline shape: Llama-3.1-8B, batch 1.
    "llama8b": Workload(
        "llama8b", batch=1, vocab=128256, topk=10, depth=8, budget_n=60,
        threshold=0.0, logits_dtype="bf16", sharpness=_uniform(1, 2.5),
        n_q_heads=32, n_kv_heads=8, head_dim=128, prefix_cap=4096,
        prefix_range=(4096, 4096), qkv_dtype="bf16", seed=3),
    # Batch 64, ragged prefixes; sequences b < 32 flat, b >= 32 sharp.
    "llama8b_b64": Workload(
        "llama8b_b64", batch=64, vocab=128256, topk=8, depth=6, budget_n=32,
        threshold=0.0, logits_dtype="bf16",
        sharpness=tuple([0.8] * 32 + [2.5] * 32),
        n_q_heads=32, n_kv_heads=8, head_dim=128, prefix_cap=4096,
        prefix_range=(512, 4096), qkv_dtype="bf16", seed=4),
    "llama70b_b8": Workload(
        "llama70b_b8", batch=8, vocab=128256, topk=10, depth=8, budget_n=60,
        threshold=0.0, logits_dtype="bf16", sharpness=_uniform(8, 2.5),
        n_q_heads=64, n_kv_heads=8, head_dim=128, prefix_cap=16384,
        prefix_range=(16384, 16384), qkv_dtype="bf16", seed=5),
}

HEADLINE = "llama8b"
