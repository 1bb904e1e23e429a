"""Seeded synthetic inputs for the draft-tree cycle (numpy PCG64).

The pages measure on public chat, code and math suites with trained
models; none of that is available here.  These generators stand in for
them with logits "landscapes" of a given sharpness s, following the
explainer's demo (sharp ~ 2.5 predictable text, flat ~ 0.8 open-ended):

    row = s * N(0, 1) over the vocabulary, plus one planted token whose
    logit is raised by s * U(0, 8).

Every component of every sequence draws from its own PCG64 stream keyed
by (seed, component, sequence), so any piece can be regenerated alone.
bf16 values are produced by round-to-nearest-even from fp32 and returned
as uint16 bit patterns.  Nothing here computes any step of the method.
"""
from __future__ import annotations

import numpy as np

from .configs import Workload

# component ids of the PCG64 streams
DRAFT, TARGET, Q, KCACHE, VCACHE, KTREE, VTREE, ROOT, PREFIX = range(1, 10)


def stream(seed: int, component: int, b: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([int(seed), component, b]))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (h.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x.astype(np.float32))
    raise ValueError(dtype)


def landscape_rows(g: np.random.Generator, n_rows: int, V: int, s: float,
                   dtype: str, planted=None, boost=None) -> np.ndarray:
    """n_rows rows of s*N(0,1) with one raised token each.

    planted / boost override the drawn planted ids / boosts (tests use this
    to place the target's peak on a chosen token)."""
    x = s * g.standard_normal((n_rows, V))
    ids = g.integers(0, V, n_rows)
    up = s * g.uniform(0.0, 8.0, n_rows)
    if planted is not None:
        ids = np.asarray(planted, dtype=np.int64)
    if boost is not None:
        up = np.broadcast_to(np.asarray(boost, dtype=np.float64), (n_rows,))
    x[np.arange(n_rows), ids] += up
    return _cast(x, dtype)


def draft_logits(w: Workload, seed: int | None = None) -> np.ndarray:
    """[B][D][k][V] draft logits; step l, frontier slot j reads [b][l-1][j]."""
    seed = w.seed if seed is None else seed
    out = np.empty((w.batch, w.depth, w.topk, w.vocab),
                   dtype=np.float32 if w.logits_dtype == "f32" else np.uint16)
    for b in range(w.batch):
        g = stream(seed, DRAFT, b)
        out[b] = landscape_rows(g, w.depth * w.topk, w.vocab, w.sharpness[b],
                                w.logits_dtype).reshape(w.depth, w.topk, w.vocab)
    return out


def target_logits(w: Workload, seed: int | None = None, planted=None,
                  boost=None) -> np.ndarray:
    """[B][T][V] target logits, one row per tree slot (slot 0 = root).

    planted: optional int array [B][T] of peak tokens (-1 = draw); boost:
    optional scalar added instead of s*U(0,8) where planted is given."""
    seed = w.seed if seed is None else seed
    out = np.empty((w.batch, w.T, w.vocab),
                   dtype=np.float32 if w.logits_dtype == "f32" else np.uint16)
    for b in range(w.batch):
        g = stream(seed, TARGET, b)
        x = w.sharpness[b] * g.standard_normal((w.T, w.vocab))
        ids = g.integers(0, w.vocab, w.T)
        up = w.sharpness[b] * g.uniform(0.0, 8.0, w.T)
        if planted is not None:
            pb = np.asarray(planted[b])
            sel = pb >= 0
            ids = np.where(sel, pb, ids)
            if boost is not None:
                up = np.where(sel, boost, up)
        x[np.arange(w.T), ids] += up
        out[b] = _cast(x, w.logits_dtype)
    return out


def root_tokens(w: Workload, seed: int | None = None) -> np.ndarray:
    seed = w.seed if seed is None else seed
    return stream(seed, ROOT).integers(0, w.vocab, w.batch).astype(np.int32)


def prefix_lens(w: Workload, seed: int | None = None) -> np.ndarray:
    seed = w.seed if seed is None else seed
    lo, hi = w.prefix_range
    if lo == hi:
        return np.full(w.batch, lo, dtype=np.int32)
    return stream(seed, PREFIX).integers(lo, hi, w.batch,
                                         endpoint=True).astype(np.int32)


def _normal(seed, comp, b, shape, dtype):
    return _cast(stream(seed, comp, b).standard_normal(shape), dtype)


def attention_inputs(w: Workload, seed: int | None = None) -> dict:
    """q [B][T][Hq][d]; k_cache, v_cache [B][Hkv][P_cap][d];
    k_tree, v_tree [B][Hkv][T][d]; all N(0, 1) in qkv_dtype."""
    seed = w.seed if seed is None else seed
    dt = np.float32 if w.qkv_dtype == "f32" else np.uint16
    B, T, d = w.batch, w.T, w.head_dim
    out = {
        "q": np.empty((B, T, w.n_q_heads, d), dt),
        "k_cache": np.empty((B, w.n_kv_heads, w.prefix_cap, d), dt),
        "v_cache": np.empty((B, w.n_kv_heads, w.prefix_cap, d), dt),
        "k_tree": np.empty((B, w.n_kv_heads, T, d), dt),
        "v_tree": np.empty((B, w.n_kv_heads, T, d), dt),
    }
    comps = {"q": Q, "k_cache": KCACHE, "v_cache": VCACHE, "k_tree": KTREE,
             "v_tree": VTREE}
    for b in range(B):
        for name, comp in comps.items():
            out[name][b] = _normal(seed, comp, b, out[name].shape[1:],
                                   w.qkv_dtype)
    return out


TIED, TIED_TARGET = 13, 14


def _tied_rows(g: np.random.Generator, n_rows: int, V: int, s: float) -> np.ndarray:
    """fp32 rows full of exact ties, by row index r mod 4: 0: every logit
    0; 1: N(0,1) / 2 rounded to integers (about 16% of a row share the
    largest common value); 2: N(0,1) with the value 6 at max(300, V/64)
    random ids; 3: the landscape of draft_logits."""
    rows = landscape_rows(g, n_rows, V, s, "f32")
    for r in range(n_rows):
        kind = r % 4
        if kind == 0:
            rows[r] = 0.0
        elif kind == 1:
            rows[r] = np.rint(0.5 * g.standard_normal(V))
        elif kind == 2:
            x = g.standard_normal(V).astype(np.float32)
            x[g.choice(V, size=min(V, max(300, V // 64)), replace=False)] = 6.0
            rows[r] = x
    return rows


def tied_draft_logits(w: Workload, seed: int | None = None) -> np.ndarray:
    """[B][D][k][V] draft logits of _tied_rows (row index = layer * k +
    frontier slot).  Values are rounded to the workload's dtype like
    draft_logits; the integers are exact in both, so the ties survive."""
    seed = w.seed if seed is None else seed
    out = np.empty((w.batch, w.depth, w.topk, w.vocab),
                   dtype=np.float32 if w.logits_dtype == "f32" else np.uint16)
    for b in range(w.batch):
        rows = _tied_rows(stream(seed, TIED, b), w.depth * w.topk, w.vocab,
                          w.sharpness[b])
        out[b] = _cast(rows, w.logits_dtype).reshape(w.depth, w.topk, w.vocab)
    return out


def tied_target_logits(w: Workload, seed: int | None = None) -> np.ndarray:
    """[B][T][V] target logits of _tied_rows (row index = slot)."""
    seed = w.seed if seed is None else seed
    out = np.empty((w.batch, w.T, w.vocab),
                   dtype=np.float32 if w.logits_dtype == "f32" else np.uint16)
    for b in range(w.batch):
        rows = _tied_rows(stream(seed, TIED_TARGET, b), w.T, w.vocab,
                          w.sharpness[b])
        out[b] = _cast(rows, w.logits_dtype)
    return out


LM_HIDDEN, LM_WEIGHT = 11, 12


def lm_head_inputs(w: Workload, hidden: int, seed: int | None = None) -> dict:
    """Synthetic draft-model hidden states and LM head (bf16 bits): rows
    [B][D][k][H] ~ s_b * N(0, 1) per sequence, weight [V][H] ~ N(0, 1/H),
    so every logit row is again an s_b * N(0, 1) landscape (no planted
    token).  The weight is drawn in blocks of 4096 vocab rows."""
    seed = w.seed if seed is None else seed
    h = np.empty((w.batch, w.depth, w.topk, hidden), np.uint16)
    for b in range(w.batch):
        g = stream(seed, LM_HIDDEN, b)
        x = g.standard_normal((w.depth, w.topk, hidden), dtype=np.float32)
        h[b] = f32_to_bf16_bits(x * np.float32(w.sharpness[b]))
    W = np.empty((w.vocab, hidden), np.uint16)
    g = stream(seed, LM_WEIGHT)
    scale = np.float32(1.0 / np.sqrt(hidden))
    for v0 in range(0, w.vocab, 4096):
        v1 = min(w.vocab, v0 + 4096)
        W[v0:v1] = f32_to_bf16_bits(
            g.standard_normal((v1 - v0, hidden), dtype=np.float32) * scale)
    return dict(hidden=h, lm_head=W)


def static_shape(w: Workload, q0: float = 0.6, decay: float = 0.4):
    """A fixed tree shape of w.budget_n nodes for the static-tree baseline:
    nodes taken best first by the product, along their path, of a fixed
    per-rank weight q_r = q0 * decay^r (rank r < k, depth <= D, at most k
    nodes with children per depth); ties go to the earlier-created
    candidate.  Returns (parent, rank), int32 [M + 1] in slot order (entry
    0 is the root)."""
    import heapq
    k, D, N = w.topk, w.depth, w.budget_n
    parent, rank, depth, weight = [-1], [-1], [0], [1.0]
    expanded = [0] * (D + 1)      # nodes with a child, per depth
    has_child = [False]
    heap, made = [], 0

    def offer(p):
        nonlocal made
        if depth[p] >= D:
            return
        for r in range(k):
            heapq.heappush(heap, (-weight[p] * q0 * decay ** r, made, p, r))
            made += 1

    offer(0)
    while heap and len(parent) - 1 < N:
        _, _, p, r = heapq.heappop(heap)
        if not has_child[p]:
            if expanded[depth[p]] >= k:
                continue
            expanded[depth[p]] += 1
            has_child[p] = True
        parent.append(p)
        rank.append(r)
        depth.append(depth[p] + 1)
        weight.append(weight[p] * q0 * decay ** r)
        has_child.append(False)
        offer(len(parent) - 1)
    return np.array(parent, np.int32), np.array(rank, np.int32)
