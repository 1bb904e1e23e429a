"""CPU oracle of the EAGLE-2 draft-tree cycle -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and the CPU-baseline leg of bench.py may use
this package.  It marshals numpy arrays into liboracle_eagletree.so (plain
C in eagletree_ref.c, fp64) and shares no code with the HIP library.

Every function here is pinned by tests/test_oracle_pins.py against facts
the pages or the mathematics fix (library routines on special cases,
closed forms, the explainer's chain example, brute force, invariants);
none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "eagletree_ref.c")
_SO = os.path.join(_HERE, "liboracle_eagletree.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
             "-ffp-contract=off", "-fno-fast-math", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        _lib = ctypes.CDLL(_SO)
        _lib.etref_attention_row.restype = None
        _lib.etref_tree_attention.restype = None
        _lib.etref_kv_commit.restype = None
        _lib.etref_set_num_threads.restype = None
    return _lib


_DT = {"f32": 0, "bf16": 1}


def _p(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


class TreeState:
    """Pool and frontier of every sequence between draft steps."""

    def __init__(self, w):
        B, cap, k = w.batch, w.pool_cap, w.topk
        self.w = w
        self.token = np.full((B, cap), -1, np.int32)
        self.parent = np.full((B, cap), -1, np.int32)
        self.depth = np.full((B, cap), -1, np.int32)
        self.conf = np.zeros((B, cap), np.float32)
        self.value = np.zeros((B, cap), np.float32)
        self.count = np.zeros(B, np.int32)
        self.root = np.zeros(B, np.int32)
        self.frontier = np.full((B, k), -1, np.int32)
        self.frontier_count = np.zeros(B, np.int32)

    def copy(self) -> "TreeState":
        c = TreeState.__new__(TreeState)
        c.w = self.w
        for name in ("token", "parent", "depth", "conf", "value", "count",
                     "root", "frontier", "frontier_count"):
            setattr(c, name, getattr(self, name).copy())
        return c


def _rows(a: np.ndarray):
    """(pointer, batch stride, row stride) in elements of a [B][rows][V]
    array whose last axis is contiguous."""
    if a.strides[-1] != a.itemsize:
        raise ValueError("last axis must be contiguous")
    return _p(a), a.strides[0] // a.itemsize, a.strides[1] // a.itemsize


def draft_step(w, st: TreeState, step: int, root_tokens, logits):
    """One expansion layer.  logits: [B][rows>=F][V] (f32 or bf16 bits)."""
    root_tokens = _i32(root_tokens)
    ptr, bs, rs = _rows(logits)
    nt = np.full((w.batch, w.topk), -1, np.int32)
    nc = np.zeros(w.batch, np.int32)
    rc = lib().etref_draft_step(
        w.batch, w.vocab, w.topk, w.depth, ctypes.c_float(w.threshold),
        _DT[w.logits_dtype], step, _p(root_tokens), ptr, ctypes.c_int64(bs),
        ctypes.c_int64(rs), w.pool_cap, _p(st.token), _p(st.parent),
        _p(st.depth), _p(st.conf), _p(st.value), _p(st.count), _p(st.root),
        _p(st.frontier), _p(st.frontier_count), _p(nt), _p(nc))
    if rc != 0:
        raise RuntimeError(f"etref_draft_step failed: {rc}")
    return nt, nc


def build_tree(w, root_tokens, draft, st: TreeState | None = None):
    """Run steps 1..D with draft[b][step-1][j] as frontier row j."""
    st = TreeState(w) if st is None else st
    for step in range(1, w.depth + 1):
        draft_step(w, st, step, root_tokens, draft[:, step - 1])
    return st


def rerank(w, st: TreeState):
    B, T = w.batch, w.T
    tokens = np.empty((B, T), np.int32)
    parent = np.empty((B, T), np.int32)
    conf = np.empty((B, T), np.float32)
    value = np.empty((B, T), np.float32)
    n_kept = np.empty(B, np.int32)
    rc = lib().etref_rerank(
        B, w.topk, w.depth, w.budget_n, w.pool_cap, _p(st.token),
        _p(st.parent), _p(st.depth), _p(st.conf), _p(st.value), _p(st.count),
        _p(st.root), _p(tokens), _p(parent), _p(conf), _p(value), _p(n_kept))
    if rc != 0:
        raise RuntimeError(f"etref_rerank failed: {rc}")
    return dict(tokens=tokens, parent_slot=parent, conf=conf, value=value,
                n_kept=n_kept)


def tree_mask(w, parent_slot, n_kept, prefix_len):
    B, T, W = w.batch, w.T, w.W
    parent_slot, n_kept, prefix_len = map(_i32, (parent_slot, n_kept,
                                                 prefix_len))
    mask = np.zeros((B, T, W), np.uint64)
    depth = np.empty((B, T), np.int32)
    pos = np.empty((B, T), np.int32)
    rc = lib().etref_tree_mask(B, w.budget_n, _p(parent_slot), _p(n_kept),
                               _p(prefix_len), _p(mask), _p(depth), _p(pos))
    if rc != 0:
        raise RuntimeError(f"etref_tree_mask failed: {rc}")
    return dict(mask=mask, depth=depth, pos_ids=pos)


def _attn_args(w, inp, prefix_len, mask, n_kept):
    arrs = [np.ascontiguousarray(inp[n]) for n in
            ("q", "k_cache", "v_cache", "k_tree", "v_tree")]
    prefix_len, n_kept = _i32(prefix_len), _i32(n_kept)
    mask = np.ascontiguousarray(mask, dtype=np.uint64)
    keep = arrs + [prefix_len, mask, n_kept]
    head = (w.batch, w.T, w.n_q_heads, w.n_kv_heads, w.head_dim,
            w.prefix_cap, _DT[w.qkv_dtype])
    ptrs = [_p(a) for a in arrs] + [_p(prefix_len), _p(mask), _p(n_kept)]
    return head, ptrs, keep


def tree_attention(w, inp, prefix_len, mask, n_kept, scale=None):
    """All rows, fp64 [B][T][Hq][d]."""
    scale = w.scale if scale is None else scale
    head, ptrs, keep = _attn_args(w, inp, prefix_len, mask, n_kept)
    out = np.zeros((w.batch, w.T, w.n_q_heads, w.head_dim), np.float64)
    lib().etref_tree_attention(*head, *ptrs, ctypes.c_double(scale), _p(out))
    del keep
    return out


def attention_rows(w, inp, prefix_len, mask, n_kept, rows, scale=None):
    """Selected (b, s, h) rows only, fp64 [len(rows)][d]."""
    scale = w.scale if scale is None else scale
    head, ptrs, keep = _attn_args(w, inp, prefix_len, mask, n_kept)
    out = np.zeros((len(rows), w.head_dim), np.float64)
    for i, (b, s, h) in enumerate(rows):
        lib().etref_attention_row(*head, *ptrs, ctypes.c_double(scale),
                                  int(b), int(s), int(h),
                                  _p(out[i:i + 1]))
    del keep
    return out


def accept(w, target, tokens, parent_slot, n_kept):
    B, D = w.batch, w.depth
    ptr, bs, rs = _rows(target)
    tokens, parent_slot, n_kept = map(_i32, (tokens, parent_slot, n_kept))
    alen = np.empty(B, np.int32)
    path = np.empty((B, D + 1), np.int32)
    otok = np.empty((B, D + 1), np.int32)
    rc = lib().etref_accept(B, w.T, w.vocab, D, _DT[w.logits_dtype], ptr,
                            ctypes.c_int64(bs), ctypes.c_int64(rs),
                            _p(tokens), _p(parent_slot), _p(n_kept),
                            _p(alen), _p(path), _p(otok))
    if rc != 0:
        raise RuntimeError(f"etref_accept failed: {rc}")
    return dict(accept_len=alen, path_slots=path, out_tokens=otok)


def accept_sample(w, target, tokens, parent_slot, n_kept, temperature,
                  uniforms):
    """Stochastic acceptance at temperature > 0 (see etref_accept_sample);
    uniforms is fp32 [B][T] in [0, 1).  Also returns the smallest decision
    margin per sequence (relative to the row's total target mass)."""
    B, D = w.batch, w.depth
    ptr, bs, rs = _rows(target)
    tokens, parent_slot, n_kept = map(_i32, (tokens, parent_slot, n_kept))
    u = np.ascontiguousarray(uniforms, dtype=np.float32)
    assert u.shape == (B, w.T)
    alen = np.empty(B, np.int32)
    path = np.empty((B, D + 1), np.int32)
    otok = np.empty((B, D + 1), np.int32)
    margin = np.empty(B, np.float64)
    rc = lib().etref_accept_sample(
        B, w.T, w.vocab, D, _DT[w.logits_dtype], ptr, ctypes.c_int64(bs),
        ctypes.c_int64(rs), _p(tokens), _p(parent_slot), _p(n_kept),
        ctypes.c_double(float(temperature)), _p(u), _p(alen), _p(path),
        _p(otok), _p(margin))
    if rc != 0:
        raise RuntimeError(f"etref_accept_sample failed: {rc}")
    return dict(accept_len=alen, path_slots=path, out_tokens=otok,
                margin=margin)


def static_tree(w, root_tokens, draft, shape_parent, shape_rank):
    """The fixed-shape tree (see etref_static_tree) on draft logits
    [B][D][k][V]; shape_parent / shape_rank are [M + 1] with entry 0 (the
    root) ignored.  Returns the rerank-style slot arrays."""
    B, T = w.batch, w.T
    if draft.strides[-1] != draft.itemsize:
        raise ValueError("last axis must be contiguous")
    es = draft.itemsize
    bs, ls, rs = (draft.strides[0] // es, draft.strides[1] // es,
                  draft.strides[2] // es)
    sp, sr = _i32(shape_parent), _i32(shape_rank)
    M = len(sp) - 1
    out = dict(tokens=np.empty((B, T), np.int32),
               parent_slot=np.empty((B, T), np.int32),
               conf=np.empty((B, T), np.float32),
               value=np.empty((B, T), np.float32),
               n_kept=np.empty(B, np.int32))
    rc = lib().etref_static_tree(
        B, w.vocab, w.topk, w.depth, T, _DT[w.logits_dtype],
        _p(_i32(root_tokens)), _p(draft), ctypes.c_int64(bs),
        ctypes.c_int64(ls), ctypes.c_int64(rs), M, _p(sp), _p(sr),
        _p(out["tokens"]), _p(out["parent_slot"]), _p(out["conf"]),
        _p(out["value"]), _p(out["n_kept"]))
    if rc != 0:
        raise ValueError(f"etref_static_tree rejected the shape: {rc}")
    return out


def lm_head_logits(hidden_bits, weight_bits, block=8192):
    """Logits of a draft step taken from hidden states: fp64 sums of the
    exact bf16 products, logits[..., v] = sum_h hidden[..., h] * W[v, h]
    (the draft model reusing the target's LM head).  hidden_bits
    [..., H] and weight_bits [V][H] are bf16 bit patterns; the vocab is
    done in blocks to bound memory.  Returns fp64 [..., V]."""
    def widen(bits):  # bf16 bits -> exact fp64
        return (np.asarray(bits).astype(np.uint32) << np.uint32(16)).view(
            np.float32).astype(np.float64)

    h = widen(hidden_bits)
    V = weight_bits.shape[0]
    out = np.empty(h.shape[:-1] + (V,), np.float64)
    for v0 in range(0, V, block):
        v1 = min(V, v0 + block)
        out[..., v0:v1] = h @ widen(weight_bits[v0:v1]).T
    return out


def kv_commit(w, attn, prefix_len, path_slots, accept_len):
    """Commit the accepted paths to copies of the K/V caches (see
    etref_kv_commit); returns (k_cache, v_cache, prefix_len)."""
    kc = np.array(attn["k_cache"], copy=True, order="C")
    vc = np.array(attn["v_cache"], copy=True, order="C")
    kt = np.ascontiguousarray(attn["k_tree"])
    vt = np.ascontiguousarray(attn["v_tree"])
    plen = np.array(prefix_len, dtype=np.int32, copy=True)
    path, alen = _i32(path_slots), _i32(accept_len)
    lib().etref_kv_commit(w.batch, w.T, w.n_kv_heads, w.head_dim, w.prefix_cap,
                          w.depth, kc.dtype.itemsize, _p(kc), _p(vc), _p(kt),
                          _p(vt), _p(plen), _p(path), _p(alen))
    return kc, vc, plen


def num_threads() -> int:
    return int(lib().etref_num_threads())


def set_num_threads(n: int) -> None:
    """Cap the threads of the attention loop (OpenMP)."""
    lib().etref_set_num_threads(int(n))


def cycle(w, inputs: dict):
    """One whole cycle on generated inputs (see synth.gen)."""
    st = build_tree(w, inputs["root_tokens"], inputs["draft"])
    rr = rerank(w, st)
    mk = tree_mask(w, rr["parent_slot"], rr["n_kept"], inputs["prefix_len"])
    att = tree_attention(w, inputs["attn"], inputs["prefix_len"], mk["mask"],
                         rr["n_kept"])
    acc = accept(w, inputs["target"], rr["tokens"], rr["parent_slot"],
                 rr["n_kept"])
    return dict(state=st, rerank=rr, mask=mk, attention=att, accept=acc)
