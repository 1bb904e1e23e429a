"""ctypes binding of libeagletree (include/eagletree.h).

Argument marshalling only: torch tensors become device pointers and
element strides, the current torch stream becomes the hipStream_t.  Every
step of the cycle runs in the library's HIP kernels; there is no other
code path.  If the library is not built, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libeagletree.so")

ET_OK, ET_EINVAL, ET_EUNSUPPORTED, ET_ESTATE, ET_EHIP = 0, -1, -2, -3, -4
ET_F32, ET_BF16 = 0, 1
_STATUS = {ET_EINVAL: "ET_EINVAL", ET_EUNSUPPORTED: "ET_EUNSUPPORTED",
           ET_ESTATE: "ET_ESTATE", ET_EHIP: "ET_EHIP"}

EXPORTS = ("et_plan_create", "et_plan_destroy", "et_workspace_bytes",
           "et_pool_capacity", "et_workspace_init", "et_draft_step",
           "et_rerank", "et_tree_mask", "et_rerank_mask", "et_draft_step_last",
           "et_tree_attention", "et_accept",
           "et_accept_sample", "et_kv_commit", "et_pool_export",
           "et_set_static_shape", "et_draft_step_static", "et_static_tree",
           "et_draft_step_hidden", "et_accept_noalloc", "et_check_tree",
           "et_check_prefix", "et_plan_debug", "et_last_error")


class et_config(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("depth", ctypes.c_int32),
                ("budget_n", ctypes.c_int32),
                ("expand_threshold", ctypes.c_float),
                ("logits_dtype", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("prefix_cap", ctypes.c_int32),
                ("qkv_dtype", ctypes.c_int32)]


class EtError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{_STATUS.get(code, code)}: {msg}")
        self.code = code


_lib = None


def lib():
    """Load libeagletree.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                             ctypes.c_float)
        sig = {
            "et_plan_create": ([ctypes.POINTER(et_config), ctypes.POINTER(vp)], ctypes.c_int),
            "et_plan_destroy": ([vp], ctypes.c_int),
            "et_workspace_bytes": ([vp], ctypes.c_size_t),
            "et_pool_capacity": ([vp], i32),
            "et_workspace_init": ([vp, vp, vp], ctypes.c_int),
            "et_draft_step": ([vp, vp, i32, vp, vp, i64, i64, vp, vp, vp], ctypes.c_int),
            "et_rerank": ([vp, vp, vp, vp, vp, vp, vp, vp], ctypes.c_int),
            "et_tree_mask": ([vp, vp, vp, vp, vp, vp, vp, vp], ctypes.c_int),
            "et_rerank_mask": ([vp] * 12, ctypes.c_int),
            "et_draft_step_last": ([vp, vp, vp, vp, i64, i64] + [vp] * 12, ctypes.c_int),
            "et_tree_attention": ([vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, f32, vp, vp],
                                  ctypes.c_int),
            "et_accept": ([vp, vp, vp, i64, i64, vp, vp, vp, vp, vp, vp, vp], ctypes.c_int),
            "et_accept_sample": ([vp, vp, vp, i64, i64, vp, vp, vp, f32, vp, vp, vp, vp,
                                  vp], ctypes.c_int),
            "et_accept_noalloc": ([vp, vp, i64, i64, vp, vp, vp, vp, vp, vp, vp],
                                  ctypes.c_int),
            "et_kv_commit": ([vp, vp, vp, vp, vp, vp, vp, vp, vp], ctypes.c_int),
            "et_set_static_shape": ([vp, vp, vp, i32], ctypes.c_int),
            "et_draft_step_hidden": ([vp, vp, i32, vp, vp, i64, i64, vp, i32, vp, vp, vp],
                                     ctypes.c_int),
            "et_draft_step_static": ([vp, vp, i32, vp, vp, i64, i64, vp, vp, vp], ctypes.c_int),
            "et_static_tree": ([vp, vp, vp, vp, vp, vp, vp, vp], ctypes.c_int),
            "et_pool_export": ([vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp], ctypes.c_int),
            "et_check_tree": ([vp, vp, vp, vp], ctypes.c_int),
            "et_check_prefix": ([vp, vp], ctypes.c_int),
            "et_plan_debug": ([vp], ctypes.c_int),
            "et_last_error": ([], ctypes.c_char_p),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _check(rc):
    if rc != ET_OK:
        raise EtError(rc, lib().et_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(name):
    return {"f32": ET_F32, "bf16": ET_BF16, ET_F32: ET_F32,
            ET_BF16: ET_BF16}[name]


def make_config(w) -> et_config:
    """et_config from any object with the workload attribute names."""
    return et_config(w.batch, w.vocab, w.topk, w.depth, w.budget_n,
                     float(w.threshold), _dtype_code(w.logits_dtype),
                     w.n_q_heads, w.n_kv_heads, w.head_dim, w.prefix_cap,
                     _dtype_code(w.qkv_dtype))


def et_plan_create(cfg: et_config):
    h = ctypes.c_void_p()
    _check(lib().et_plan_create(ctypes.byref(cfg), ctypes.byref(h)))
    return h


def et_plan_destroy(plan):
    _check(lib().et_plan_destroy(plan))


def et_workspace_bytes(plan) -> int:
    return int(lib().et_workspace_bytes(plan))


def et_pool_capacity(plan) -> int:
    return int(lib().et_pool_capacity(plan))


def et_workspace_init(plan, ws, stream=None):
    _check(lib().et_workspace_init(plan, _ptr(ws), _stream(stream)))


def _rows(t):
    """(batch stride, row stride) in elements of a [B][rows][V] tensor."""
    if t.stride(-1) != 1:
        raise ValueError("logits rows must be contiguous")
    return t.stride(0), t.stride(1)


def et_draft_step(plan, ws, step, root_tokens, logits, next_tokens,
                  next_count, stream=None):
    bs, rs = _rows(logits)
    _check(lib().et_draft_step(plan, _ptr(ws), int(step), _ptr(root_tokens),
                               _ptr(logits), bs, rs, _ptr(next_tokens),
                               _ptr(next_count), _stream(stream)))


def et_draft_step_static(plan, ws, step, root_tokens, logits, next_tokens,
                         next_count, stream=None):
    bs, rs = _rows(logits)
    _check(lib().et_draft_step_static(plan, _ptr(ws), int(step),
                                      _ptr(root_tokens), _ptr(logits), bs, rs,
                                      _ptr(next_tokens), _ptr(next_count),
                                      _stream(stream)))


def et_draft_step_hidden(plan, ws, step, root_tokens, hidden, lm_head,
                         next_tokens, next_count, stream=None):
    """hidden: bf16 [B][rows][H]; lm_head: bf16 [V][H], contiguous."""
    if hidden.stride(-1) != 1 or not lm_head.is_contiguous():
        raise ValueError("hidden rows and lm_head must be contiguous")
    H = int(lm_head.shape[1])
    if int(hidden.shape[-1]) != H:
        raise ValueError("hidden and lm_head disagree on the hidden size")
    _check(lib().et_draft_step_hidden(plan, _ptr(ws), int(step),
                                      _ptr(root_tokens), _ptr(hidden),
                                      hidden.stride(0), hidden.stride(1),
                                      _ptr(lm_head), H, _ptr(next_tokens),
                                      _ptr(next_count), _stream(stream)))


def et_set_static_shape(plan, parent, rank):
    """parent / rank: host int sequences for slots 1..n (parent slot 0 is
    the root)."""
    n = len(parent)
    if len(rank) != n:
        raise ValueError("parent and rank differ in length")
    pa = (ctypes.c_int32 * max(n, 1))(*[int(x) for x in parent])
    ra = (ctypes.c_int32 * max(n, 1))(*[int(x) for x in rank])
    _check(lib().et_set_static_shape(plan, pa, ra, n))


def et_static_tree(plan, ws, tokens, parent_slot, conf, value, n_kept,
                   stream=None):
    _check(lib().et_static_tree(plan, _ptr(ws), _ptr(tokens),
                                _ptr(parent_slot), _ptr(conf), _ptr(value),
                                _ptr(n_kept), _stream(stream)))


def et_rerank(plan, ws, tokens, parent_slot, conf, value, n_kept,
              stream=None):
    _check(lib().et_rerank(plan, _ptr(ws), _ptr(tokens), _ptr(parent_slot),
                           _ptr(conf), _ptr(value), _ptr(n_kept),
                           _stream(stream)))


def et_draft_step_last(plan, ws, root_tokens, logits, next_tokens, next_count,
                       prefix_len, tokens, parent_slot, conf, value, n_kept, mask,
                       depth, pos_ids, stream=None):
    bs, rs = _rows(logits)
    _check(lib().et_draft_step_last(plan, _ptr(ws), _ptr(root_tokens), _ptr(logits), bs, rs,
                                    _ptr(next_tokens), _ptr(next_count),
                                    _ptr(prefix_len), _ptr(tokens), _ptr(parent_slot),
                                    _ptr(conf), _ptr(value), _ptr(n_kept), _ptr(mask),
                                    _ptr(depth), _ptr(pos_ids), _stream(stream)))


def et_rerank_mask(plan, ws, tokens, parent_slot, conf, value, n_kept,
                   prefix_len, mask, depth, pos_ids, stream=None):
    _check(lib().et_rerank_mask(plan, _ptr(ws), _ptr(tokens), _ptr(parent_slot),
                                _ptr(conf), _ptr(value), _ptr(n_kept),
                                _ptr(prefix_len), _ptr(mask), _ptr(depth),
                                _ptr(pos_ids), _stream(stream)))


def et_tree_mask(plan, parent_slot, n_kept, prefix_len, mask, depth, pos_ids,
                 stream=None):
    _check(lib().et_tree_mask(plan, _ptr(parent_slot), _ptr(n_kept),
                              _ptr(prefix_len), _ptr(mask), _ptr(depth),
                              _ptr(pos_ids), _stream(stream)))


def et_tree_attention(plan, ws, q, k_cache, v_cache, k_tree, v_tree,
                      prefix_len, mask, n_kept, scale, out, stream=None):
    for t in (q, k_cache, v_cache, k_tree, v_tree, out):
        if not t.is_contiguous():
            raise ValueError("attention tensors must be contiguous")
    _check(lib().et_tree_attention(plan, _ptr(ws), _ptr(q), _ptr(k_cache),
                                   _ptr(v_cache), _ptr(k_tree), _ptr(v_tree),
                                   _ptr(prefix_len), _ptr(mask), _ptr(n_kept),
                                   float(scale), _ptr(out), _stream(stream)))


def et_accept(plan, ws, target_logits, tokens, parent_slot, n_kept,
              accept_len, path_slots, out_tokens, stream=None):
    bs, rs = _rows(target_logits)
    _check(lib().et_accept(plan, _ptr(ws), _ptr(target_logits), bs, rs,
                           _ptr(tokens), _ptr(parent_slot), _ptr(n_kept),
                           _ptr(accept_len), _ptr(path_slots),
                           _ptr(out_tokens), _stream(stream)))


def _host_i32(a):
    import numpy as np
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, ctypes.c_void_p(a.ctypes.data)


def et_check_tree(plan, tokens, parent_slot, n_kept):
    """Host check of a tree in et_rerank's layout (numpy arrays)."""
    keep = []
    ptrs = []
    for a in (tokens, parent_slot, n_kept):
        if a is None:
            ptrs.append(None)
        else:
            h, p = _host_i32(a)
            keep.append(h)
            ptrs.append(p)
    _check(lib().et_check_tree(plan, *ptrs))


def et_check_prefix(plan, prefix_len):
    h, p = _host_i32(prefix_len)
    _check(lib().et_check_prefix(plan, p))


def et_accept_noalloc(plan, target_logits, tokens, parent_slot, n_kept,
                      accept_len, path_slots, out_tokens, stream=None):
    bs, rs = _rows(target_logits)
    _check(lib().et_accept_noalloc(plan, _ptr(target_logits), bs, rs,
                                   _ptr(tokens), _ptr(parent_slot), _ptr(n_kept),
                                   _ptr(accept_len), _ptr(path_slots),
                                   _ptr(out_tokens), _stream(stream)))


def et_accept_sample(plan, ws, target_logits, tokens, parent_slot, n_kept,
                     temperature, uniforms, accept_len, path_slots, out_tokens,
                     stream=None):
    bs, rs = _rows(target_logits)
    if not uniforms.is_contiguous() or uniforms.dtype != torch.float32:
        raise ValueError("uniforms must be contiguous float32 [B][T]")
    _check(lib().et_accept_sample(plan, _ptr(ws), _ptr(target_logits), bs, rs,
                                  _ptr(tokens), _ptr(parent_slot),
                                  _ptr(n_kept), float(temperature),
                                  _ptr(uniforms), _ptr(accept_len),
                                  _ptr(path_slots), _ptr(out_tokens),
                                  _stream(stream)))


def et_kv_commit(plan, k_cache, v_cache, k_tree, v_tree, prefix_len,
                 path_slots, accept_len, stream=None):
    for t in (k_cache, v_cache, k_tree, v_tree):
        if not t.is_contiguous():
            raise ValueError("K/V tensors must be contiguous")
    _check(lib().et_kv_commit(plan, _ptr(k_cache), _ptr(v_cache), _ptr(k_tree),
                              _ptr(v_tree), _ptr(prefix_len), _ptr(path_slots),
                              _ptr(accept_len), _stream(stream)))


def et_pool_export(plan, ws, token=None, parent=None, depth=None, conf=None,
                   value=None, pool_count=None, frontier=None,
                   frontier_count=None, stream=None):
    _check(lib().et_pool_export(plan, _ptr(ws), _ptr(token), _ptr(parent),
                                _ptr(depth), _ptr(conf), _ptr(value),
                                _ptr(pool_count), _ptr(frontier),
                                _ptr(frontier_count), _stream(stream)))


class Plan:
    """Owns an et_plan_t, its workspace and the output buffers of a cycle."""

    def __init__(self, w, device="cuda"):
        self.w = w
        self.cfg = make_config(w)
        self.handle = et_plan_create(self.cfg)
        self.device = torch.device(device)
        nb = et_workspace_bytes(self.handle)
        self.ws = torch.empty(max(nb, 256), dtype=torch.uint8,
                              device=self.device)
        et_workspace_init(self.handle, self.ws)
        B, k, T, D = w.batch, w.topk, w.T, w.depth
        i32 = dict(dtype=torch.int32, device=self.device)
        self.cap = et_pool_capacity(self.handle)
        self.next_tokens = torch.empty((B, k), **i32)
        self.next_count = torch.empty((B,), **i32)
        self.tokens = torch.empty((B, T), **i32)
        self.parent_slot = torch.empty((B, T), **i32)
        self.conf = torch.empty((B, T), dtype=torch.float32, device=self.device)
        self.value = torch.empty((B, T), dtype=torch.float32, device=self.device)
        self.n_kept = torch.empty((B,), **i32)
        self.mask = torch.empty((B, T, w.W), dtype=torch.int64, device=self.device)
        self.depth = torch.empty((B, T), **i32)
        self.pos_ids = torch.empty((B, T), **i32)
        qdt = torch.bfloat16 if w.qkv_dtype == "bf16" else torch.float32
        self.attn_out = torch.empty((B, T, w.n_q_heads, w.head_dim),
                                    dtype=qdt, device=self.device)
        self.accept_len = torch.empty((B,), **i32)
        self.path_slots = torch.empty((B, D + 1), **i32)
        self.out_tokens = torch.empty((B, D + 1), **i32)

    def __del__(self):
        try:
            if getattr(self, "handle", None) is not None and _lib is not None:
                _lib.et_plan_destroy(self.handle)
                self.handle = None
        except Exception:
            pass

    # one call per C entry point, writing into the plan's buffers
    def draft_step(self, step, root_tokens, logits, stream=None):
        et_draft_step(self.handle, self.ws, step, root_tokens, logits,
                      self.next_tokens, self.next_count, stream)

    def rerank(self, stream=None):
        et_rerank(self.handle, self.ws, self.tokens, self.parent_slot,
                  self.conf, self.value, self.n_kept, stream)

    def draft_step_hidden(self, step, root_tokens, hidden, lm_head, stream=None):
        """Draft step from hidden states [B][rows][H] through lm_head [V][H]."""
        et_draft_step_hidden(self.handle, self.ws, step, root_tokens, hidden,
                             lm_head, self.next_tokens, self.next_count, stream)

    def set_static_shape(self, parent, rank):
        """Fixed shape for slots 1..n: parent slot and child rank each."""
        et_set_static_shape(self.handle, parent, rank)

    def draft_step_static(self, step, root_tokens, logits, stream=None):
        et_draft_step_static(self.handle, self.ws, step, root_tokens, logits,
                             self.next_tokens, self.next_count, stream)

    def static_tree(self, stream=None):
        et_static_tree(self.handle, self.ws, self.tokens, self.parent_slot,
                       self.conf, self.value, self.n_kept, stream)

    def tree_mask(self, prefix_len, stream=None):
        et_tree_mask(self.handle, self.parent_slot, self.n_kept, prefix_len,
                     self.mask, self.depth, self.pos_ids, stream)

    def draft_step_last(self, root_tokens, logits, prefix_len, stream=None):
        """draft_step(D) and rerank_mask, the rerank in the step's merge."""
        et_draft_step_last(self.handle, self.ws, root_tokens, logits, self.next_tokens,
                           self.next_count, prefix_len, self.tokens, self.parent_slot,
                           self.conf, self.value, self.n_kept, self.mask, self.depth,
                           self.pos_ids, stream)

    def rerank_mask(self, prefix_len, stream=None):
        """rerank and tree_mask in one launch (same outputs)."""
        et_rerank_mask(self.handle, self.ws, self.tokens, self.parent_slot,
                       self.conf, self.value, self.n_kept, prefix_len,
                       self.mask, self.depth, self.pos_ids, stream)

    def tree_attention(self, q, k_cache, v_cache, k_tree, v_tree, prefix_len,
                       scale=None, stream=None):
        scale = self.w.scale if scale is None else scale
        et_tree_attention(self.handle, self.ws, q, k_cache, v_cache, k_tree,
                          v_tree, prefix_len, self.mask, self.n_kept, scale,
                          self.attn_out, stream)

    def accept(self, target_logits, stream=None):
        et_accept(self.handle, self.ws, target_logits, self.tokens,
                  self.parent_slot, self.n_kept, self.accept_len,
                  self.path_slots, self.out_tokens, stream)

    def accept_noalloc(self, target_logits, stream=None):
        """et_accept on the library's fixed scratch (no workspace)."""
        et_accept_noalloc(self.handle, target_logits, self.tokens,
                          self.parent_slot, self.n_kept, self.accept_len,
                          self.path_slots, self.out_tokens, stream)

    def accept_sample(self, target_logits, temperature, uniforms, stream=None):
        """Ratio-test acceptance at temperature > 0; uniforms [B][T] f32."""
        et_accept_sample(self.handle, self.ws, target_logits, self.tokens,
                         self.parent_slot, self.n_kept, temperature, uniforms,
                         self.accept_len, self.path_slots, self.out_tokens,
                         stream)

    def kv_commit(self, k_cache, v_cache, k_tree, v_tree, prefix_len,
                  stream=None):
        """Append the last accept's path to the cache; advances prefix_len."""
        et_kv_commit(self.handle, k_cache, v_cache, k_tree, v_tree, prefix_len,
                     self.path_slots, self.accept_len, stream)

    def cycle(self, root_tokens, draft, prefix_len, attn, target,
              stream=None):
        """One whole cycle; draft is [B][D][k][V], draft[:, l] feeds step l+1."""
        for step in range(1, self.w.depth):
            self.draft_step(step, root_tokens, draft[:, step - 1], stream)
        self.draft_step_last(root_tokens, draft[:, self.w.depth - 1], prefix_len, stream)
        self.tree_attention(attn["q"], attn["k_cache"], attn["v_cache"],
                            attn["k_tree"], attn["v_tree"], prefix_len,
                            stream=stream)
        self.accept(target, stream)

    def export_pool(self, stream=None):
        B, k = self.w.batch, self.w.topk
        i32 = dict(dtype=torch.int32, device=self.device)
        out = dict(token=torch.empty((B, self.cap), **i32),
                   parent=torch.empty((B, self.cap), **i32),
                   depth=torch.empty((B, self.cap), **i32),
                   conf=torch.empty((B, self.cap), dtype=torch.float32,
                                    device=self.device),
                   value=torch.empty((B, self.cap), dtype=torch.float32,
                                     device=self.device),
                   pool_count=torch.empty((B,), **i32),
                   frontier=torch.empty((B, k), **i32),
                   frontier_count=torch.empty((B,), **i32))
        et_pool_export(self.handle, self.ws, stream=stream, **out)
        return out
