"""Host-only checks of the C ABI (no GPU needed): the library loads,
exports every entry point include/eagletree.h declares, and rejects bad
arguments with the documented codes before launching anything."""
import ctypes
import os
import re

import pytest

import dynamic_draft_tree_amd as d
from dynamic_draft_tree_amd import binding
from synth import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            names |= set(re.findall(r"\b(et_[a-z_]+)\s*\(", text))
    return names


def test_library_exports_every_declared_symbol():
    L = d.lib()
    declared = _declared()
    assert {"et_draft_step", "et_rerank", "et_tree_mask", "et_tree_attention",
            "et_accept"} <= declared
    for name in declared:
        assert hasattr(L, name), name
    assert declared <= set(binding.EXPORTS)


def _cfg(**kw):
    c = d.make_config(WORKLOADS["llama8b"])
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("field,value,code", [
    ("topk", 0, binding.ET_EUNSUPPORTED), ("topk", 17, binding.ET_EUNSUPPORTED),
    ("depth", 0, binding.ET_EUNSUPPORTED), ("depth", 16, binding.ET_EUNSUPPORTED),
    ("budget_n", 0, binding.ET_EUNSUPPORTED),
    ("budget_n", 256, binding.ET_EUNSUPPORTED),
    ("vocab", 1, binding.ET_EUNSUPPORTED),
    ("vocab", (1 << 18) + 1, binding.ET_EUNSUPPORTED),
    ("head_dim", 96, binding.ET_EUNSUPPORTED),
    ("n_kv_heads", 3, binding.ET_EINVAL),
    ("n_kv_heads", 0, binding.ET_EINVAL),
    ("logits_dtype", 7, binding.ET_EUNSUPPORTED),
    ("qkv_dtype", 2, binding.ET_EUNSUPPORTED),
    ("batch", 0, binding.ET_EINVAL),
    ("prefix_cap", 0, binding.ET_EINVAL),
    ("expand_threshold", -0.5, binding.ET_EINVAL),
    ("expand_threshold", float("nan"), binding.ET_EINVAL),
])
def test_plan_rejects(field, value, code):
    with pytest.raises(binding.EtError) as e:
        d.et_plan_create(_cfg(**{field: value}))
    assert e.value.code == code
    assert field.split("_")[0] in str(e.value) or "heads" in str(e.value) \
        or "pool" in str(e.value)


def test_largest_supported_tree_is_accepted():
    """k = 16, D = 15 gives the largest pool (16 + 14 * 256 = 3600)."""
    h = d.et_plan_create(_cfg(topk=16, depth=15, budget_n=255))
    assert d.et_pool_capacity(h) == 3600
    d.et_plan_destroy(h)


def test_plan_sizes():
    for name, w in WORKLOADS.items():
        h = d.et_plan_create(d.make_config(w))
        assert d.et_pool_capacity(h) == w.pool_cap
        assert d.et_workspace_bytes(h) % 256 == 0
        d.et_plan_destroy(h)


def test_calls_validate_before_launch():
    """Null pointers, bad steps and out-of-order calls fail on the host."""
    L = d.lib()
    h = d.et_plan_create(d.make_config(WORKLOADS["tiny"]))
    fake = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced
    nul = None
    assert L.et_draft_step(h, fake, 1, fake, nul, 1024, 1024, fake, fake,
                           nul) == binding.ET_EINVAL
    assert L.et_draft_step(h, fake, 0, fake, fake, 1024, 1024, fake, fake,
                           nul) == binding.ET_EINVAL
    assert L.et_draft_step(h, fake, 4, fake, fake, 1024, 1024, fake, fake,
                           nul) == binding.ET_EINVAL
    assert L.et_draft_step(h, fake, 1, fake, fake, 1024, 1000, fake, fake,
                           nul) == binding.ET_EINVAL
    assert b"row_stride" in L.et_last_error()
    assert L.et_draft_step(h, fake, 2, fake, fake, 1024, 1024, fake, fake,
                           nul) == binding.ET_ESTATE
    assert L.et_rerank(h, fake, fake, fake, fake, fake, fake,
                       nul) == binding.ET_ESTATE
    # rerank and mask in one launch: the tree must be complete; every
    # output pointer is checked
    assert L.et_rerank_mask(h, fake, fake, fake, fake, fake, fake, fake, fake,
                            fake, fake, nul) == binding.ET_ESTATE
    assert L.et_rerank_mask(h, fake, fake, fake, fake, fake, fake, nul, fake,
                            fake, fake, nul) == binding.ET_EINVAL
    assert b"prefix_len" in L.et_last_error()
    # the last step (D = 3 for tiny) must follow step D - 1
    last = [h, fake, fake, fake, 1024, 1024, fake, fake, fake, fake, fake, fake,
            fake, fake, fake, fake, fake, nul]
    assert L.et_draft_step_last(*last) == binding.ET_ESTATE
    for i in (8, 13, 16):  # prefix_len, n_kept, pos_ids
        args = list(last)
        args[i] = nul
        assert L.et_draft_step_last(*args) == binding.ET_EINVAL, i
    assert L.et_draft_step(h, ctypes.c_void_p((1 << 20) + 8), 1, fake, fake,
                           1024, 1024, fake, fake, nul) == binding.ET_EINVAL
    assert L.et_tree_attention(h, fake, fake, fake, fake, fake, fake, fake,
                               fake, fake, ctypes.c_float(0.0), fake,
                               nul) == binding.ET_EINVAL
    assert L.et_accept(h, fake, fake, 0, 10, fake, fake, fake, fake, fake,
                       fake, nul) == binding.ET_EINVAL
    assert L.et_tree_mask(h, fake, nul, fake, fake, fake, fake,
                          nul) == binding.ET_EINVAL
    assert L.et_kv_commit(h, fake, fake, fake, fake, fake, fake, nul,
                          nul) == binding.ET_EINVAL
    assert L.et_kv_commit(h, fake, ctypes.c_void_p((1 << 20) + 4), fake, fake,
                          fake, fake, fake, nul) == binding.ET_EINVAL
    assert b"aligned" in L.et_last_error()
    f = ctypes.c_float
    assert L.et_accept_sample(h, fake, fake, 0, 1024, fake, fake, fake, f(1.0),
                              nul, fake, fake, fake, nul) == binding.ET_EINVAL
    assert L.et_accept_sample(h, fake, fake, 0, 1000, fake, fake, fake, f(1.0),
                              fake, fake, fake, fake, nul) == binding.ET_EINVAL
    # draft step from hidden states: hidden size and alignment rules
    assert L.et_draft_step_hidden(h, fake, 1, fake, fake, 0, 256, fake, 200,
                                  fake, fake, nul) == binding.ET_EUNSUPPORTED
    assert L.et_draft_step_hidden(h, fake, 1, fake, ctypes.c_void_p((1 << 20) + 8),
                                  0, 256, fake, 256, fake, fake,
                                  nul) == binding.ET_EINVAL
    assert L.et_draft_step_hidden(h, fake, 1, fake, fake, 0, 100, fake, 256,
                                  fake, fake, nul) == binding.ET_EINVAL
    # fixed shapes: tiny has topk 2, depth 3, budget 8
    i32a = lambda xs: (ctypes.c_int32 * max(len(xs), 1))(*xs)
    for par, rk in (([1], [0]), ([0], [2]), ([0, 0], [1, 1]),
                    ([0, 1, 2, 3], [0, 0, 0, 0]),
                    ([0, 0, 1, 1, 2, 3, 4, 5], [0, 1, 0, 1, 0, 0, 0, 0])):
        assert L.et_set_static_shape(h, i32a(par), i32a(rk),
                                     len(par)) == binding.ET_EINVAL, (par, rk)
    assert L.et_draft_step_static(h, fake, 1, fake, fake, 1024, 1024, fake,
                                  fake, nul) == binding.ET_ESTATE
    assert b"shape" in L.et_last_error()
    assert L.et_set_static_shape(h, i32a([0, 0, 1]), i32a([0, 1, 0]), 3) == 0
    assert L.et_static_tree(h, fake, fake, fake, fake, fake, fake,
                            nul) == binding.ET_ESTATE
    for bad in (0.0, -1.0, 1e-40, float("nan"), float("inf")):
        assert L.et_accept_sample(h, fake, fake, 0, 1024, fake, fake, fake,
                                  f(bad), fake, fake, fake, fake,
                                  nul) == binding.ET_EINVAL, bad
        assert b"temperature" in L.et_last_error()
    d.et_plan_destroy(h)


def test_accept_noalloc_rejects_plans_beyond_its_scratch():
    """The fixed scratch holds batch * T * chunks * 4 keys of 8 bytes: 300
    sequences of 61 slots over 128256 bf16 ids need 4.7 MB, more than its
    4 MiB, and the call fails before touching any pointer."""
    w = WORKLOADS["llama8b"]
    h = d.et_plan_create(d.make_config(w.with_(batch=300)))
    dummy = ctypes.c_void_p(16)  # never dereferenced: rejected on the host
    rc = binding.lib().et_accept_noalloc(h, dummy, 0, w.vocab, dummy, dummy,
                                         dummy, dummy, dummy, dummy, None)
    assert rc == binding.ET_EINVAL
    assert "scratch" in binding.lib().et_last_error().decode()
    d.et_plan_destroy(h)


def test_static_shape_validation_on_the_host():
    """et_set_static_shape (host only): the generated shape of every
    workload is accepted; shapes breaking a rule are rejected."""
    from synth import gen
    for name, w in WORKLOADS.items():
        h = d.et_plan_create(d.make_config(w))
        p, r = gen.static_shape(w)
        binding.et_set_static_shape(h, p[1:], r[1:])
        d.et_plan_destroy(h)
    w = WORKLOADS["tiny"]  # k = 2, D = 3, N = 8
    h = d.et_plan_create(d.make_config(w))
    bad = [([0], [2]),                 # rank >= k
           ([1], [0]),                 # parent not an earlier slot
           ([0, 0], [1, 1]),           # repeated sibling rank
           ([0, 1, 2, 3], [0] * 4),    # depth 4 > D
           # three depth-2 slots with children, more than k
           ([0, 0, 1, 1, 2, 3, 4, 5], [0, 1, 0, 1, 0, 0, 0, 0]),
           ([0] * 9, list(range(9)))]  # more nodes than N (and ranks >= k)
    for parent, rank in bad:
        with pytest.raises(binding.EtError) as e:
            binding.et_set_static_shape(h, parent, rank)
        assert e.value.code == binding.ET_EINVAL
    d.et_plan_destroy(h)
