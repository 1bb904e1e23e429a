"""Debug mode (ET_DEBUG) and the host checks of the device data the calls
expect.  The checks are tested on host arrays (no GPU): a tree the
oracle's rerank produced passes, and each planted violation of the
documented layout is rejected with ET_EINVAL and a message naming it.  On
a GPU, a whole cycle runs in debug mode, and corrupted n_kept or prefix
lengths are rejected before anything is launched."""
import os

import numpy as np
import pytest

import dynamic_draft_tree_amd as d
import oracle
from dynamic_draft_tree_amd import binding
from synth import WORKLOADS, gen

W = WORKLOADS["tiny"].with_(batch=2, vocab=2000, topk=3, depth=4, budget_n=12,
                            threshold=0.0, sharpness=(1.0, 2.5), seed=31)


def _tree():
    inp = dict(root_tokens=gen.root_tokens(W), draft=gen.draft_logits(W))
    st = oracle.build_tree(W, inp["root_tokens"], inp["draft"])
    return oracle.rerank(W, st)


@pytest.fixture()
def plan():
    h = d.et_plan_create(d.make_config(W))
    yield h
    d.et_plan_destroy(h)


def test_rerank_output_passes(plan):
    rr = _tree()
    binding.et_check_tree(plan, rr["tokens"], rr["parent_slot"], rr["n_kept"])
    binding.et_check_tree(plan, None, rr["parent_slot"], rr["n_kept"])
    binding.et_check_prefix(plan, np.array([0, W.prefix_cap], np.int32))


@pytest.mark.parametrize("case", [
    ("n_kept", lambda r: r["n_kept"].__setitem__(0, W.budget_n + 1)),
    ("n_kept", lambda r: r["n_kept"].__setitem__(1, -1)),
    ("parent_slot", lambda r: r["parent_slot"].__setitem__((0, 0), 0)),   # root
    ("parent_slot", lambda r: r["parent_slot"].__setitem__((0, 3), 3)),   # not earlier
    ("parent_slot", lambda r: r["parent_slot"].__setitem__((1, 2), -1)),  # kept, no parent
    # the last kept slot (a leaf: rank order is topological) turned into a
    # pad slot that still names a parent
    ("parent_slot", lambda r: r["n_kept"].__setitem__(0, r["n_kept"][0] - 1)),
    ("tokens", lambda r: r["tokens"].__setitem__((1, 1), W.vocab)),
    ("tokens", lambda r: r["tokens"].__setitem__((0, 0), -1)),
], ids=lambda c: c[0])
def test_planted_violations_are_rejected(plan, case):
    field, mutate = case
    rr = {k: np.array(v, copy=True) for k, v in _tree().items()}
    mutate(rr)
    with pytest.raises(binding.EtError) as e:
        binding.et_check_tree(plan, rr["tokens"], rr["parent_slot"], rr["n_kept"])
    assert e.value.code == binding.ET_EINVAL
    assert field in str(e.value)


def test_pad_token_must_be_minus_one(plan):
    rr = {k: np.array(v, copy=True) for k, v in _tree().items()}
    rr["n_kept"][0] = min(int(rr["n_kept"][0]), W.budget_n - 1)
    s = int(rr["n_kept"][0]) + 1  # first pad slot
    rr["parent_slot"][0, s:] = -1
    rr["tokens"][0, s:] = -1
    binding.et_check_tree(plan, rr["tokens"], rr["parent_slot"], rr["n_kept"])
    rr["tokens"][0, s] = 5
    with pytest.raises(binding.EtError, match="tokens"):
        binding.et_check_tree(plan, rr["tokens"], rr["parent_slot"], rr["n_kept"])


@pytest.mark.parametrize("bad", [-1, W.prefix_cap + 1])
def test_prefix_out_of_range_is_rejected(plan, bad):
    with pytest.raises(binding.EtError, match="prefix_len"):
        binding.et_check_prefix(plan, np.array([3, bad], np.int32))


@pytest.mark.parametrize("value,on", [("1", 1), ("0", 0), (None, 0)])
def test_debug_mode_is_read_at_plan_creation(monkeypatch, value, on):
    if value is None:
        monkeypatch.delenv("ET_DEBUG", raising=False)
    else:
        monkeypatch.setenv("ET_DEBUG", value)
    h = d.et_plan_create(d.make_config(W))
    assert binding.lib().et_plan_debug(h) == on
    d.et_plan_destroy(h)


@pytest.mark.gpu
def test_cycle_in_debug_mode(monkeypatch):
    """A whole cycle passes every debug check; corrupted n_kept (beyond N)
    or prefix lengths (beyond the cache) are rejected before a launch."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    from gpu_util import dev_inputs, make_inputs
    monkeypatch.setenv("ET_DEBUG", "1")
    w = W.with_(logits_dtype="bf16", qkv_dtype="bf16", head_dim=128,
                n_q_heads=4, n_kv_heads=2, prefix_cap=200, prefix_range=(50, 200))
    dev = dev_inputs(make_inputs(w))
    plan = d.Plan(w)
    assert binding.lib().et_plan_debug(plan.handle) == 1
    plan.cycle(dev["root_tokens"], dev["draft"], dev["prefix_len"], dev["attn"],
               dev["target"])
    torch.cuda.synchronize()
    a = dev["attn"]
    good = plan.n_kept.clone()
    plan.n_kept.fill_(w.budget_n + 3)
    with pytest.raises(binding.EtError, match="n_kept"):
        plan.tree_attention(a["q"], a["k_cache"], a["v_cache"], a["k_tree"],
                            a["v_tree"], dev["prefix_len"])
    plan.n_kept.copy_(good)
    with pytest.raises(binding.EtError, match="prefix_len"):
        plan.tree_mask(dev["prefix_len"] + w.prefix_cap)
    plan.tree_mask(dev["prefix_len"])
    torch.cuda.synchronize()
    assert os.environ["ET_DEBUG"] == "1"
