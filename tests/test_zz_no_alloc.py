"""et_accept_noalloc (no workspace: the library's fixed per-device scratch)
against et_accept (workspace) on the same inputs, through the C ABI: two
calls in a row, the second with a smaller input, so stale keys from the
first call sit in the scratch when the second runs.  Outputs must be bit
for bit those of et_accept."""
import numpy as np
import pytest
import torch

import dynamic_draft_tree_amd as d
from gpu_util import dev_inputs, make_inputs, random_path_targets, to_dev
from synth import WORKLOADS, gen

pytestmark = pytest.mark.gpu

SMALL = WORKLOADS["tiny"].with_(batch=3, vocab=5000, topk=4, depth=4,
                                budget_n=20, threshold=0.0, logits_dtype="bf16",
                                sharpness=(0.8, 1.5, 2.5), n_q_heads=8,
                                n_kv_heads=2, head_dim=128, prefix_cap=300,
                                prefix_range=(1, 300), qkv_dtype="bf16", seed=21)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    d.lib()  # fail loudly if the library is missing


def _tree_and_targets(w):
    """A built tree (one whole cycle) and target logits whose peaks follow
    random kept paths, so the walks are long."""
    inp = make_inputs(w)
    dev = dev_inputs(inp)
    plan = d.Plan(w)
    plan.cycle(dev["root_tokens"], dev["draft"], dev["prefix_len"], dev["attn"],
               dev["target"])
    torch.cuda.synchronize()
    rr = dict(tokens=plan.tokens.cpu().numpy(),
              parent_slot=plan.parent_slot.cpu().numpy(),
              n_kept=plan.n_kept.cpu().numpy())
    planted = random_path_targets(w, rr, np.random.default_rng(w.seed))
    target = to_dev(gen.target_logits(w, planted=planted, boost=300.0))
    return plan, target


def test_accept_noalloc_equals_accept_on_two_calls():
    for w in (WORKLOADS["llama8b"], SMALL):  # the second input is smaller
        print(f"[no_alloc] {w.name}: batch {w.batch}, vocab {w.vocab}, T {w.T}",
              flush=True)
        plan, target = _tree_and_targets(w)
        plan.accept(target)
        torch.cuda.synchronize()
        ref = [t.clone() for t in (plan.accept_len, plan.path_slots, plan.out_tokens)]
        for t in (plan.accept_len, plan.path_slots, plan.out_tokens):
            t.fill_(-7)
        plan.accept_noalloc(target)
        torch.cuda.synchronize()
        for a, t in zip(ref, (plan.accept_len, plan.path_slots, plan.out_tokens)):
            assert torch.equal(a, t)
        assert int(plan.accept_len.max()) > 0  # the walks go somewhere
        del plan, target
