"""Saved cycles (tests/golden/replays/*.npz, written by
tests/golden/make_replays.py from seeded inputs and the oracle): the
oracle reproduces the stored outputs exactly, and on a GPU the library's
cycle on the stored inputs matches them to the parity bars (ids, masks
and paths bit-exact; conf and value within 1e-5 relative; attention within
1e-2 max-abs for bf16 inputs, 1e-4 for fp32).  A GPU parity test that
fails saves its inputs the same way (tests/conftest.py), so the case can
be kept here and run again."""
import glob
import os

import numpy as np
import pytest

import oracle
import replay

HERE = os.path.dirname(os.path.abspath(__file__))
REPLAYS = sorted(glob.glob(os.path.join(HERE, "golden", "replays", "*.npz")))
EXACT = ("tokens", "parent_slot", "n_kept", "mask", "depth", "pos_ids",
         "accept_len", "path_slots", "out_tokens")


def test_there_are_replays():
    assert len(REPLAYS) >= 2


@pytest.mark.parametrize("path", REPLAYS, ids=os.path.basename)
def test_oracle_reproduces_saved_outputs(path):
    w, inputs, expected = replay.load(path)
    got = replay.oracle_outputs(w, inputs)
    assert set(expected) == set(got)
    for k, v in expected.items():
        np.testing.assert_array_equal(got[k], v, err_msg=k)


@pytest.mark.gpu
@pytest.mark.parametrize("path", REPLAYS, ids=os.path.basename)
def test_gpu_cycle_on_saved_inputs(path):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import dynamic_draft_tree_amd as d
    from gpu_util import ATTN_TOL_BF16, ATTN_TOL_F32, bf16_dev_to_f64, dev_inputs, rel_close
    w, inputs, expected = replay.load(path)
    dev = dev_inputs(inputs)
    plan = d.Plan(w)
    plan.cycle(dev["root_tokens"], dev["draft"], dev["prefix_len"], dev["attn"],
               dev["target"])
    torch.cuda.synchronize()
    got = dict(tokens=plan.tokens, parent_slot=plan.parent_slot, n_kept=plan.n_kept,
               mask=plan.mask, depth=plan.depth, pos_ids=plan.pos_ids,
               accept_len=plan.accept_len, path_slots=plan.path_slots,
               out_tokens=plan.out_tokens)
    for k in EXACT:
        g = got[k].cpu().numpy()
        if k == "mask":
            g = g.view(np.uint64)
        np.testing.assert_array_equal(g, expected[k], err_msg=k)
    for k in ("conf", "value"):
        assert rel_close(getattr(plan, k).cpu().numpy(), expected[k]).all(), k
    if w.qkv_dtype == "bf16":
        out, tol = bf16_dev_to_f64(plan.attn_out), ATTN_TOL_BF16
    else:
        out, tol = plan.attn_out.cpu().numpy().astype(np.float64), ATTN_TOL_F32
    err = float(np.abs(out - expected["attention"]).max())
    assert err <= tol, err
