"""Helpers shared by the GPU parity tests (not a test module).

Inputs come from synth.gen (numpy, seeded); they are copied to the GPU
unchanged (bf16 as raw bit patterns), so both sides see identical values.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from synth import gen

REL_TOL = 1e-5          # conf / value / near-tie tolerance (relative)
# Near-tie events seen by the draft-step replays, per workload: reported in
# the session summary (tests/conftest.py) so a -q run still shows them.
NEAR_TIES: dict = {}
ATTN_TOL_BF16 = 1e-2    # max-abs vs fp64 oracle on the same bf16 inputs
ATTN_TOL_F32 = 1e-4     # fp32 inputs: fp32 dot products and exp


def to_dev(a: np.ndarray, dtype_name: str | None = None) -> torch.Tensor:
    """numpy -> cuda tensor; uint16 arrays are bf16 bit patterns."""
    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
        return t.view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bf16_dev_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def make_inputs(w, seed=None, planted_target=None, boost=None):
    seed = w.seed if seed is None else seed
    return dict(
        draft=gen.draft_logits(w, seed),
        target=gen.target_logits(w, seed, planted=planted_target, boost=boost),
        root_tokens=gen.root_tokens(w, seed),
        prefix_len=gen.prefix_lens(w, seed),
        attn=gen.attention_inputs(w, seed),
    )


def dev_inputs(inp):
    return dict(
        draft=to_dev(inp["draft"]),
        target=to_dev(inp["target"]),
        root_tokens=to_dev(inp["root_tokens"]),
        prefix_len=to_dev(inp["prefix_len"]),
        attn={k: to_dev(v) for k, v in inp["attn"].items()},
    )


def state_from_export(w, ex, roots) -> oracle.TreeState:
    st = oracle.TreeState(w)
    for name in ("token", "parent", "depth", "conf", "value"):
        setattr(st, name, ex[name].cpu().numpy().copy())
    st.count = ex["pool_count"].cpu().numpy().copy()
    st.frontier = ex["frontier"].cpu().numpy().copy()
    st.frontier_count = ex["frontier_count"].cpu().numpy().copy()
    st.root = np.asarray(roots, np.int32).copy()
    return st


def rel_close(a, b, tol=REL_TOL):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.abs(a - b) <= tol * np.maximum(np.abs(a), np.abs(b)) + 1e-30


def check_draft_step(w, before: oracle.TreeState, gpu_after, ora_after,
                     gpu_next, ora_next):
    """Compare one draft step (both sides started from `before`).

    Children (token, parent, depth) must be bit-exact; conf and value
    within REL_TOL; the frontier must be the oracle's, except where oracle
    values of swapped candidates lie within REL_TOL (near-tie event), in
    which case the two selections must agree value by value.  Returns the
    sequences with a near-tie event at this step."""
    events = []
    for b in range(w.batch):
        p0 = int(before.count[b])
        p1 = int(ora_after.count[b])
        assert int(gpu_after.count[b]) == p1, f"b={b} pool count"
        sl = slice(p0, p1)
        for name in ("token", "parent", "depth"):
            np.testing.assert_array_equal(getattr(gpu_after, name)[b, sl],
                                          getattr(ora_after, name)[b, sl],
                                          err_msg=f"b={b} {name}")
        assert rel_close(gpu_after.conf[b, sl], ora_after.conf[b, sl]).all(), \
            f"b={b} conf"
        assert rel_close(gpu_after.value[b, sl], ora_after.value[b, sl]).all(), \
            f"b={b} value"
        fg = list(gpu_after.frontier[b, :gpu_after.frontier_count[b]])
        fo = list(ora_after.frontier[b, :ora_after.frontier_count[b]])
        if fg != fo:
            events.append(b)
            vo = ora_after.value[b]
            n = max(len(fg), len(fo))
            vg = sorted((float(vo[i]) for i in fg), reverse=True)
            vr = sorted((float(vo[i]) for i in fo), reverse=True)
            for i in range(n):
                a = vg[i] if i < len(vg) else w.threshold
                c = vr[i] if i < len(vr) else w.threshold
                assert rel_close(a, c), f"b={b} frontier differs beyond a near tie"
        # next_tokens are the frontier's tokens in frontier order
        nt = gpu_next[0][b]
        assert int(gpu_next[1][b]) == len(fg)
        assert list(nt[:len(fg)]) == [int(gpu_after.token[b, i]) for i in fg]
        assert (nt[len(fg):] == -1).all()
        if fg == fo:
            np.testing.assert_array_equal(nt, ora_next[0][b])
    return events


def random_path_targets(w, rr, rng, hit=0.9):
    """Target peaks that follow a random kept path (so the walk is long):
    each slot's peak is one kept child with probability `hit`."""
    planted = np.full((w.batch, w.T), -1, np.int64)
    for b in range(w.batch):
        n = int(rr["n_kept"][b])
        cur = 0
        while True:
            kids = [s for s in range(1, n + 1) if rr["parent_slot"][b, s] == cur]
            if not kids or rng.random() > hit:
                break
            c = int(rng.choice(kids))
            planted[b, cur] = rr["tokens"][b, c]
            cur = c
    return planted
