"""Writes the committed saved cycles (tests/golden/replays/*.npz): seeded
synthetic inputs of two small workloads and, beside them, the outputs of
the CPU oracle on them.  Calls only synth (random draws) and oracle/.

    python tests/golden/make_replays.py
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path[:0] = [os.path.dirname(os.path.dirname(HERE)), os.path.dirname(HERE)]

import replay  # noqa: E402
from gpu_util import make_inputs  # noqa: E402
from synth import WORKLOADS, gen  # noqa: E402

CASES = {
    # fp32, threshold rule on
    "tiny_seed0": (WORKLOADS["tiny"], False),
    # bf16 with rows of exact ties (lowest id wins), GQA 2/1, ragged prefix
    "small_bf16_tied": (WORKLOADS["tiny"].with_(
        batch=2, vocab=1500, topk=3, depth=3, budget_n=10, threshold=0.0,
        logits_dtype="bf16", sharpness=(0.8, 2.5), n_q_heads=2, n_kv_heads=1,
        head_dim=64, prefix_cap=32, prefix_range=(1, 32), qkv_dtype="bf16",
        seed=41), True),
}


def main():
    out = os.path.join(HERE, "replays")
    os.makedirs(out, exist_ok=True)
    for name, (w, tied) in CASES.items():
        inp = make_inputs(w)
        if tied:
            inp["draft"] = gen.tied_draft_logits(w)
            inp["target"] = gen.tied_target_logits(w)
        exp = replay.oracle_outputs(w, inp)
        path = os.path.join(out, name + ".npz")
        replay.save(path, w, inp, exp, note="written by tests/golden/make_replays.py")
        print(path, os.path.getsize(path))


if __name__ == "__main__":
    main()
