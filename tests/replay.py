"""Saved cycles: a workload and its exact inputs in one .npz file, so a
failing case can be kept and run again (tests/golden/replays/ holds the
committed ones together with the oracle's outputs for them).  Helpers
only, not a test module."""
from __future__ import annotations

import dataclasses
import json

import numpy as np

from synth import Workload

INPUT_KEYS = ("draft", "target", "root_tokens", "prefix_len")


def save(path, w: Workload, inputs: dict, expected: dict | None = None, note: str = ""):
    """inputs as gpu_util.make_inputs builds them (attn: a dict of arrays);
    expected: oracle outputs to store beside them (name -> array)."""
    arrays = {k: np.asarray(inputs[k]) for k in INPUT_KEYS}
    for k, v in inputs["attn"].items():
        arrays["attn_" + k] = np.asarray(v)
    for k, v in (expected or {}).items():
        arrays["expected_" + k] = np.asarray(v)
    meta = dict(workload=dataclasses.asdict(w), note=note)
    np.savez_compressed(path, meta=np.array(json.dumps(meta)), **arrays)


def load(path):
    """(workload, inputs, expected) of a saved cycle."""
    z = np.load(path, allow_pickle=False)
    meta = json.loads(str(z["meta"]))
    wd = meta["workload"]
    for k in ("sharpness", "prefix_range"):
        wd[k] = tuple(wd[k])
    w = Workload(**wd)
    inputs = {k: z[k] for k in INPUT_KEYS}
    inputs["attn"] = {k[5:]: z[k] for k in z.files if k.startswith("attn_")}
    expected = {k[9:]: z[k] for k in z.files if k.startswith("expected_")}
    return w, inputs, expected


def oracle_outputs(w, inputs):
    """The outputs stored beside a saved cycle: the oracle's cycle on it."""
    import oracle
    ref = oracle.cycle(w, inputs)
    rr, mk, acc = ref["rerank"], ref["mask"], ref["accept"]
    return dict(tokens=rr["tokens"], parent_slot=rr["parent_slot"],
                conf=rr["conf"], value=rr["value"], n_kept=rr["n_kept"],
                mask=mk["mask"], depth=mk["depth"], pos_ids=mk["pos_ids"],
                attention=ref["attention"], accept_len=acc["accept_len"],
                path_slots=acc["path_slots"], out_tokens=acc["out_tokens"])
