"""Throughput of one EAGLE-2 draft-tree build + verify cycle on one MI355X.

A step is one whole cycle over one batch: D - 1 x et_draft_step, then
et_draft_step_last (the last draft step, whose merge also reranks the pool
and flattens the tree), et_tree_attention (one attention layer) and
et_accept, on
synthetic inputs already resident in HBM.  The default workload is the
Llama-3.1-8B shape at batch 1 (vocab 128256, top-k 10, depth 8, N 60,
GQA 32/8 x 128, prefix 4096, bf16).  Input sets rotate so the working set
exceeds the 256 MB MALL and every cycle reads HBM.

Prints one JSON line: cycles/s, the roofline of the dominant call
(algorithmic bytes / its average duration, HIP events on the launch
stream; a call is one or two back-to-back launches), the whole cycle's
roofline fraction (sum over calls of max(bytes / 8 TB/s, flops / 2.5
PFLOP/s) over the measured cycle time), per-call GB/s against the peak and
against a measured streaming copy, and the CPU oracle timed on this host
(one thread and all threads) as a reported baseline, with the near-tie
events of input set 0.  Beside the metric, timed after it: the spread of
the cycle time (p10 / median / p90 over groups of 10 cycles), KV commit,
sampled acceptance, the fixed-shape tree build against the dynamic one
with each tree's expected accepted tokens, the draft step from hidden
states (LM head fused) against torch's GEMM, and the batch-64 and 70B
workloads' cycles/s and rooflines.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, published
MALL_BYTES = 256 << 20


# Each measured call, the kernels one call launches (one dispatch each) and
# the files whose change invalidates its counters.
CALLS = {
    "draft_step": (["draft_scan_kernel", "draft_merge_kernel"],
                   ["draft.hip", "device.h", "internal.h"]),
    "draft_step_last": (["draft_scan_kernel", "draft_merge_last_kernel"],
                        ["draft.hip", "rerank.h", "device.h", "internal.h"]),
    "accept": (["accept_scan_kernel", "accept_walk_kernel"],
               ["accept.hip", "device.h", "internal.h"]),
    "tree_attention": (["tree_attn_bf16_kernel", "tree_attn_merge_kernel",
                        "tree_attn_order_kernel"],
                       ["attention.hip", "device.h", "internal.h"]),
}


def source_digest(call):
    import hashlib
    h = hashlib.sha256()
    for f in CALLS[call][1]:
        with open(os.path.join(ROOT, "dynamic_draft_tree_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_path(call, workload):
    return os.path.join(ROOT, "profiles", f"{call}_{workload}_traffic.json")


def measured_traffic(call, workload):
    """HBM bytes per call from the committed counter summary, or None when
    there is none or the call's sources changed since it was taken."""
    p = traffic_path(call, workload)
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        t = json.load(fh)
    if t.get("source_digest") != source_digest(call):
        return None
    return t["traffic_bytes_per_call"]


def pmc_rows(d):
    """(kernel name, counter, value) rows of a rocprofv3 --pmc csv run."""
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                rows.append((r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])))
    return rows


def summarize_pmc(args):
    """Write profiles/<call>_<workload>_traffic.json from four --pmc runs:
    FETCH_SIZE and WRITE_SIZE of the bench and of the copy calibration.
    A call's traffic is the sum over its kernels of the mean per dispatch."""
    fetch, write, cfetch, cwrite = args.summarize_pmc
    copy_bytes = args.copy_mb * (1 << 20)
    call = args.summarize_call

    def per_dispatch(d, name_part, counter):
        """Mean over the dispatches (a call's launches differ in size, as
        its algorithmic bytes do)."""
        v = [x for k, c, x in pmc_rows(d) if name_part in k and c == counter]
        if not v:
            raise SystemExit(f"no {counter} rows for {name_part} under {d}")
        return float(np.mean(v)), len(v)

    # the copy kernel reads and writes copy_bytes per dispatch
    cf, _ = per_dispatch(cfetch, "neg_kernel", "FETCH_SIZE")
    cw, _ = per_dispatch(cwrite, "neg_kernel", "WRITE_SIZE")
    f_fetch = copy_bytes / cf
    f_write = copy_bytes / cw
    kernels = {}
    for kn in CALLS[call][0]:
        kf, nf = per_dispatch(fetch, kn, "FETCH_SIZE")
        kw, nw = per_dispatch(write, kn, "WRITE_SIZE")
        kernels[kn] = {"fetch_size_kib_mean": kf, "write_size_kib_mean": kw,
                       "dispatches": [nf, nw],
                       "fetch_bytes": kf * f_fetch, "write_bytes": kw * f_write}
    out = {
        "call": call, "workload": args.workload, "kernels": kernels,
        "copy_calibration": {"bytes": copy_bytes, "fetch_kib": cf, "write_kib": cw,
                             "fetch_bytes_per_unit": f_fetch,
                             "write_bytes_per_unit": f_write},
        "traffic_bytes_per_call": round(sum(k["fetch_bytes"] + k["write_bytes"]
                                            for k in kernels.values())),
        "source_digest": source_digest(call),
    }
    with open(traffic_path(call, args.workload), "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


def trace_durations_us(path):
    """Mean duration (us) per kernel name in a rocprofv3 kernel trace: its
    rocpd SQLite database (table kernels) or its kernel_trace.csv (-f csv)."""
    out = {}
    if path.endswith(".csv"):
        import csv
        with open(path) as fh:
            for r in csv.DictReader(fh):
                out.setdefault(r["Kernel_Name"], []).append(
                    float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
    else:
        import sqlite3
        con = sqlite3.connect(path)
        for name, dur in con.execute("select name, duration from kernels"):
            out.setdefault(name, []).append(float(dur))
        con.close()
    return {k: float(np.mean(v)) / 1e3 for k, v in out.items()}


# Engine clock for converting busy cycles to time: 2.4 GHz, the clock an
# s_memtime / s_memrealtime comparison reads inside a kernel on this part.
SCLK_GHZ = 2.4
N_SIMD = 1024  # 256 compute units x 4


def summarize_counters(args):
    """Write profiles/<call>_<workload>_counters.json: per kernel of the
    call, the mean per dispatch of every counter in the given --pmc runs
    of the bench, HBM bytes (FETCH_SIZE, WRITE_SIZE scaled by the copy
    calibration runs), instructions per wave, the matrix-core busy fraction
    and achieved bf16 rate over the kernel's mean duration in a
    kernel-trace run of the same command."""
    call = args.summarize_call
    cfetch, cwrite = args.copy_dirs
    copy_bytes = args.copy_mb * (1 << 20)

    def means(dirs, name_part):
        acc = {}
        for d in dirs:
            for k, c, x in pmc_rows(d):
                if name_part in k:
                    acc.setdefault(c, []).append(x)
        return {c: float(np.mean(v)) for c, v in acc.items()}, \
            max((len(v) for v in acc.values()), default=0)

    cf = means([cfetch], "neg_kernel")[0]["FETCH_SIZE"]
    cw = means([cwrite], "neg_kernel")[0]["WRITE_SIZE"]
    f_fetch, f_write = copy_bytes / cf, copy_bytes / cw
    durs = trace_durations_us(args.trace_db)
    kernels = {}
    for kn in CALLS[call][0]:
        c, n = means(args.summarize_counters, kn)
        if not c:  # not launched at this workload (e.g. no key split)
            kernels[kn] = {"dispatches": 0}
            continue
        dur = [v for k, v in durs.items() if kn in k]
        us = float(np.mean(dur)) if dur else None
        waves = c.get("SQ_WAVES", 0.0)
        e = {"dispatches": n, "avg_us": round(us, 3) if us else None,
             "counters": {k: round(v, 1) for k, v in sorted(c.items())}}
        if "FETCH_SIZE" in c and "WRITE_SIZE" in c:
            e["fetch_bytes"] = round(c["FETCH_SIZE"] * f_fetch)
            e["write_bytes"] = round(c["WRITE_SIZE"] * f_write)
            if us:
                gbs = (e["fetch_bytes"] + e["write_bytes"]) / (us * 1e3)
                e["hbm_gbs"] = round(gbs, 1)
                e["frac_hbm_peak"] = round(gbs / HBM_PEAK_GBS, 4)
        if "TCC_HIT_sum" in c and "TCC_MISS_sum" in c:
            tot = c["TCC_HIT_sum"] + c["TCC_MISS_sum"]
            e["l2_hit_rate"] = round(c["TCC_HIT_sum"] / tot, 4) if tot else None
        if waves:
            e["per_wave"] = {k[len("SQ_INSTS_"):].lower(): round(v / waves, 1)
                             for k, v in c.items()
                             if k.startswith("SQ_INSTS_") and "MOPS" not in k}
        if us and "SQ_VALU_MFMA_BUSY_CYCLES" in c:
            busy_us = c["SQ_VALU_MFMA_BUSY_CYCLES"] / N_SIMD / (SCLK_GHZ * 1e3)
            e["mfma_busy_us_per_simd"] = round(busy_us, 3)
            e["mfma_busy_frac"] = round(busy_us / us, 4)
        if us and c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16"):
            tf = c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / (us * 1e-6) / 1e12
            e["bf16_tflops"] = round(tf, 1)
            e["frac_mfma_peak"] = round(tf / MFMA_BF16_PEAK_TFLOPS, 4)
        kernels[kn] = e
    out = {"call": call, "workload": args.workload, "kernels": kernels,
           "copy_calibration": {"bytes": copy_bytes, "fetch_kib": cf, "write_kib": cw,
                                "fetch_bytes_per_unit": f_fetch,
                                "write_bytes_per_unit": f_write},
           "sclk_ghz": SCLK_GHZ, "source_digest": source_digest(call)}
    path = os.path.join(ROOT, "profiles", f"{call}_{args.workload}_counters.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


def copy_calibration(args):
    """A plain device copy of --copy-mb MiB, the reference for scaling the
    FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    n = args.copy_mb * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)  # one elementwise kernel: reads n, writes n
    torch.cuda.synchronize()
    print(json.dumps({"copy_mb": args.copy_mb, "dispatches": 5}), flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama8b")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch every call eagerly instead of replaying "
                         "one HIP graph per input set")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget for the CPU oracle baseline (0 = skip)")
    ap.add_argument("--no-extras", action="store_true",
                    help="leave out the calls measured beside the cycle (KV "
                         "commit, sampled acceptance, the two tree builds), "
                         "so a counter run sees only the cycle's dispatches")
    ap.add_argument("--sets", type=int, default=0,
                    help="input sets to rotate (0 = enough to pass the MALL)")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="only run the copy used to calibrate HBM counters")
    ap.add_argument("--summarize-pmc", nargs=4, metavar="DIR",
                    help="write the traffic summary from the FETCH_SIZE and "
                         "WRITE_SIZE runs of the bench and of the copy")
    ap.add_argument("--summarize-call", default="draft_step", choices=sorted(CALLS))
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                    help="write the counter summary of --summarize-call from "
                         "these --pmc runs of the bench (with --copy-dirs and "
                         "--trace-db)")
    ap.add_argument("--copy-dirs", nargs=2, metavar="DIR",
                    help="FETCH_SIZE and WRITE_SIZE runs of the copy")
    ap.add_argument("--trace-db", help="rocprofv3 kernel-trace database of the "
                                       "same bench command")
    return ap.parse_args()


def algorithmic(w, n_kept, frontier_rows, prefix_len):
    """Bytes (and flops) each call must move, per launch, from the shapes:
    logits rows read once; K/V of every prefix and kept tree position read
    once; q and out of every kept slot once; q.k and p.v over the prefix
    for every kept slot and head (the few tree keys are left out)."""
    esz = 2 if w.logits_dtype == "bf16" else 4
    qsz = 2 if w.qkv_dtype == "bf16" else 4
    rows = n_kept.astype(np.float64) + 1.0   # kept slots incl. the root
    P = prefix_len.astype(np.float64)
    draft = [r * w.vocab * esz for r in frontier_rows]
    accept = float(np.sum(rows)) * w.vocab * esz
    kv = float(np.sum(w.n_kv_heads * (P + rows) * w.head_dim * 2 * qsz))
    qo = float(np.sum(2 * rows * w.n_q_heads * w.head_dim * qsz))
    flops = float(np.sum(4.0 * w.n_q_heads * rows * P * w.head_dim))
    return dict(draft=draft, accept=accept, attention=kv + qo,
                attention_flops=flops)


def cycle_roof_us(w, alg):
    """Roofline time of one cycle: each call at max(bytes / HBM peak,
    flops / bf16 MFMA peak) from its algorithmic bytes and flops (the
    rerank and mask call moves negligible bytes)."""
    bw = HBM_PEAK_GBS * 1e3      # bytes per us
    mf = MFMA_BF16_PEAK_TFLOPS * 1e6  # flops per us
    t = sum(b / bw for b in alg["draft"])
    t += max(alg["attention"] / bw, alg["attention_flops"] / mf)
    t += alg["accept"] / bw
    return t


def draft_step_bytes(alg):
    """Mean logits bytes of the ordinary draft steps (all but the last,
    which the cycle takes as et_draft_step_last)."""
    d = alg["draft"]
    return float(np.mean(d[:-1])) if len(d) > 1 else float(d[0])


def call_rooflines(w, alg, avg_us, copy_gbs):
    """Per call: algorithmic GB/s (TFLOP/s for attention too) against the
    8 TB/s peak and against the measured streaming copy."""
    out = {}
    for name, byts, flops in (("draft", draft_step_bytes(alg), 0.0),
                              ("draft_last", alg["draft"][-1], 0.0),
                              ("attention", alg["attention"], alg["attention_flops"]),
                              ("accept", alg["accept"], 0.0)):
        if name not in avg_us:
            continue
        us = avg_us[name]
        gbs = byts / (us * 1e-6) / 1e9
        e = {"us": round(us, 3), "bytes": byts, "gbs": round(gbs, 1),
             "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
             "frac_copy": round(gbs / copy_gbs, 4) if copy_gbs else None}
        if flops and w.qkv_dtype == "bf16":
            tf = flops / (us * 1e-6) / 1e12
            e.update({"tflops": round(tf, 1),
                      "frac_mfma_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)})
        out[name] = e
    return out


def dominant_roofline(w, alg, avg_us, per_cycle_us):
    """The roofline entry of the call with the largest time per cycle:
    algorithmic bytes (or flops, above the ridge) per call over its
    average duration."""
    names = list(per_cycle_us)
    dominant = max(names, key=lambda n: per_cycle_us[n])
    call = {"draft": "draft_step", "draft_last": "draft_step_last", "accept": "accept",
            "attention": "tree_attention"}.get(dominant)
    bytes_per_call = {"draft": draft_step_bytes(alg), "draft_last": alg["draft"][-1],
                      "accept": alg["accept"],
                      "attention": alg["attention"]}.get(dominant, 0.0)
    achieved = bytes_per_call / (avg_us[dominant] * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(call, w.name) if call else None,
                "call": call or dominant,
                "kernels": CALLS[call][0] if call else [],
                "avg_us": round(avg_us[dominant], 3),
                "bytes_per_call": bytes_per_call}
    if dominant == "attention" and w.qkv_dtype == "bf16":
        # above the ridge (flops per byte > peak flops / peak bytes) the
        # matrix cores, not HBM, bound the call
        flops = alg["attention_flops"]
        if flops / bytes_per_call > MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
            tf = flops / (avg_us[dominant] * 1e-6) / 1e12
            roofline.update({"bound": "mfma", "achieved": round(tf, 1),
                             "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                             "flops_per_call": flops})
    return roofline


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


class Bench:
    """One workload on one GPU: resident input sets, one HIP graph per set,
    the timed replays, and the per-call timing pass."""

    def __init__(self, w, n_sets, torch, d, gen):
        self.w, self.torch, self.d, self.gen = w, torch, d, gen
        t0 = time.time()
        self.sets = []
        seed = w.seed
        while True:
            s = dict(draft=gen.draft_logits(w, seed), target=gen.target_logits(w, seed),
                     roots=gen.root_tokens(w, seed), prefix=gen.prefix_lens(w, seed),
                     attn=gen.attention_inputs(w, seed))
            ds = dict(draft=self.dev(s["draft"]), target=self.dev(s["target"]),
                      roots=self.dev(s["roots"]), prefix=self.dev(s["prefix"]),
                      attn={k: self.dev(v) for k, v in s["attn"].items()})
            if not self.sets:
                self.host0 = s
                self.set_bytes = sum(t.numel() * t.element_size() for t in
                                     [ds["draft"], ds["target"], *ds["attn"].values()])
            else:
                del s
            self.sets.append(ds)
            seed += 1000
            want = n_sets or max(2, -(-2 * MALL_BYTES // self.set_bytes))
            if len(self.sets) >= min(want, 64):
                break
        self.gen_s = time.time() - t0
        self.plan = d.Plan(w)
        self.stream = torch.cuda.current_stream()
        self.graphs = None

    def dev(self, a):
        if a.dtype == np.uint16:
            return self.torch.from_numpy(a.view(np.int16)).view(self.torch.bfloat16).cuda()
        return self.torch.from_numpy(np.ascontiguousarray(a)).cuda()

    def cycle(self, ds, stream=None):
        self.plan.cycle(ds["roots"], ds["draft"], ds["prefix"], ds["attn"],
                        ds["target"], stream or self.stream)

    def capture(self):
        torch = self.torch
        self.cycle(self.sets[0])  # warm the code objects before capture
        torch.cuda.synchronize()
        self.graphs = []
        for ds in self.sets:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self.cycle(ds, torch.cuda.current_stream())
            self.graphs.append(g)
        torch.cuda.synchronize()

    def run(self, i):
        if self.graphs is not None:
            self.graphs[i % len(self.sets)].replay()
        else:
            self.cycle(self.sets[i % len(self.sets)])

    def timed(self, steps, warmup):
        torch = self.torch
        for i in range(warmup):
            self.run(i)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(steps):
            self.run(i)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps

    def spread(self, n_groups=20, per_group=10):
        """Per-cycle time of groups of cycles (events between whole cycles,
        all groups enqueued at once)."""
        torch = self.torch
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_groups + 1)]
        evs[0].record()
        for g_ in range(n_groups):
            for i in range(per_group):
                self.run(g_ * per_group + i)
            evs[g_ + 1].record()
        torch.cuda.synchronize()
        grp = np.array([evs[g_].elapsed_time(evs[g_ + 1]) * 1e3 / per_group
                        for g_ in range(n_groups)])
        return {"groups": n_groups, "cycles_per_group": per_group,
                "p10_us": round(float(np.percentile(grp, 10)), 2),
                "median_us": round(float(np.median(grp)), 2),
                "p90_us": round(float(np.percentile(grp, 90)), 2)}

    def per_call(self, K, spin_per_ms, hold_ms=20.0):
        """Average duration of each call, in an eager pass bracketed by HIP
        events on the launch stream (events recorded inside a graph cannot
        be timed).  A spin kernel at the head of every batch holds the GPU
        until the host has enqueued the whole batch, so the calls run back
        to back as in the graph and the events time the GPU work, not the
        host's launch rate.  The D draft steps of a cycle sit between one
        pair of events."""
        torch, w, plan, stream = self.torch, self.w, self.plan, self.stream
        names = (["draft"] if w.depth > 1 else []) + ["draft_last", "attention", "accept"]
        acc = {n: 0.0 for n in names}
        cnt = {n: 0 for n in names}

        def enqueue_cycle(ds, row):
            if w.depth > 1:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for step in range(1, w.depth):
                    plan.draft_step(step, ds["roots"], ds["draft"][:, step - 1], stream)
                e1.record(stream)
                row.append(("draft", e0, e1))
            for n, fn in (("draft_last", lambda: plan.draft_step_last(
                              ds["roots"], ds["draft"][:, w.depth - 1], ds["prefix"], stream)),
                          ("attention", lambda: plan.tree_attention(
                              ds["attn"]["q"], ds["attn"]["k_cache"],
                              ds["attn"]["v_cache"], ds["attn"]["k_tree"],
                              ds["attn"]["v_tree"], ds["prefix"], stream=stream)),
                          ("accept", lambda: plan.accept(ds["target"], stream))):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                row.append((n, e0, e1))

        per_batch = 10
        done = starved = 0
        while done < K:
            nb = min(per_batch, K - done)
            rows = []
            torch.cuda._sleep(int(hold_ms * spin_per_ms))
            gate = torch.cuda.Event()
            gate.record(stream)
            t_host = time.time()
            for i in range(nb):
                row = []
                enqueue_cycle(self.sets[(done + i) % len(self.sets)], row)
                rows.append(row)
            host_ms = (time.time() - t_host) * 1e3
            if gate.query():  # the GPU caught up with the host: hold longer
                torch.cuda.synchronize()
                starved += 1
                if starved > 6:
                    raise RuntimeError("bench: could not hold the GPU while enqueueing")
                hold_ms = max(2 * hold_ms, 3 * host_ms)
                continue
            torch.cuda.synchronize()
            for row in rows:
                for n, e0, e1 in row:
                    acc[n] += e0.elapsed_time(e1) * 1e3  # us
                    cnt[n] += w.depth - 1 if n == "draft" else 1
            done += nb
        avg_us = {n: acc[n] / cnt[n] for n in names}
        per_cycle_us = {n: acc[n] / K for n in names}
        return avg_us, per_cycle_us, hold_ms

    def algorithmic(self):
        w = self.w
        n_kept = self.plan.n_kept.cpu().numpy()
        # frontier rows per step: 1 at step 1; with the threshold off every
        # later step reads k rows per sequence
        fr = [w.batch] + [w.batch * w.topk] * (w.depth - 1)
        return algorithmic(w, n_kept, fr, self.host0["prefix"])

    def release(self):
        self.graphs = None
        self.sets = None
        self.plan = None
        self.torch.cuda.synchronize()
        self.torch.cuda.empty_cache()


def spin_rate(torch):
    """Cycles per ms of torch's spin kernel (its argument counts clock
    cycles), to size the hold of the per-call pass."""
    torch.cuda.synchronize()
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    torch.cuda._sleep(2_000_000)
    s1.record()
    torch.cuda.synchronize()
    return 2_000_000 / max(s0.elapsed_time(s1), 1e-3)


def near_ties(b, oracle):
    """The GPU tree of input set 0 against the oracle: each draft step is
    compared with the oracle run from the GPU's own state; a frontier that
    differs only where two oracle values lie within 1e-5 relative is a
    near-tie event, any other difference a mismatch.  Also whether the
    final GPU tree equals an independent oracle run (with no event, it
    must).  Outside the timed region."""
    torch, w, plan, ds = b.torch, b.w, b.plan, b.sets[0]
    h = b.host0
    roots = np.asarray(h["roots"], np.int32)
    before = oracle.TreeState(w)
    indep = oracle.TreeState(w)
    events = mismatches = 0
    for step in range(1, w.depth + 1):
        plan.draft_step(step, ds["roots"], ds["draft"][:, step - 1])
        torch.cuda.synchronize()
        ex = plan.export_pool()
        after = oracle.TreeState(w)
        for f in ("token", "parent", "depth", "conf", "value"):
            setattr(after, f, ex[f].cpu().numpy().copy())
        after.count = ex["pool_count"].cpu().numpy().copy()
        after.frontier = ex["frontier"].cpu().numpy().copy()
        after.frontier_count = ex["frontier_count"].cpu().numpy().copy()
        after.root = roots.copy()
        ref = before.copy()
        oracle.draft_step(w, ref, step, roots, h["draft"][:, step - 1])
        oracle.draft_step(w, indep, step, roots, h["draft"][:, step - 1])
        for q in range(w.batch):
            fg = list(after.frontier[q, :after.frontier_count[q]])
            fo = list(ref.frontier[q, :ref.frontier_count[q]])
            if fg == fo:
                continue
            vo = ref.value[q]
            vg = sorted((float(vo[i]) for i in fg), reverse=True)
            vr = sorted((float(vo[i]) for i in fo), reverse=True)
            near = len(vg) == len(vr) and all(
                abs(x - y) <= 1e-5 * max(abs(x), abs(y)) for x, y in zip(vg, vr))
            events += near
            mismatches += not near
        before = after
    plan.rerank()
    torch.cuda.synchronize()
    ind = oracle.rerank(w, indep)
    same = bool(np.array_equal(plan.tokens.cpu().numpy(), ind["tokens"]) and
                np.array_equal(plan.parent_slot.cpu().numpy(), ind["parent_slot"]))
    return {"events": int(events), "mismatches": int(mismatches),
            "sequence_steps": w.batch * w.depth, "tree_equals_oracle": same}


def cpu_baseline(w, host0, seconds, oracle):
    """The oracle (as is: OpenMP over (sequence, head) in attention only)
    on this host's cores: single-threaded, then on all its threads, each
    for up to half the budget (at least one cycle)."""
    inputs = dict(root_tokens=host0["roots"], draft=host0["draft"],
                  prefix_len=host0["prefix"], attn=host0["attn"],
                  target=host0["target"])
    n_all = oracle.num_threads()
    res = {}
    for label, nt in (("single", 1), ("all", n_all)):
        oracle.set_num_threads(nt)
        t1 = time.time()
        n = 0
        while True:
            oracle.cycle(w, inputs)
            n += 1
            if time.time() - t1 >= seconds / 2 or n >= 50:
                break
        res[label] = (n, time.time() - t1, nt)
    oracle.set_num_threads(n_all)
    n, el, nt = res["all"]
    n1, el1, _ = res["single"]
    return {"value": round(n / el, 4), "unit": "cycles/s", "cores": nt,
            "kind": "oracle",
            "sample": f"{n} full oracle cycle(s) of the {w.name} workload "
                      f"(input set 0) in {el:.1f} s on {nt} threads; "
                      f"{n1} in {el1:.1f} s on 1 thread",
            "single_thread": round(n1 / el1, 4), "threads_all": nt,
            "cpu_model": cpu_model(), "nproc": os.cpu_count()}


def extra_workload(name, args, torch, d, gen, WORKLOADS, copy_gbs, spin_per_ms):
    """cycles/s and rooflines of another workload, measured in the same
    run: one input set (each is larger than twice the MALL), graph
    replay, then the per-call pass."""
    w = WORKLOADS[name]
    b = Bench(w, 1, torch, d, gen)
    b.capture()
    # (20 warm-up cycles: the extras follow the CPU leg, which leaves the
    # GPU idle for seconds)
    ms = b.timed(min(args.steps, 100), 20)
    avg_us, per_cycle_us, _ = b.per_call(10, spin_per_ms)
    alg = b.algorithmic()
    out = {"cycles_per_s": round(1e3 / ms, 2), "ms_per_cycle": round(ms, 5),
           "per_call_us": {n: round(v, 3) for n, v in avg_us.items()},
           "cycle_roofline_frac": round(cycle_roof_us(w, alg) / (ms * 1e3), 4),
           "calls": call_rooflines(w, alg, avg_us, copy_gbs),
           "roofline": dominant_roofline(w, alg, avg_us, per_cycle_us),
           "set_mb": round(b.set_bytes / 1e6, 1)}
    b.release()
    del b
    return out


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(args)
        return
    if args.summarize_counters:
        summarize_counters(args)
        return
    if args.copy_mb:
        copy_calibration(args)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is "
              "not supported (a batch would shard by sequence across GPUs "
              "with no exchange between them)", file=sys.stderr)
        sys.exit(2)

    import torch

    import dynamic_draft_tree_amd as d
    from synth import WORKLOADS, gen

    d.lib()  # fail loudly if the HIP library is missing
    w = WORKLOADS[args.workload]
    torch.cuda.set_device(0)

    b = Bench(w, args.sets, torch, d, gen)
    if not args.no_graph:
        b.capture()
    ms = b.timed(args.steps, args.warmup)
    spread = b.spread()

    # ---- streaming-copy bandwidth: the practical HBM ceiling beside the
    # 8 TB/s peak (an elementwise kernel over 512 MiB in, 512 MiB out) ------
    cn = 512 * (1 << 20) // 4
    csrc = torch.ones(cn, dtype=torch.float32, device="cuda")
    cdst = torch.empty_like(csrc)
    torch.neg(csrc, out=cdst)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(10):
        torch.neg(csrc, out=cdst)
    c1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * cn * 4 * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del csrc, cdst

    spin_per_ms = spin_rate(torch)
    K = max(10, min(args.steps, 200))
    avg_us, per_cycle_us, hold_ms = b.per_call(K, spin_per_ms)
    plan, stream, sets = b.plan, b.stream, b.sets

    # ---- calls beside the cycle (not part of the metric) ----
    # KV commit: the last cycle's accepted paths are appended to copies of
    # input set 0's caches, with the prefix lengths lowered to leave room
    # (the workloads fill their caches), restored before each call.
    # Sampled acceptance (temperature 1) of the last cycle's tree on set
    # 0's targets, in place of the greedy walk.  Each call is timed on its
    # own, 20 times, the GPU held as above; the median is reported.
    commit_us = sample_us = None
    build_us, readout, shape_p, lm_step = {}, {}, [], None
    if not args.no_extras:
        def time_next(call, before=None):
            torch.cuda.synchronize()
            torch.cuda._sleep(int(hold_ms * spin_per_ms))
            ev = []
            for _ in range(20):
                if before is not None:
                    before()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                call()
                e1.record(stream)
                ev.append((e0, e1))
            torch.cuda.synchronize()
            return float(np.median([a.elapsed_time(b_) * 1e3 for a, b_ in ev]))

        ds0 = sets[0]
        kc = ds0["attn"]["k_cache"].clone()
        vc = ds0["attn"]["v_cache"].clone()
        plen0 = torch.clamp(ds0["prefix"], max=w.prefix_cap - w.depth - 1)
        plen = plen0.clone()
        commit_us = time_next(
            lambda: plan.kv_commit(kc, vc, ds0["attn"]["k_tree"], ds0["attn"]["v_tree"],
                                   plen, stream),
            lambda: plen.copy_(plen0))
        del kc, vc
        uni = torch.rand((w.batch, w.T), device="cuda",
                         generator=torch.Generator(device="cuda").manual_seed(w.seed))
        sample_us = time_next(lambda: plan.accept_sample(ds0["target"], 1.0, uni, stream))
        # Fixed-shape baseline against the dynamic tree on set 0's draft logits
        # (a plan of its own): each build (D steps, then the slot gather or the
        # rerank) timed as one call, and each tree's readout, the mean over
        # sequences of the kept values' sum (expected accepted tokens).
        splan = d.Plan(w)
        shape_p, shape_r = gen.static_shape(w)
        splan.set_static_shape(shape_p[1:], shape_r[1:])

        def build(static):
            for step in range(1, w.depth + 1):
                if static:
                    splan.draft_step_static(step, ds0["roots"], ds0["draft"][:, step - 1], stream)
                else:
                    splan.draft_step(step, ds0["roots"], ds0["draft"][:, step - 1], stream)
            if static:
                splan.static_tree(stream)
            else:
                splan.rerank(stream)

        for static in (True, False):
            name = "static" if static else "dynamic"
            build_us[name] = time_next(lambda: build(static))
            readout[name] = round(float(splan.value[:, 1:].double().sum(1).mean()), 5)
        del splan
        # Draft steps from hidden states (hidden size 4096, the draft model
        # reusing this vocabulary's LM head): fused (et_draft_step_hidden)
        # against the plain pipeline, torch's GEMM writing bf16 logits then
        # et_draft_step; D steps timed as one call, reported per step.
        H = 4096
        lm = gen.lm_head_inputs(w, H)
        hid = b.dev(lm["hidden"])
        wlm = b.dev(lm["lm_head"])
        del lm
        lplan = d.Plan(w)

        def fused():
            for step in range(1, w.depth + 1):
                lplan.draft_step_hidden(step, ds0["roots"], hid[:, step - 1], wlm, stream)

        def unfused():
            for step in range(1, w.depth + 1):
                logits = torch.nn.functional.linear(hid[:, step - 1], wlm)
                lplan.draft_step(step, ds0["roots"], logits, stream)

        fused_us = time_next(fused) / w.depth
        unfused_us = time_next(unfused) / w.depth
        w_bytes = float(w.vocab) * H * 2
        lm_step = {"hidden_dim": H, "fused_us": round(fused_us, 2),
                   "unfused_us": round(unfused_us, 2),
                   "weight_bytes": int(w_bytes),
                   "fused_gbs": round(w_bytes / fused_us / 1e3, 1),
                   "fused_frac_hbm": round(w_bytes / fused_us / 1e3 / HBM_PEAK_GBS, 4)}
        del hid, wlm, lplan

    alg = b.algorithmic()
    roofline = dominant_roofline(w, alg, avg_us, per_cycle_us)
    calls = call_rooflines(w, alg, avg_us, copy_gbs)
    t_roof = cycle_roof_us(w, alg)

    # ---- CPU oracle baseline and near-tie events on input set 0 ----------
    cpu = ties = None
    if args.cpu_seconds > 0:
        import oracle
        ties = near_ties(b, oracle)
        cpu = cpu_baseline(w, b.host0, args.cpu_seconds, oracle)
    set_mb = round(b.set_bytes / 1e6, 1)
    n_sets, gen_s, mode = len(sets), b.gen_s, "eager" if b.graphs is None else "hip_graph"
    b.release()
    del plan, sets, stream

    # ---- the other large workloads in the same run ------------------------
    others = {}
    if not args.no_extras and args.workload == "llama8b":
        for name in ("llama8b_b64", "llama70b_b8"):
            others[name] = extra_workload(name, args, torch, d, gen, WORKLOADS,
                                          copy_gbs, spin_per_ms)

    line = {
        "metric": "draft-tree build+verify cycles/sec at Llama-3.1-8B shape, "
                  "N=60; % HBM roofline",
        "value": round(1e3 / ms, 2),
        "unit": "cycles/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.logits_dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "vocab": w.vocab,
                   "topk": w.topk, "depth": w.depth, "budget_n": w.budget_n,
                   "heads": f"{w.n_q_heads}/{w.n_kv_heads}x{w.head_dim}",
                   "prefix": list(w.prefix_range), "input_sets": n_sets,
                   "set_mb": set_mb, "mode": mode},
        "roofline": roofline,
        "cycle_roofline_frac": round(t_roof / (ms * 1e3), 4),
        "cycle_roof_us": round(t_roof, 3),
        "calls": calls,
        "hbm_copy_gbs": round(copy_gbs, 1),
        "per_call_us": {n: round(avg_us[n], 3) for n in avg_us},
        "cycle_us_spread": spread,
        "per_cycle_us": {n: round(per_cycle_us[n], 3) for n in per_cycle_us},
        "near_ties": ties,
        "next_calls_us": None if args.no_extras else {
            "kv_commit": round(commit_us, 3),
            "accept_sample": round(sample_us, 3),
            "static_tree_build": round(build_us["static"], 3),
            "dynamic_tree_build": round(build_us["dynamic"], 3)},
        "lm_head_step": lm_step,
        "tree_readout": None if args.no_extras else {
            "expected_accepted_dynamic": readout["dynamic"],
            "expected_accepted_static": readout["static"],
            "static_nodes": int(len(shape_p) - 1)},
        "workloads": others or None,
        "cpu_baseline": cpu,
        "gen_seconds": round(gen_s, 1),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
