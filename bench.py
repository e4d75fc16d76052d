#!/usr/bin/env python3
"""Benchmark of one prioritized-replay step on one MI355X.

A step is the whole hot path over one batch of synthetic input, with every
input already resident in HBM:
    sample(B masses) -> update(the B sampled slots, B TD errors)
    -> intake(count new transitions at the running max priority)
Default workload: the Ape-X replay shard, 2^21 leaves, B = 512, 400-item
intake, indices only.  Prints one JSON line.

The timed region is K steps between two HIP events on the launch stream
(torch's current stream).  A second pass of K steps records an event
around every operation to time each kernel live; the roofline figure uses
the dominant one.  The CPU baseline is the plain single-threaded oracle
running the same workload for a bounded number of steps on the host.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "PER samples/s + priority updates/s at 2^21 leaves (B=512); % of HBM roofline"
PEAK_HBM_GBS = 8000.0


def expected_dirty_internal(n: int, U: int) -> float:
    """Expected distinct internal ancestors of U uniform distinct leaves."""
    L = int(math.log2(n))
    return sum((2.0 ** l) * (1.0 - (1.0 - 2.0 ** -l) ** U) for l in range(L))


def algorithmic_bytes(spec: dict) -> dict:
    """Bytes each operation must move per launch (per unit x units)."""
    n, B, D = spec["capacity"], spec["batch"], spec["state_dim"]
    L = int(math.log2(n))
    U = spec.get("unique", B)
    sample = B * (4 + 8 * L + 8)                     # mass in, L sibling pairs, index out
    if spec["weights"]:
        sample += B * 4
    if D > 0:
        sample += B * 2 * (2 * 4 * D + 9)            # rows + scalars, read and written
    update = B * 12 + U * 8 + 16 * expected_dirty_internal(n, U)
    c = spec["intake"]
    intake = 0.0
    if c:
        intake = 8 * c + 16 * (c + 2 * L)            # leaves + contiguous dirty frontier
    return {"sample": float(sample), "update": float(update), "add": float(intake)}


def cpu_baseline(spec: dict, seconds: float) -> dict:
    """The oracle, single-threaded, on a bounded number of steps of the workload."""
    import oracle
    n, B = spec["capacity"], spec["batch"]
    o = oracle.Oracle(n, 0)
    pr = workloads.initial_priorities(spec["name"])
    o.add(n, prio=pr)
    inp = workloads.StepInputs(spec["name"])
    steps, t_total = 0, 0.0
    while t_total < seconds and steps < 1_000_000:
        u, td = inp.u(), inp.td()
        t0 = time.perf_counter()
        res = o.sample(u, weights=spec["weights"])
        idx = inp.update_idx() if "unique" in spec else res["idx"]
        o.update(idx, td)
        if spec["intake"]:
            o.add(spec["intake"])
        t_total += time.perf_counter() - t0
        steps += 1
    per_step = t_total / steps
    return {"value": B / per_step, "unit": "samples/s", "cores": 1, "kind": "oracle",
            "sample": "%d steps of %s (sample %d + update %d%s) on the single-threaded C "
                      "oracle, %.1f s of CPU time; host has %d usable cores" % (
                          steps, spec["name"], B, B,
                          (" + intake %d" % spec["intake"]) if spec["intake"] else "",
                          t_total, len(os.sched_getaffinity(0))),
            "ms_per_step": per_step * 1e3}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="apex_shard_2m", choices=list(workloads.WORKLOADS))
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the sum tree runs on a single device "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from sum_tree_sampling_amd import PerBuffer

    spec = workloads.spec(args.workload)
    n, B, D = spec["capacity"], spec["batch"], spec["state_dim"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    g = PerBuffer(n, D, max_batch=B, device=dev)
    pr = workloads.initial_priorities(args.workload)
    chunk = 1 << 20
    for lo in range(0, n, chunk):
        c = min(chunk, n - lo)
        p = None if pr is None else torch.from_numpy(pr[lo:lo + c]).to(dev)
        if D > 0:
            r = workloads.rows(args.workload, lo, c)
            g.add(c, torch.from_numpy(r["states"]).to(dev),
                  torch.from_numpy(r["next_states"]).to(dev),
                  torch.from_numpy(r["actions"].view(np.int32)).to(dev),
                  torch.from_numpy(r["rewards"]).to(dev), torch.from_numpy(r["dones"]).to(dev),
                  prio=p)
        else:
            g.add(c, prio=p)
    torch.cuda.synchronize()

    total = args.warmup + 2 * args.steps
    inp = workloads.StepInputs(args.workload)
    u_all = np.stack([inp.u() for _ in range(total)])
    td_all = np.stack([inp.td() for _ in range(total)])
    u_d = torch.from_numpy(u_all).to(dev)
    td_d = torch.from_numpy(td_all).to(dev)
    idx_d = None
    if "unique" in spec:
        idx_d = torch.from_numpy(np.stack([inp.update_idx() for _ in range(total)])).to(dev)
    rows = D > 0
    out = {"idx": torch.empty(B, dtype=torch.int64, device=dev)}
    if spec["weights"]:
        out["w"] = torch.empty(B, dtype=torch.float32, device=dev)
    if rows:
        out.update(states=torch.empty((B, D), dtype=torch.float32, device=dev),
                   next_states=torch.empty((B, D), dtype=torch.float32, device=dev),
                   actions=torch.empty(B, dtype=torch.int32, device=dev),
                   rewards=torch.empty(B, dtype=torch.float32, device=dev),
                   dones=torch.empty(B, dtype=torch.uint8, device=dev))
    intake = spec["intake"]

    def step(s, ev=None):
        if ev is not None:
            ev[0].record(stream)
        g.sample(u_d[s], beta=spec["beta"], weights=spec["weights"], out=out)
        if ev is not None:
            ev[1].record(stream)
        g.update(idx_d[s] if idx_d is not None else out["idx"], td_d[s])
        if ev is not None:
            ev[2].record(stream)
        if intake:
            g.add(intake)
        if ev is not None:
            ev[3].record(stream)

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()

    # Pass 1: the headline, K whole steps between two events.
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    base = args.warmup
    t0 = time.perf_counter()
    e0.record(stream)
    for s in range(args.steps):
        step(base + s)
    e1.record(stream)
    torch.cuda.synchronize()
    host_ms = (time.perf_counter() - t0) * 1e3
    ms_per_step = e0.elapsed_time(e1) / args.steps

    # Pass 2: an event around every operation of K more steps.
    base = args.warmup + args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for s in range(args.steps):
        step(base + s, evs[s])
    torch.cuda.synchronize()
    op_ms = {"sample": [], "update": [], "add": []}
    for ev in evs:
        op_ms["sample"].append(ev[0].elapsed_time(ev[1]))
        op_ms["update"].append(ev[1].elapsed_time(ev[2]))
        if intake:
            op_ms["add"].append(ev[2].elapsed_time(ev[3]))
    op_avg = {k: float(np.mean(v)) for k, v in op_ms.items() if v}
    op_med = {k: float(np.median(v)) for k, v in op_ms.items() if v}

    byts = algorithmic_bytes(spec)
    dom = max(op_avg, key=op_avg.get)
    achieved = byts[dom] / (op_avg[dom] * 1e-3) / 1e9
    step_bytes = sum(byts.values())

    res = {
        "metric": METRIC,
        "value": B / (ms_per_step * 1e-3),
        "unit": "samples/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "capacity": n, "batch": B, "state_dim": D,
                   "intake": intake, "unique_updates": spec.get("unique", B),
                   "weights": spec["weights"], "parallelism": "single GPU"},
        "samples_per_s": B / (op_avg["sample"] * 1e-3),
        "updates_per_s": B / (op_avg["update"] * 1e-3),
        "op_ms_avg": op_avg,
        "op_ms_median": op_med,
        "host_ms_per_step": host_ms / args.steps,
        "step_algorithmic_bytes": step_bytes,
        "step_hbm_roofline_frac": step_bytes / (ms_per_step * 1e-3) / (PEAK_HBM_GBS * 1e9),
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS, "traffic": None,
                     "bytes_per_launch": byts[dom]},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(spec, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
