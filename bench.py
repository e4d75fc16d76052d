#!/usr/bin/env python3
"""Benchmark of one prioritized-replay step on one MI355X.

A step is the whole hot path over one batch of synthetic input, with every
input already resident in HBM:
    sample(B masses) -> update(the B sampled slots, B TD errors)
    -> intake(count new transitions at the running max priority)
Default workload: the Ape-X replay shard, 2^21 leaves, B = 512, 400-item
intake, indices only.  Prints one JSON line.

The timed region is K steps between two HIP events on the launch stream
(torch's current stream).  A second pass runs each operation on its own, K
back-to-back launches between two events, to time each kernel live; the
roofline figure uses the dominant one.  The CPU baseline is the plain single-threaded oracle
running the same workload for a bounded number of steps on the host.

The roofline's "traffic" is the HBM bytes one launch of the dominant
operation moves as the hardware counts them (rocprofv3 FETCH_SIZE and
WRITE_SIZE per dispatch, each scaled by what the same counter reads for a
plain device copy of known size).  The counters cannot be read from inside
this process, so they are taken in separate profiler runs and ingested into
profiles/hbm_traffic.json together with a digest of the kernel sources; the
figure is reported only while the sources still match that digest.
    python3 bench.py --copy-calibration      # the copy the counters are scaled by
    python3 bench.py --ingest-pmc DIR        # DIR holds the rocprofv3 csv runs
"""
from __future__ import annotations

import argparse
import hashlib
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
CSRC = os.path.join(ROOT, "sum_tree_sampling_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
CALIB_FLOATS = 64 << 20          # 256 MiB copied by --copy-calibration
CALIB_REPS = 3
# Kernels that make up each operation (the sample may be preceded by a top
# rebuild, the update is one kernel or a bucket pass plus its update).
OP_KERNELS = {
    "sample": ("sample_kernel", "top_kernel"),
    "update": ("update_scan_kernel", "bucket_kernel", "update_bucket_kernel"),
    "add": ("add_kernel",),
    "update_add": ("update_add_kernel",),
}


def kernel_source_digest() -> str:
    """sha256 over the HIP sources and headers the counted kernels are built
    from (the rank sort's file is left out: none of them comes from it)."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h")) and f != "rank_kernels.hip":
            h.update(f.encode())
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def _short_kernel(name: str) -> str:
    import re
    name = name.replace("per::(anonymous namespace)::", "").replace("void ", "")
    return re.sub(r"[<(].*$", "", name).strip()


def _counter_rows(path: str) -> dict:
    """{short kernel name: [counter value per dispatch]} of a rocprofv3 csv."""
    import csv
    out: dict = {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            out.setdefault(_short_kernel(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return out


def ingest_pmc(d: str) -> None:
    """Write profiles/hbm_traffic.json from rocprofv3 --pmc csv runs under d:
    d/calib_{FETCH_SIZE,WRITE_SIZE}/run_counter_collection.csv (the copy of
    --copy-calibration) and d/<workload>_{FETCH_SIZE,WRITE_SIZE}/... (this
    bench on that workload).  Per-dispatch values are medians (the few setup
    dispatches of the fill do not move them)."""
    counters = ("FETCH_SIZE", "WRITE_SIZE")
    true_kib = CALIB_FLOATS * 4 / 1024.0
    calib = {}
    for c in counters:
        rows = _counter_rows(os.path.join(d, "calib_%s" % c, "run_counter_collection.csv"))
        copy = [k for k in rows if "copy" in k.lower()]
        if not copy:
            raise SystemExit("no copy kernel in the %s calibration run" % c)
        reported = float(np.median(rows[copy[0]]))
        calib[c] = {"kernel": copy[0], "reported_kib": reported, "true_kib": true_kib,
                    "factor": true_kib / reported}
    res = {"source_sha256": kernel_source_digest(), "calibration": calib, "workloads": {}}
    for w in workloads.WORKLOADS:
        paths = [os.path.join(d, "%s_%s" % (w, c), "run_counter_collection.csv") for c in counters]
        if not all(os.path.exists(p) for p in paths):
            continue
        per_c = [_counter_rows(p) for p in paths]
        ops = {}
        for op, names in OP_KERNELS.items():
            if op in ("add", "update_add") and not workloads.spec(w)["intake"]:
                continue  # only the fill before the timed steps
            kern, tot = {}, 0.0
            for k in names:
                if k not in per_c[0] or len(per_c[0][k]) < 5:
                    continue  # not run, or only by the set-up (the fill's intake)
                f = float(np.median(per_c[0][k])) * calib["FETCH_SIZE"]["factor"] * 1024
                wr = float(np.median(per_c[1][k])) * calib["WRITE_SIZE"]["factor"] * 1024
                kern[k] = {"fetch_bytes": f, "write_bytes": wr, "dispatches": len(per_c[0][k])}
                tot += f + wr
            if kern:
                ops[op] = {"bytes": tot, "kernels": kern}
        res["workloads"][w] = ops
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(res, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps(res, indent=1, sort_keys=True))


def measured_traffic(workload: str, op: str):
    """Counted HBM bytes per launch of op, or None (not profiled, or the
    kernel sources changed since)."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != kernel_source_digest():
        return None
    e = t.get("workloads", {}).get(workload, {}).get(op)
    return None if e is None else float(e["bytes"])


def graph_replay(g, step, K: int, base: int, stream, use_graph_mode: bool = True) -> dict:
    """K whole steps captured as one HIP graph in the library's graph mode
    and replayed: the step time without per-launch host work, a labelled
    extra figure next to the eager headline.  In graph mode the intakes take
    the ring cursor and size from the device, so every replay writes the
    next slots as eager steps would; K is even, so each slot parity
    (running max, overflow list, ring state) is flipped an even number of
    times and a replay starts on the slots the capture started on.  The
    rank-based step re-ranks from the host's filled size, which graph mode
    refuses: it is captured in eager mode, valid while the ring is full (its
    captured intakes rewrite the same slots on every replay)."""
    import torch
    entered = False
    try:
        gr = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(base)  # warm the capture stream
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        if use_graph_mode:
            g.graph_mode(True)
            entered = True
        with torch.cuda.graph(gr):
            for s in range(K):
                step(base + s)
        torch.cuda.synchronize()
        for _ in range(3):
            gr.replay()
        torch.cuda.synchronize()
        reps = 20
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(torch.cuda.current_stream())
        for _ in range(reps):
            gr.replay()
        b.record(torch.cuda.current_stream())
        torch.cuda.synchronize()
        if entered:
            entered = False
            g.graph_mode(False)
        mode = "graph mode, device ring state" if use_graph_mode else "eager mode, full ring"
        return {"steps_per_graph": K, "replays": reps, "mode": mode,
                "ms_per_step": a.elapsed_time(b) / (reps * K)}
    except Exception as e:  # capture not available: report instead of failing the line
        if entered:
            try:
                g.graph_mode(False)
            except Exception:
                pass
        return {"error": "%s: %s" % (type(e).__name__, e)}


def latency_floor() -> dict:
    """The floor under a step of short launches (libper_probe.so): an empty
    kernel launched back to back, and one lane's chain of dependent loads
    through a random cyclic permutation -- in a 1 MiB table, warm in L2 (4
    MiB per XCD), and over 100000 lines (12.5 MiB) of a 64 MiB table, warm
    in the MALL but not in L2.  A descent pays one such load per tree level
    below the levels it keeps in LDS."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "sum_tree_sampling_amd", "libper_probe.so"))
    lib.per_probe_empty.argtypes = [ctypes.c_int64, ctypes.c_void_p]
    lib.per_probe_chain.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_void_p, ctypes.c_void_p]
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def timed(fn) -> float:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    def check(rc):
        if rc != 0:
            raise RuntimeError("latency probe failed (%d)" % rc)

    K = 2000
    check(lib.per_probe_empty(K, sp))
    empty_us = timed(lambda: check(lib.per_probe_empty(K, sp))) * 1e3 / K
    res = {"empty_kernel_us": empty_us}
    rng = np.random.default_rng(0x1A7)
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    for name, nbytes, depth in (("l2", 1 << 20, 20000), ("mall", 64 << 20, 100000)):
        length = nbytes // 4
        order = rng.permutation(length).astype(np.uint32)
        nxt = np.empty(length, np.uint32)
        nxt[order] = np.roll(order, -1)  # one cycle through every slot
        d = torch.from_numpy(nxt.view(np.int32)).cuda()
        torch.cuda.synchronize()
        run = lambda: check(lib.per_probe_chain(ctypes.c_void_p(d.data_ptr()), length, depth,
                                                ctypes.c_void_p(out.data_ptr()), sp))
        run()  # warm: the timed walk revisits the same lines
        res["%s_dependent_load_ns" % name] = timed(run) * 1e6 / depth
        del d
    return res


def copy_calibration() -> None:
    """A plain device-to-device copy of CALIB_FLOATS f32, CALIB_REPS times."""
    import torch
    x = torch.ones(CALIB_FLOATS, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(CALIB_REPS):
        y.copy_(x)
    torch.cuda.synchronize()
    print("copied %d bytes x %d" % (CALIB_FLOATS * 4, CALIB_REPS), flush=True)


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
    if spec.get("masses") == "philox":
        sample -= B * 4                              # masses made on the device
    if spec.get("rank"):
        # ranking: priorities read, ranking written (4 + 4 bytes a slot); the
        # rank-weight descent as the proportional one, plus the order lookup
        sample += 8 * n + 4 * B
    if spec.get("uniform"):
        sample = B * 8                               # index out; no tree walk, no weight
    elif spec["weights"]:
        sample += B * 4
    W = spec.get("out_stride") or D
    if D > 0 and W == D:
        sample += B * 2 * (2 * 4 * D + 9)            # rows + scalars, read and written
    elif D > 0:
        # padded trainer layout: rows read at D, written at W floats; action,
        # reward and done read as 4 + 4 + 1 bytes, written as 4 + 4 + 4
        sample += B * (2 * (4 * D + 4 * W) + 9 + 12)
    update = 0.0 if spec.get("uniform") else B * 12 + U * 8 + 16 * expected_dirty_internal(n, U)
    c = spec["intake"]
    intake = 0.0
    if c:
        intake = 8 * c + 16 * (c + 2 * L)            # leaves + contiguous dirty frontier
    if spec.get("fused"):
        # one launch does both: the bytes of each, nothing shared counted twice
        return {"sample": float(sample), "update_add": float(update + intake)}
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
    ap.add_argument("--padded", type=int, default=0, metavar="STRIDE",
                    help="sample with per_sample_padded into rows of STRIDE floats "
                         "(the trainer layout; workloads with rows only)")
    ap.add_argument("--masses", choices=["array", "philox"], default="array",
                    help="sample masses from a pre-uploaded array (default) or drawn on "
                         "the device (per_sample_philox)")
    ap.add_argument("--uniform", action="store_true",
                    help="prioritisation off: per_sample_uniform, no priority update")
    ap.add_argument("--rank", action="store_true",
                    help="rank-based prioritisation: every step refreshes the ranking "
                         "(per_rank_refresh) and samples with per_sample_rank")
    ap.add_argument("--unfused", action="store_true",
                    help="the step's update and intake as two calls (per_update, per_add) "
                         "instead of the one per_update_add launch")
    ap.add_argument("--no-latency-floor", action="store_true",
                    help="skip the empty-kernel and dependent-load probes (profiling runs)")
    ap.add_argument("--graph-steps", type=int, default=64,
                    help="whole steps captured as one HIP graph for the labelled replay "
                         "figure (even; 0 skips it)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the plain copy the HBM counters are scaled by")
    ap.add_argument("--ingest-pmc", metavar="DIR",
                    help="only write profiles/hbm_traffic.json from rocprofv3 runs in DIR")
    args = ap.parse_args()
    if args.ingest_pmc:
        ingest_pmc(args.ingest_pmc)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the sum tree runs on a single device "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from sum_tree_sampling_amd import PerBuffer

    spec = workloads.spec(args.workload)
    n, B, D = spec["capacity"], spec["batch"], spec["state_dim"]
    if args.padded:
        if D == 0 or args.padded < D:
            raise SystemExit("--padded needs a workload with rows and STRIDE >= state_dim")
        if args.uniform or args.masses != "array" or args.rank:
            raise SystemExit("--padded goes with array masses and proportional sampling")
        spec = dict(spec, out_stride=args.padded)
    if args.rank and (args.uniform or args.masses != "array"):
        raise SystemExit("--rank goes with array masses")
    # The update and the intake of a step in one launch (per_update_add)
    # unless asked for separately; without an update there is nothing to fuse.
    fused = bool(spec["intake"]) and not args.uniform and not args.unfused
    spec = dict(spec, masses=args.masses, uniform=args.uniform, rank=args.rank, fused=fused)
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
    # One view per step, made before timing: indexing a tensor inside the
    # loop costs microseconds of host time per call, which the short steps
    # would otherwise wait on.
    u_d = list(torch.from_numpy(u_all).to(dev).unbind(0))
    td_d = list(torch.from_numpy(td_all).to(dev).unbind(0))
    idx_d = None
    if "unique" in spec:
        idx_d = list(torch.from_numpy(np.stack([inp.update_idx() for _ in range(total)]))
                     .to(dev).unbind(0))
    rows = D > 0
    out = {"idx": torch.empty(B, dtype=torch.int64, device=dev)}
    if spec["weights"]:
        out["w"] = torch.empty(B, dtype=torch.float32, device=dev)
    W = spec.get("out_stride")
    if W:
        out.update(states=torch.empty((B, W), dtype=torch.float32, device=dev),
                   next_states=torch.empty((B, W), dtype=torch.float32, device=dev),
                   actions=torch.empty(B, dtype=torch.int32, device=dev),
                   rewards=torch.empty(B, dtype=torch.float32, device=dev),
                   dones=torch.empty(B, dtype=torch.float32, device=dev))
    elif rows:
        out.update(states=torch.empty((B, D), dtype=torch.float32, device=dev),
                   next_states=torch.empty((B, D), dtype=torch.float32, device=dev),
                   actions=torch.empty(B, dtype=torch.int32, device=dev),
                   rewards=torch.empty(B, dtype=torch.float32, device=dev),
                   dones=torch.empty(B, dtype=torch.uint8, device=dev))
    intake = spec["intake"]

    seed = 0x5EED
    if args.uniform:
        out.pop("w", None)

    if args.rank:
        g.rank_attach()

    def do_sample(s, o):
        if args.rank:
            g.rank_refresh()
            g.sample_rank(u_d[s], beta=spec["beta"], out=o)
        elif args.uniform:
            g.sample_uniform(B, seed, s * B, out=o)
        elif args.masses == "philox":
            g.sample_philox(B, seed, s * B, beta=spec["beta"], out=o)
        elif W:
            g.sample_padded(u_d[s], W, beta=spec["beta"], out=o)
        else:
            g.sample(u_d[s], beta=spec["beta"], weights=spec["weights"], out=o)

    def do_update(s, idx):
        if not args.uniform:
            g.update(idx, td_d[s])

    def step(s):
        do_sample(s, out)
        idx = idx_d[s] if idx_d is not None else out["idx"]
        if fused:
            g.update_add(idx, td_d[s], intake)
        else:
            do_update(s, idx)
            if intake:
                g.add(intake)

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

    # Pass 2: each operation on its own, K back-to-back launches between two
    # events (an event pair around every launch would add its own dispatch
    # gap to each one).  The sampled indices of this pass feed its updates.
    base = args.warmup + args.steps
    idx_hist = torch.empty((args.steps, B), dtype=torch.int64, device=dev)
    ops = {
        "sample": lambda s: do_sample(base + s, dict(out, idx=idx_hist[s])),
    }
    def hist_idx(s):
        return idx_d[base + s] if idx_d is not None else idx_hist[s]

    if fused:
        ops["update_add"] = lambda s: g.update_add(hist_idx(s), td_d[base + s], intake)
    else:
        if not args.uniform:
            ops["update"] = lambda s: g.update(hist_idx(s), td_d[base + s])
        if intake:
            ops["add"] = lambda s: g.add(intake)
    op_avg = {}
    for name, fn in ops.items():
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for s in range(args.steps):
            fn(s)
        b.record(stream)
        torch.cuda.synchronize()
        op_avg[name] = a.elapsed_time(b) / args.steps

    # Pass 3: whole steps again, an event pair around every operation, for the
    # spread of each (every pair also spans the dispatch gap in front of its
    # kernel, so these run above the back-to-back averages).
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for s in range(args.steps):
        e = evs[s]
        e[0].record(stream)
        do_sample(base + s, out)
        e[1].record(stream)
        idx = idx_d[base + s] if idx_d is not None else out["idx"]
        if fused:
            g.update_add(idx, td_d[base + s], intake)
        else:
            do_update(base + s, idx)
        e[2].record(stream)
        if intake and not fused:
            g.add(intake)
        e[3].record(stream)
    torch.cuda.synchronize()
    spread = {}
    names = ["sample", "update_add"] if fused else ["sample", "update", "add"]
    for k, name in enumerate(names):
        if (name == "add" and not intake) or (name == "update" and args.uniform):
            continue
        t = np.array([e[k].elapsed_time(e[k + 1]) for e in evs])
        spread[name] = {q: float(np.percentile(t, v)) for q, v in (("p10", 10), ("p50", 50), ("p90", 90))}

    graph = None
    kg = min(args.graph_steps, args.steps)  # inputs exist for K steps past base
    kg -= kg % 2
    if kg > 0:
        graph = graph_replay(g, step, kg, base, stream, use_graph_mode=not args.rank)

    floor = None
    if not args.no_latency_floor:
        floor = latency_floor()
        floor["kernels_per_step"] = len(op_avg)
        floor["launch_floor_us_per_step"] = floor["empty_kernel_us"] * len(op_avg)

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
                   "weights": spec["weights"], "parallelism": "single GPU",
                   "out_stride": W or D, "masses": args.masses,
                   "update_and_intake": "one launch" if fused else "separate calls",
                   "sampling": ("uniform" if args.uniform else
                                ("rank" if args.rank else "proportional"))},
        "samples_per_s": B / (op_avg["sample"] * 1e-3),
        "updates_per_s": (B / (op_avg["update"] * 1e-3) if "update" in op_avg else
                          (B / (op_avg["update_add"] * 1e-3) if fused else None)),
        "op_ms_avg": op_avg,
        "op_ms_bracketed": spread,
        "graph_replay": graph,
        "latency_floor": floor,
        "host_ms_per_step": host_ms / args.steps,
        "step_algorithmic_bytes": step_bytes,
        "step_hbm_roofline_frac": step_bytes / (ms_per_step * 1e-3) / (PEAK_HBM_GBS * 1e9),
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": measured_traffic(args.workload, dom),
                     "bytes_per_launch": byts[dom]},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(spec, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
