#!/usr/bin/env python3
"""Benchmark of one prioritized-replay step on one MI355X.

A step is the whole hot path over one batch of synthetic input, with every
input already resident in HBM:
    sample(B masses) -> update(the B sampled slots, B TD errors)
    -> intake(count new transitions at the running max priority)
Default workload: the Ape-X replay shard, 2^21 leaves, B = 512, 400-item
intake, indices only.  Prints one JSON line.

The timed region is K steps between two HIP events on the launch stream
(torch's current stream); every call of every step is marshalled for the C
ABI before the first event, so the loop does nothing on the host but call
the library.  A second pass times each operation's kernels live, step by
step: per_time_next makes the library launch the operation through
hipExtLaunchKernel with a start and a stop event, which bracket its kernels
on the device (what a kernel trace measures, without the dispatch gap in
front of each launch).  The roofline figure uses the dominant operation by
that time.  A third pass records an event pair around each operation for
comparison.  The other workloads follow as sub-results ("configs").  The CPU
baseline is the plain single-threaded oracle running the same workload on
the host, each call timed in C (bench_oracle.cpp).

The roofline's "traffic" is the HBM bytes one launch of the dominant
operation moves as the hardware counts them (rocprofv3 FETCH_SIZE and
WRITE_SIZE per dispatch, each scaled by what the same counter reads for a
plain device copy of known size).  The counters cannot be read from inside
this process, so they are taken in separate profiler runs and ingested into
profiles/hbm_traffic.json together with a digest of the built library; the
figure is reported only while libper.so still matches that digest.
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
LIBRARY = os.path.join(ROOT, "sum_tree_sampling_amd", "libper.so")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
CALIB_FLOATS = 64 << 20          # 256 MiB copied by --copy-calibration
CALIB_REPS = 3
# Kernels that make up each operation (the sample may be preceded by a top
# rebuild, the update is one kernel or a bucket pass plus its update).
OP_KERNELS = {
    "sample": ("sample_kernel", "top_kernel"),
    "update": ("update_scan_kernel", "bucket_kernel", "update_bucket_kernel",
               "update_bucket_pair_kernel"),
    "add": ("add_kernel",),
    "update_add": ("update_add_kernel",),
}


def library_digest() -> str:
    """sha256 of the built library whose kernels the counters were taken on
    (the build is deterministic: the same sources give the same file)."""
    h = hashlib.sha256()
    with open(LIBRARY, "rb") as fh:
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
    res = {"library_sha256": library_digest(), "calibration": calib, "workloads": {}}
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


def measured_traffic(workload: str, op: str, default_mode: bool = True):
    """Counted HBM bytes per launch of op, or None (not profiled, the library
    rebuilt from changed sources since, or a sampling mode other than the
    default one the counters were taken in: other modes launch other
    kernels)."""
    if not default_mode:
        return None
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    try:
        if t.get("library_sha256") != library_digest():
            return None
    except OSError:
        return None
    e = t.get("workloads", {}).get(workload, {}).get(op)
    return None if e is None else float(e["bytes"])


def latency_floor() -> dict:
    """The floor under a step of short launches (libper_probe.so): an empty
    kernel launched back to back, and one lane's chain of dependent loads
    through a random cyclic permutation -- in a 1 MiB table, warm in L2 (4
    MiB per XCD), and over 100000 lines (12.5 MiB) of a 64 MiB table, warm
    in the MALL but not in L2.  A descent pays one such load per tree level
    below the levels it keeps in LDS.  Also the cost of a launch whose empty
    kernel takes an argument block of 16, 256 or 512 bytes, eager and
    replayed from a graph (the path's kernels take 200-330 bytes)."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "sum_tree_sampling_amd", "libper_probe.so"))
    lib.per_probe_empty.argtypes = [ctypes.c_int64, ctypes.c_void_p]
    lib.per_probe_chain.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_void_p, ctypes.c_void_p]
    lib.per_probe_launch_cost.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                          ctypes.POINTER(ctypes.c_double)]
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
    # what an argument block adds: eager launches wait for the host to write
    # each block to device memory, a graph's replays do not
    for nbytes in (16, 256, 512):
        for graph in (0, 1):
            us = ctypes.c_double(0.0)
            check(lib.per_probe_launch_cost(3000, nbytes, graph, ctypes.byref(us)))
            res["launch_%dB_args_%s_us" % (nbytes, "graph" if graph else "eager")] = us.value
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


STAMPS_LIB = os.path.join(ROOT, "sum_tree_sampling_amd", "libper_stamps.so")
STAMP_SLOTS = 16  # phases per block (include/per_stamps.h)


def step_phases(raw: np.ndarray, entries: np.ndarray | None = None) -> dict:
    """Phase times, in µs from the first block's start, of one launch of the
    fused update + intake kernel, from its stamps (libper_stamps.so; slots as
    in include/per_stamps.h).  raw: [blocks, 16] 100 MHz clock values, 0
    where nothing was stored; values below the launch's first start are a
    launch before's and are dropped.  Blocks that stored slot 3 meet the ring
    range (the intake's); the others end at their repair.  Repair phases are
    taken over the blocks that sorted entries.  entries (optional): the
    update's entries per block (partition), for the median end of the blocks
    without intake by entries held (0 to 4, then 5 or more) and the entries of
    the last of them to end."""
    t = raw.astype(np.float64)
    t0 = t[:, 0][t[:, 0] > 0].min()
    t = np.where(t >= t0, (t - t0) / 100.0, np.nan)
    intake = ~np.isnan(t[:, 3])
    end = np.fmax(t[:, 2], t[:, 5])
    o = ~intake
    rep = o & ~np.isnan(t[:, 14])
    res = {
        "span": float(np.nanmax(end)),
        "others_end_p50": float(np.nanmedian(end[o])),
        "others_end_max": float(np.nanmax(end[o])),
        "scan_wave0_p50": float(np.nanmedian(t[o, 1])),
        "scan_all_waves_p50": float(np.nanmedian(np.nanmax(t[o][:, [1, 10, 11, 12]], axis=1))),
        "repair_start_p50": float(np.nanmedian(t[o, 8])),
        "repair_p50": float(np.nanmedian(t[rep, 2] - t[rep, 8])),
        "repair_sort_p50": float(np.nanmedian(t[rep, 13] - t[rep, 8])),
        "repair_lds_p50": float(np.nanmedian(t[rep, 14] - t[rep, 13])),
        "repair_chain_p50": float(np.nanmedian(t[rep, 2] - t[rep, 14])),
    }
    if intake.any():
        b = np.flatnonzero(intake)[np.nanargmax(end[intake])]
        for k, name in ((1, "scan"), (2, "repair_end"), (3, "boundary_loads"), (4, "barrier"),
                        (5, "climb_end"), (6, "batch_max")):
            res["intake_" + name] = float(t[b, k])
        res["intake_after_others"] = float(end[b] - np.nanmax(end[o]))
    if entries is not None:
        m = np.minimum(entries, 5)
        for k in range(6):
            sel = o & (m == k)
            if sel.any():
                res["end_with_%d%s_entries" % (k, "+" if k == 5 else "")] = float(np.nanmedian(end[sel]))
        oi = np.flatnonzero(o)
        res["last_block_entries"] = float(entries[oi[np.nanargmax(end[oi])]])
    return res


def sampler_spread(raw: np.ndarray) -> dict:
    """Start and end of the proportional sampler's blocks, in µs from the
    launch's first wave start, from its stamps (libper_stamps.so): raw is
    [blocks, 8] 100 MHz clock values, waves' starts in columns 0-3 and ends in
    4-7, 0 where nothing was stored.  A block starts with its first wave and
    ends with its last; blocks are dealt to the XCDs in turn (block mod 8)."""
    t = raw.astype(np.float64)
    used = t[:, 0] > 0
    if not used.any():  # no proportional-sampler launch in the step
        return {}
    t = t[used]
    st, en = t[:, 0:4].min(axis=1), t[:, 4:8].max(axis=1)
    t0 = st.min()
    st, en = (st - t0) / 100.0, (en - t0) / 100.0
    x = np.flatnonzero(used) % 8
    dur = en - st
    return {
        "span": float(en.max()),
        "last_block_start": float(st.max()),
        "block_time_p50": float(np.median(dur)),
        "block_time_max": float(dur.max()),
        "last_end_after_median_end": float(en.max() - np.median(en)),
        **{"xcd%d_start_p50" % k: float(np.median(st[x == k])) for k in range(8) if (x == k).any()},
        **{"xcd%d_last_end" % k: float(en[x == k].max()) for k in range(8) if (x == k).any()},
    }


def phase_stamps(workload: str, groups: int) -> dict:
    """The fused update + intake kernel's phases (step_phases, when the step
    fuses them) and the sampler's block spread (sampler_spread) over `groups`
    launches, each the last of three whole steps after the stamps were
    cleared, with the phase-stamped build in place of libper.so (restored
    after): p10, p50 and p90 of each figure over the launches."""
    from sum_tree_sampling_amd import per
    if not os.path.exists(STAMPS_LIB):
        raise SystemExit("libper_stamps.so not built: run sum_tree_sampling_amd.build.build()")
    prev = per._lib
    per._lib = per.load(STAMPS_LIB)
    try:
        return _phase_stamps_run(per._lib, workload, groups)
    finally:
        per._lib = prev


def _phase_stamps_run(lib, workload: str, groups: int) -> dict:
    import ctypes

    import torch
    lib.per_stamps_clear.argtypes = [ctypes.c_void_p]
    lib.per_stamps_clear.restype = ctypes.c_int
    lib.per_stamps_read.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p]
    lib.per_stamps_read.restype = ctypes.c_int
    lib.per_sample_stamps_clear.argtypes = [ctypes.c_void_p]
    lib.per_sample_stamps_clear.restype = ctypes.c_int
    lib.per_sample_stamps_read.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p]
    lib.per_sample_stamps_read.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    warm, per_group = 50, 3
    run = Run(workload, warm + per_group * groups, {}, dev)
    fused = "update_add" in run.ops
    sp = torch.cuda.current_stream().cuda_stream
    run.run_steps(0, warm, sp)
    torch.cuda.synchronize()
    nb = min(max(run.n >> 12, 1), 4096)  # the update kernel's tree blocks (partitions)
    buf = np.zeros(4096 * STAMP_SLOTS, np.uint64)
    sbuf = np.zeros(4096 * 8, np.uint64)
    rows, srows = [], []
    for gi in range(groups):
        if lib.per_stamps_clear(sp) != 0 or lib.per_sample_stamps_clear(sp) != 0:
            raise RuntimeError("clearing the stamps failed")
        run.run_steps(warm + per_group * gi, per_group, sp)
        if (lib.per_stamps_read(ctypes.c_void_p(buf.ctypes.data), buf.size, sp) != 0 or
                lib.per_sample_stamps_read(ctypes.c_void_p(sbuf.ctypes.data), sbuf.size, sp) != 0):
            raise RuntimeError("reading the stamps failed")
        if fused:
            # the update's entries per partition in the launch read: the last
            # step's batch (the step's own samples unless the workload brings
            # its own update indices)
            last = warm + per_group * gi + per_group - 1
            ui = (run.idx[last] if run.idx is not None else run.out["idx"]).cpu().numpy()
            ui = ui[(ui >= 0) & (ui < run.n)]
            ent = np.bincount(ui >> 12, minlength=nb)[:nb] if run.n >= 4096 else None
            rows.append(step_phases(buf.reshape(4096, STAMP_SLOTS)[:nb], ent))
        srows.append(sampler_spread(sbuf.reshape(4096, 8)))
    run.close()

    def summary(rs):
        keys = sorted({k for r in rs for k in r}, key=lambda k: (k.startswith("xcd"), k))
        return {k: [round(float(np.percentile([r[k] for r in rs if k in r], q)), 3)
                    for q in (10, 50, 90)] for k in keys}

    out = {"sampler": summary([r for r in srows if r])}
    if fused:
        out["update_add"] = summary(rows)
    return out


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
    """Expected distinct internal ancestors of U leaves drawn uniformly with
    replacement (a batch of sampled slots, duplicates included).  For U
    distinct leaves the count is higher by under 0.2% at the workloads'
    sizes (1.1% at 2^10 leaves)."""
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




# ------------------------------------------------------------ CPU baseline

ORACLE_TIMER_SRC = os.path.join(ROOT, "bench_oracle.cpp")
ORACLE_TIMER_LIB = os.path.join(ROOT, "bench_oracle.so")


def build_oracle_timer(force: bool = True) -> str:
    """Compile bench_oracle.cpp and a copy of the oracle (pero.c, with the
    oracle's own flags) into bench_oracle.so next to this file."""
    if not force and os.path.exists(ORACLE_TIMER_LIB):
        return ORACLE_TIMER_LIB
    import subprocess
    import oracle
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    obj = os.path.join(objdir, "pero_timer.o")
    cflags = [f for f in oracle.CFLAGS if f != "-shared"]
    subprocess.check_call(["gcc", *cflags, "-c", os.path.join(ROOT, "oracle", "pero.c"), "-o", obj])
    tmp = ORACLE_TIMER_LIB + ".tmp"
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-I", ROOT, "-o", tmp,
                           ORACLE_TIMER_SRC, obj, "-lm"])
    os.replace(tmp, ORACLE_TIMER_LIB)
    return ORACLE_TIMER_LIB


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(spec: dict, seconds: float) -> dict:
    """The oracle as it stands, one thread, on the workload's own steps: each
    call timed in C with std::chrono::steady_clock (bench_oracle.cpp) until
    `seconds` of CPU time are spent.  Workloads with rows gather them too."""
    import ctypes
    lib = ctypes.CDLL(build_oracle_timer(force=False))
    vp, i64, i32, f64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
    lib.oracle_time_steps.restype = ctypes.c_int
    lib.oracle_time_steps.argtypes = [i64, i32, f64, f64, vp, vp, vp, vp, vp, vp, i64, i64, vp, vp,
                                      vp, i64, f64, i32, i32, i64, f64, vp]
    n, B, D = spec["capacity"], spec["batch"], spec["state_dim"]
    if D > 0:
        raise ValueError("the CPU baseline runs the index-only workloads")
    pr = workloads.initial_priorities(spec["name"])
    inp = workloads.StepInputs(spec["name"])
    nsteps = 256  # inputs cycle after this many steps
    u = np.ascontiguousarray(np.stack([inp.u() for _ in range(nsteps)]))
    td = np.ascontiguousarray(np.stack([inp.td() for _ in range(nsteps)]))
    idx = None
    if "unique" in spec:
        idx = np.ascontiguousarray(np.stack([inp.update_idx() for _ in range(nsteps)]))
    out = (ctypes.c_double * 4)()
    ptr = lambda a: None if a is None else a.ctypes.data
    rc = lib.oracle_time_steps(n, 0, workloads.ALPHA, workloads.EPS, ptr(pr), None, None, None,
                               None, None, B, nsteps, ptr(u), ptr(td), ptr(idx), spec["intake"],
                               spec["beta"], 1 if spec["weights"] else 0, 0, 1_000_000, seconds,
                               out)
    if rc != 0:
        raise RuntimeError("oracle timing failed")
    ts, tu, ta, steps = out[0], out[1], out[2], int(out[3])
    per_step = (ts + tu + ta) / steps
    return {"value": B / per_step, "unit": "samples/s", "cores": 1, "kind": "oracle",
            "sample": "%d steps of %s (sample %d + update %d%s) on the single-threaded C oracle, "
                      "each call timed with std::chrono::steady_clock, %.1f s of CPU time; "
                      "CPU %s, %d usable cores on the host" % (
                          steps, spec["name"], B, B,
                          (" + intake %d" % spec["intake"]) if spec["intake"] else "",
                          ts + tu + ta, cpu_model(), len(os.sched_getaffinity(0))),
            "ms_per_step": per_step * 1e3,
            "op_ms": {"sample": ts / steps * 1e3, "update": tu / steps * 1e3,
                      **({"add": ta / steps * 1e3} if spec["intake"] else {})},
            "cpu_model": cpu_model()}


# ------------------------------------------------------------ GPU runs

class Run:
    """One workload on the GPU: the buffer filled, every step's inputs
    resident in HBM, and each step's calls marshalled for the C ABI ahead of
    time, so that the timed loops do nothing on the host but call into the
    library.  Rows are drawn on the device (torch's generator, seeded; the
    workload's distributions): their values never change a step's work,
    which only copies them."""

    def __init__(self, name: str, steps_total: int, mode: dict, dev):
        import torch
        from sum_tree_sampling_amd import PerBuffer, per
        self.torch = torch
        self.lib = per.load()
        spec = workloads.spec(name)
        self.name = name
        n, B, D = spec["capacity"], spec["batch"], spec["state_dim"]
        self.n, self.B, self.D = n, B, D
        W = mode.get("padded") or 0
        if W:
            spec = dict(spec, out_stride=W)
        self.uniform, self.rank = mode.get("uniform", False), mode.get("rank", False)
        self.masses = mode.get("masses", "array")
        self.fused = bool(spec["intake"]) and not self.uniform and not mode.get("unfused", False)
        # the mode the HBM counters of the traffic file are taken in
        self.default_mode = (not W and not self.uniform and not self.rank
                             and self.masses == "array" and not mode.get("unfused", False))
        self.spec = dict(spec, masses=self.masses, uniform=self.uniform, rank=self.rank,
                         fused=self.fused)
        self.W = W
        self.dev = dev
        self.g = g = PerBuffer(n, D, max_batch=B, device=dev)
        pr = workloads.initial_priorities(name)
        gen = torch.Generator(device=dev)
        gen.manual_seed(spec["seed"])
        chunk = 1 << 20
        for lo in range(0, n, chunk):
            c = min(chunk, n - lo)
            p = None if pr is None else torch.from_numpy(pr[lo:lo + c]).to(dev)
            if D > 0:
                g.add(c, torch.randn((c, D), generator=gen, device=dev),
                      torch.randn((c, D), generator=gen, device=dev),
                      torch.randint(0, 3, (c,), generator=gen, device=dev, dtype=torch.int32),
                      torch.randn(c, generator=gen, device=dev),
                      (torch.rand(c, generator=gen, device=dev) < 0.01).to(torch.uint8), prio=p)
            else:
                g.add(c, prio=p)
        torch.cuda.synchronize()
        if self.rank:
            g.rank_attach()
        inp = workloads.StepInputs(name)
        self.u = torch.from_numpy(np.stack([inp.u() for _ in range(steps_total)])).to(dev)
        self.td = torch.from_numpy(np.stack([inp.td() for _ in range(steps_total)])).to(dev)
        self.idx = None
        if "unique" in spec:
            self.idx = torch.from_numpy(np.stack([inp.update_idx() for _ in range(steps_total)])
                                        ).to(dev)
        self.steps_total = steps_total
        out = {"idx": torch.empty(B, dtype=torch.int64, device=dev)}
        if spec["weights"] and not self.uniform:
            out["w"] = torch.empty(B, dtype=torch.float32, device=dev)
        if D > 0:
            Wo = W or D
            out.update(states=torch.empty((B, Wo), dtype=torch.float32, device=dev),
                       next_states=torch.empty((B, Wo), dtype=torch.float32, device=dev),
                       actions=torch.empty(B, dtype=torch.int32, device=dev),
                       rewards=torch.empty(B, dtype=torch.float32, device=dev),
                       dones=torch.empty(B, dtype=torch.float32 if W else torch.uint8,
                                         device=dev))
        self.out = out
        self.ops = (["sample", "update_add"] if self.fused else
                    ["sample"] + ([] if self.uniform else ["update"]) +
                    (["add"] if spec["intake"] else []))
        self.torch.cuda.synchronize()

    def calls(self, s: int, sp: int):
        """[(op, [(c function, args), ...]), ...] of step s on stream sp."""
        lib, h, B, spec = self.lib, self.g.h, self.B, self.spec
        o = {k: v.data_ptr() for k, v in self.out.items()}
        rows = [o.get("states"), o.get("next_states")]
        scal = [o.get("actions"), o.get("rewards"), o.get("dones")]
        u = self.u[s].data_ptr()
        td = self.td[s].data_ptr()
        beta, seed = spec["beta"], 0x5EED
        if self.rank:
            smp = [(lib.per_rank_refresh, (h, sp)),
                   (lib.per_sample_rank, (h, B, u, beta, o["idx"], o.get("w"), *rows, *scal, sp))]
        elif self.uniform:
            smp = [(lib.per_sample_uniform, (h, B, seed, s * B, o["idx"], *rows, *scal, sp))]
        elif self.masses == "philox":
            smp = [(lib.per_sample_philox, (h, B, seed, s * B, beta, o["idx"], o.get("w"), *rows,
                                            *scal, sp))]
        elif self.W:
            smp = [(lib.per_sample_padded, (h, B, u, beta, o["idx"], o.get("w"), *rows, self.W,
                                            *scal, sp))]
        else:
            smp = [(lib.per_sample, (h, B, u, beta, o["idx"], o.get("w"), *rows, *scal, sp))]
        res = [("sample", smp)]
        ui = self.idx[s].data_ptr() if self.idx is not None else o["idx"]
        c = spec["intake"]
        if self.fused:
            res.append(("update_add", [(lib.per_update_add, (h, B, ui, td, c, None, None, None,
                                                             None, None, None, sp))]))
        else:
            if not self.uniform:
                res.append(("update", [(lib.per_update, (h, B, ui, td, sp))]))
            if c:
                res.append(("add", [(lib.per_add, (h, c, None, None, None, None, None, None,
                                                   sp))]))
        return res

    def check(self, rc: int):
        if rc != 0:
            from sum_tree_sampling_amd import per
            raise RuntimeError("per call failed: %s" % per.per_last_error())

    def run_steps(self, first: int, count: int, sp: int):
        rc = 0
        for s in range(first, first + count):
            for _, cl in self.calls(s, sp):
                for f, a in cl:
                    rc |= f(*a)
        self.check(rc)

    def timed_steps(self, first: int, count: int, stream) -> float:
        """ms per step over `count` whole steps between two events; the
        calls are marshalled before the first event."""
        torch = self.torch
        sp = stream.cuda_stream
        plan = [[(f, a) for _, cl in self.calls(s, sp) for f, a in cl]
                for s in range(first, first + count)]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        rc = 0
        e0.record(stream)
        for st in plan:
            for f, a in st:
                rc |= f(*a)
        e1.record(stream)
        torch.cuda.synchronize()
        self.check(rc)
        return e0.elapsed_time(e1) / count

    def kernel_times(self, first: int, count: int, stream) -> dict:
        """Per op, the span of its kernels on the device in each of `count`
        whole steps (per_time_next: the first kernel's start to the last
        kernel's end, through hipExtLaunchKernel's events), in ms."""
        torch = self.torch
        lib = self.lib
        sp = stream.cuda_stream
        nops = len(self.ops)
        evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(nops)] for _ in range(count)]
        for row in evs:  # torch creates an event when it is first recorded
            for a, b in row:
                a.record(stream)
                b.record(stream)
        torch.cuda.synchronize()
        plan = []
        for k, s in enumerate(range(first, first + count)):
            st = []
            for j, (op, cl) in enumerate(self.calls(s, sp)):
                a, b = evs[k][j]
                for i, (f, args) in enumerate(cl):
                    start = a.cuda_event if i == 0 else None
                    stop = b.cuda_event if i == len(cl) - 1 else None
                    st.append((lib.per_time_next, (start, stop)))
                    st.append((f, args))
            plan.append(st)
        rc = 0
        for st in plan:
            for f, a in st:
                rc |= f(*a)
        torch.cuda.synchronize()
        self.check(rc)
        return {op: np.array([evs[k][j][0].elapsed_time(evs[k][j][1]) for k in range(count)])
                for j, op in enumerate(self.ops)}

    def bracketed_times(self, first: int, count: int, stream) -> dict:
        """Per op, an event pair recorded around its calls in each of
        `count` whole steps (each pair also spans the dispatch gap in front
        of the op's first kernel), in ms."""
        torch = self.torch
        sp = stream.cuda_stream
        nops = len(self.ops)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nops + 1)]
               for _ in range(count)]
        plan = [self.calls(s, sp) for s in range(first, first + count)]
        rc = 0
        for k, st in enumerate(plan):
            evs[k][0].record(stream)
            for j, (_, cl) in enumerate(st):
                for f, a in cl:
                    rc |= f(*a)
                evs[k][j + 1].record(stream)
        torch.cuda.synchronize()
        self.check(rc)
        return {op: np.array([evs[k][j].elapsed_time(evs[k][j + 1]) for k in range(count)])
                for j, op in enumerate(self.ops)}

    def graph_replay(self, first: int, K: int) -> dict:
        """K whole steps captured as one HIP graph in the library's graph mode
        and replayed: the step time without per-launch host work, a labelled
        extra figure next to the eager headline.  In graph mode the intakes
        take the ring cursor and size from the device, so every replay writes
        the next slots as eager steps would; K is even, so each slot parity
        (running max, overflow list, ring state) is flipped an even number of
        times and a replay starts on the slots the capture started on.  The
        rank-based step re-ranks from the host's filled size, which graph mode
        refuses: it is captured in eager mode, valid while the ring is full
        (its captured intakes rewrite the same slots on every replay)."""
        torch = self.torch
        g = self.g
        use_graph_mode = not self.rank
        entered = False
        try:
            gr = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                self.run_steps(first, 1, side.cuda_stream)  # warm the capture stream
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            if use_graph_mode:
                g.graph_mode(True)
                entered = True
            with torch.cuda.graph(gr):
                self.run_steps(first, K, torch.cuda.current_stream().cuda_stream)
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

    def close(self):
        self.g.close()
        self.g = None
        self.u = self.td = self.idx = self.out = None


def progress(*a) -> None:
    print("bench:", *a, file=sys.stderr, flush=True)


def pct(t: np.ndarray) -> dict:
    return {q: float(np.percentile(t, v)) for q, v in (("p10", 10), ("p50", 50), ("p90", 90))}


def central_mean(t: np.ndarray) -> float:
    """Mean of the values between the 25th and 75th percentile: steps whose
    timing events are held up (more than a tenth of them in some runs) read
    twice the kernel's span or more, and the plain mean then lies above the
    kernel durations a profiler's trace reports for the same kernels."""
    lo, hi = np.percentile(t, [25, 75])
    return float(t[(t >= lo) & (t <= hi)].mean())


def measure(run: Run, K: int, W: int, Kop: int, stream, graph_steps: int = 0) -> dict:
    """The headline pass and the per-op passes of one workload."""
    run.run_steps(0, W, stream.cuda_stream)
    run.torch.cuda.synchronize()
    ms_per_step = run.timed_steps(W, K, stream)
    base = W + K
    kt = run.kernel_times(base, Kop, stream)
    br = run.bracketed_times(base, min(K, Kop), stream)
    op_avg = {op: central_mean(t) for op, t in kt.items()}
    byts = algorithmic_bytes(run.spec)
    dom = max(op_avg, key=op_avg.get)
    achieved = byts[dom] / (op_avg[dom] * 1e-3) / 1e9
    step_bytes = sum(byts.values())
    B = run.B
    upd = "update_add" if run.fused else ("update" if "update" in op_avg else None)
    res = {
        "ms_per_step": ms_per_step,
        "samples_per_s": B / (op_avg["sample"] * 1e-3),
        "updates_per_s": None if upd is None else B / (op_avg[upd] * 1e-3),
        "op_ms_avg": op_avg,
        "op_ms_mean": {op: float(t.mean()) for op, t in kt.items()},
        "op_ms_kernel": {op: pct(t) for op, t in kt.items()},
        "op_ms_bracketed": {op: pct(t) for op, t in br.items()},
        "op_steps": Kop,
        "step_algorithmic_bytes": step_bytes,
        "step_hbm_roofline_frac": step_bytes / (ms_per_step * 1e-3) / (PEAK_HBM_GBS * 1e9),
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": measured_traffic(run.name, dom, run.default_mode),
                     "bytes_per_launch": byts[dom]},
    }
    if graph_steps > 0:
        res["graph_replay"] = run.graph_replay(base, graph_steps)
    return res


def config_of(run: Run, args_masses: str = "array") -> dict:
    spec = run.spec
    return {"workload": run.name, "capacity": run.n, "batch": run.B, "state_dim": run.D,
            "intake": spec["intake"], "unique_updates": spec.get("unique", run.B),
            "weights": spec["weights"], "parallelism": "single GPU",
            "out_stride": run.W or run.D, "masses": run.masses,
            "update_and_intake": "one launch" if run.fused else "separate calls",
            "sampling": "uniform" if run.uniform else ("rank" if run.rank else "proportional")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="apex_shard_2m", choices=list(workloads.WORKLOADS))
    ap.add_argument("--op-steps", type=int, default=200,
                    help="steps of the per-operation kernel-timing pass (at least --steps)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="measure only --workload, not the other workloads as well")
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
    ap.add_argument("--phase-stamps", type=int, default=0, metavar="LAUNCHES",
                    help="only print the per-block phase times of the fused update + intake "
                         "kernel and the sampler's block spread over LAUNCHES launches "
                         "(libper_stamps.so)")
    args = ap.parse_args()
    if args.ingest_pmc:
        ingest_pmc(args.ingest_pmc)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.phase_stamps:
        print(json.dumps({"workload": args.workload, "launches": args.phase_stamps,
                          "unit": "us (p10, p50, p90)",
                          "phases": phase_stamps(args.workload, args.phase_stamps)}), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the sum tree runs on a single device "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    spec = workloads.spec(args.workload)
    D = spec["state_dim"]
    if args.padded:
        if D == 0 or args.padded < D:
            raise SystemExit("--padded needs a workload with rows and STRIDE >= state_dim")
        if args.uniform or args.masses != "array" or args.rank:
            raise SystemExit("--padded goes with array masses and proportional sampling")
    if args.rank and (args.uniform or args.masses != "array"):
        raise SystemExit("--rank goes with array masses")
    mode = dict(padded=args.padded, masses=args.masses, uniform=args.uniform, rank=args.rank,
                unfused=args.unfused)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    K, W = args.steps, args.warmup
    Kop = max(K, args.op_steps)
    kg = min(args.graph_steps, Kop)
    kg -= kg % 2
    progress("filling", args.workload)
    run = Run(args.workload, W + K + Kop, mode, dev)
    progress("timing", args.workload)
    m = measure(run, K, W, Kop, stream, graph_steps=kg)
    floor = None
    if not args.no_latency_floor:
        floor = latency_floor()
        floor["kernels_per_step"] = len(run.ops)
        floor["launch_floor_us_per_step"] = floor["empty_kernel_us"] * len(run.ops)
    res = {
        "metric": METRIC,
        "value": run.B / (m["ms_per_step"] * 1e-3),
        "unit": "samples/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": config_of(run),
        **{k: v for k, v in m.items() if k != "ms_per_step"},
        "latency_floor": floor,
        "cpu_baseline": None,
    }
    spec_run = run.spec
    run.close()
    del run
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline and spec_run["state_dim"] == 0:
        progress("cpu baseline")
        res["cpu_baseline"] = cpu_baseline(spec_run, args.cpu_seconds)
    if not args.no_configs:
        # The other workloads, each with the same number of timed steps (at
        # most 200) and the default sampling mode: parity-test shapes, shown
        # as sub-results next to the headline.
        subs = {}
        Ks, Ws = min(K, 200), min(W, 20)
        Kops = max(Ks, min(Kop, 200))
        for name in workloads.WORKLOADS:
            if name == args.workload:
                continue
            progress("filling", name)
            r = Run(name, Ws + Ks + Kops, {}, dev)
            progress("timing", name)
            sm = measure(r, Ks, Ws, Kops, stream)
            subs[name] = {"config": config_of(r), "steps": Ks, "warmup": Ws, **sm}
            r.close()
            del r
            torch.cuda.empty_cache()
        res["configs"] = subs
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
