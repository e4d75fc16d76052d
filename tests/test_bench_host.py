"""Host-side logic of bench.py: the algorithmic byte counts the roofline
divides by, and when a counted-traffic figure may be reported."""
import json

import numpy as np
import pytest

import bench
import workloads


def test_expected_dirty_internal_matches_simulation():
    # expected number of distinct internal ancestors of U leaves drawn
    # uniformly with replacement, against a count over random draws on a
    # 2^10-leaf tree
    rng = np.random.default_rng(7)
    n, U, trials = 1 << 10, 64, 400
    L = 10
    counts = []
    for _ in range(trials):
        leaves = rng.integers(0, n, U)
        nodes = set()
        for leaf in leaves:
            v = int(leaf) + n  # heap numbering: root 1, leaves n..2n-1
            while v > 1:
                v //= 2
                nodes.add(v)
        counts.append(len(nodes))
    assert bench.expected_dirty_internal(n, U) == pytest.approx(np.mean(counts), rel=0.01)
    # every leaf dirties the root; one leaf dirties exactly L internal nodes
    assert bench.expected_dirty_internal(n, 1) == pytest.approx(L)
    # many draws dirty every internal node
    assert bench.expected_dirty_internal(n, 1 << 16) == pytest.approx(n - 1)


def test_apex_step_bytes():
    spec = dict(workloads.spec("apex_shard_2m"), masses="array", fused=True)
    b = bench.algorithmic_bytes(spec)
    assert set(b) == {"sample", "update_add"}
    # 512 descents over 21 levels: mass in, 21 sibling pairs, index out (no
    # weights in this workload)
    assert not spec["weights"]
    assert b["sample"] == 512 * (4 + 8 * 21 + 8)
    assert sum(b.values()) == pytest.approx(0.212e6, rel=0.01)
    sep = bench.algorithmic_bytes(dict(spec, fused=False))
    assert sep["update"] + sep["add"] == pytest.approx(b["update_add"])


def test_traffic_only_for_the_profiled_mode():
    with open(bench.TRAFFIC_FILE) as fh:
        t = json.load(fh)
    e = t["workloads"]["apex_shard_2m"]["update_add"]["bytes"]
    assert bench.measured_traffic("apex_shard_2m", "update_add", False) is None
    got = bench.measured_traffic("apex_shard_2m", "update_add", True)
    if t.get("library_sha256") == bench.library_digest():
        assert got == pytest.approx(float(e))
    else:
        assert got is None
    assert bench.measured_traffic("no_such_workload", "sample", True) is None


def test_build_refuses_scratch():
    # the build reads the compiler's per-kernel resource report and refuses
    # kernels that keep values in scratch memory
    from sum_tree_sampling_amd import build
    report = "\n".join([
        "x.hip:10:1: remark: Function Name: _Z1av [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:10:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "   10 | __global__ void a() {",
        "      | ^",
        "x.hip:20:1: remark: Function Name: _Z1bv [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:20:1: remark:     ScratchSize [bytes/lane]: 32 [-Rpass-analysis=kernel-resource-usage]",
    ])
    assert build.scratch_users(report) == [("_Z1bv", 32)]
    assert build.scratch_users("") == []


def test_central_mean():
    # the mean of the values between the 25th and 75th percentile: outliers
    # at either end do not move it
    t = np.concatenate([np.full(80, 4.0), np.full(20, 40.0)])
    assert bench.central_mean(t) == pytest.approx(4.0)
    assert bench.central_mean(np.arange(1, 101, dtype=float)) == pytest.approx(50.5, abs=0.6)


def test_step_phases():
    # four blocks (100 MHz ticks): three without intake, one meeting the ring
    # range; a stale slot from an earlier launch (below the first start) is
    # dropped, so block 1 does not count as an intake block
    raw = np.zeros((4, 16), np.uint64)
    t0 = 10_000
    for b in range(4):
        raw[b, 0] = t0 + 10 * b
        raw[b, 1] = t0 + 100
        raw[b, [10, 11, 12]] = t0 + 150
        raw[b, 8] = t0 + 200
        raw[b, 13] = t0 + 220
        raw[b, 14] = t0 + 230
        raw[b, 2] = t0 + 300 + 10 * b
    raw[1, 3] = t0 - 5  # stale
    raw[3, [6, 3, 4, 5]] = [t0 + 350, t0 + 400, t0 + 420, t0 + 500]
    r = bench.step_phases(raw)
    assert r["span"] == pytest.approx(5.0)
    assert r["others_end_max"] == pytest.approx(3.2)
    assert r["others_end_p50"] == pytest.approx(3.1)
    assert r["scan_all_waves_p50"] == pytest.approx(1.5)
    assert r["repair_p50"] == pytest.approx(1.1)
    assert r["repair_sort_p50"] == pytest.approx(0.2)
    assert r["repair_lds_p50"] == pytest.approx(0.1)
    assert r["repair_chain_p50"] == pytest.approx(0.8)
    assert r["intake_climb_end"] == pytest.approx(5.0)
    assert r["intake_batch_max"] == pytest.approx(3.5)
    assert r["intake_after_others"] == pytest.approx(1.8)
    # with the update's entries per partition: block ends by entries held
    # (block 3 meets the ring range and is left out), and the last block's
    r = bench.step_phases(raw, np.array([0, 7, 1, 2]))
    assert r["end_with_0_entries"] == pytest.approx(3.0)
    assert r["end_with_1_entries"] == pytest.approx(3.2)
    assert r["end_with_5+_entries"] == pytest.approx(3.1)
    assert "end_with_2_entries" not in r
    assert r["last_block_entries"] == 1


def test_sampler_spread():
    # 16 blocks of 4 waves; block b's waves start at 10b, 10b+1, ... ticks and
    # end 2000 ticks later, except block 13 (XCD 5), which ends 500 later
    raw = np.zeros((4096, 8), np.uint64)
    t0 = 50_000
    for b in range(16):
        raw[b, 0:4] = t0 + 10 * b + np.arange(4)
        raw[b, 4:8] = t0 + 10 * b + 2000 + np.arange(4)
    raw[13, 7] += 500
    r = bench.sampler_spread(raw)
    assert r["last_block_start"] == pytest.approx(1.5)
    assert r["block_time_p50"] == pytest.approx(20.03)
    assert r["block_time_max"] == pytest.approx(25.03)
    assert r["span"] == pytest.approx(1.3 + 25.03)
    assert r["xcd5_start_p50"] == pytest.approx(0.9)  # blocks 5 and 13
    assert r["xcd5_last_end"] == pytest.approx(1.3 + 25.03)
    assert r["xcd0_last_end"] == pytest.approx(0.8 + 20.03)


def test_sampler_spread_without_stamps():
    # a step without a proportional-sampler launch leaves no stamps
    assert bench.sampler_spread(np.zeros((4096, 8), np.uint64)) == {}
