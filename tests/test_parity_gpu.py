"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Trees, indices, rows and the running max are compared
bit for bit; IS weights within 1e-6 relative."""
import numpy as np
import pytest
import torch

import workloads
from oracle import Oracle
from parity_util import (compare_sample, compare_trees, compare_weights, dev, fill, host, say,
                         assert_bits_equal)

pytestmark = pytest.mark.gpu


def _buf(n, D=0, max_batch=4096, **kw):
    from sum_tree_sampling_amd import PerBuffer
    return PerBuffer(n, D, max_batch=max_batch, **kw)


# ------------------------------------------------------------ the five workloads

STEPS = {"tiny_1k": 30, "apex_shard_2m": 6, "dqn_1m": 3, "collision_stress_2m": 3}


@pytest.mark.parametrize("name", list(STEPS))
def test_workload_parity(name):
    s = workloads.spec(name)
    n, B, D = s["capacity"], s["batch"], s["state_dim"]
    say("workload", name, "n", n, "B", B, "D", D)
    o = Oracle(n, D)
    g = _buf(n, D, max_batch=max(B, 4096))
    fill(name, o, g)
    compare_trees(o, g, name + " after fill")
    inp = workloads.StepInputs(name)
    rows = D > 0
    for step in range(STEPS[name]):
        u = inp.u()
        ro = o.sample(u, beta=s["beta"], weights=True, rows=rows)
        rg = g.sample(dev(u), beta=s["beta"], weights=True, rows=rows)
        compare_sample(rg, ro, "%s step %d sample" % (name, step), rows=rows)
        # sampling leaves the trees as they were (read through per_flush,
        # which stores any top levels the writers left pending)
        compare_trees(o, g, "%s step %d after sample" % (name, step))
        idx = inp.update_idx() if "unique" in s else ro["idx"]
        td = inp.td()
        o.update(idx, td)
        if s["intake"] and step % 2:
            # the update and the intake in one launch, as the benchmark runs them
            o.add(s["intake"])
            g.update_add(dev(idx), dev(td), s["intake"])
            compare_trees(o, g, "%s step %d update + intake" % (name, step))
            continue
        g.update(dev(idx), dev(td))
        compare_trees(o, g, "%s step %d update" % (name, step))
        if s["intake"]:
            o.add(s["intake"])
            g.add(s["intake"])
            compare_trees(o, g, "%s step %d intake" % (name, step))
    say("workload", name, "ok")


# Lanes per sample of each descent layout (per_set_sample_lanes).
LANES = {"1": 64, "2": 16, "3": 1}


@pytest.mark.parametrize("mode", ["1", "2", "3"])
def test_sampler_modes_agree(mode):
    """Each descent variant (one wave, 16 lanes, one lane per sample) returns
    the oracle's indices, weights and rows."""
    n, D = 1 << 20, 64
    say("sampler mode", mode)
    o = Oracle(n, D)
    g = _buf(n, D, max_batch=20000)
    g.set_sample_lanes(LANES[mode])
    fill("dqn_1m", o, g)
    # non-uniform priorities so that every level matters
    inp = workloads.StepInputs("dqn_1m", batch=3000)
    idx = np.arange(0, n, 7, dtype=np.int64)
    td = np.random.default_rng(5).standard_normal(idx.size).astype(np.float32) * 3
    o.update(idx, td)
    for lo in range(0, idx.size, 20000):
        g.update(dev(idx[lo:lo + 20000]), dev(td[lo:lo + 20000]))
    compare_trees(o, g, "mode %s prep" % mode)
    for rep in range(3):
        u = inp.u()
        u[:3] = [0.0, np.nextafter(np.float32(1), np.float32(0)), 0.5]
        ro = o.sample(u, beta=0.4, rows=True)
        rg = g.sample(dev(u), beta=0.4, rows=True)
        compare_sample(rg, ro, "mode %s batch %d" % (mode, rep), rows=True)
        compare_trees(o, g, "mode %s batch %d tree" % (mode, rep))


@pytest.mark.parametrize("L", [22, 23, 24])
def test_sampler_top_depths(L):
    """Trees of 2^22 to 2^24 leaves (10 to 12 levels above the 4096-leaf
    partitions, each a variant of its own) in every descent mode, before and
    after an update: indices bit for bit, weights within 1e-6."""
    n = 1 << L
    say("top depth", L)
    rng = np.random.default_rng(L)
    o = Oracle(n)
    g = _buf(n, max_batch=4096)
    p0 = (rng.random(n) ** 0.6).astype(np.float32)
    o.add(n, prio=p0)
    g.add(n, prio=dev(p0))
    for step in range(2):
        for mode in ("1", "2", "3"):
            g.set_sample_lanes(LANES[mode])
            u = rng.random(700, dtype=np.float32)
            u[:2] = [0.0, np.nextafter(np.float32(1), np.float32(0))]
            compare_sample(g.sample(dev(u), beta=0.4), o.sample(u, beta=0.4),
                           "L=%d step %d mode %s" % (L, step, mode))
        g.set_sample_lanes(0)
        idx = rng.integers(0, n, 3000).astype(np.int64)
        td = (rng.standard_normal(3000) * 2).astype(np.float32)
        o.update(idx, td)
        g.update(dev(idx), dev(td))
        compare_trees(o, g, "L=%d step %d update" % (L, step))


def test_zero_priorities_never_sampled():
    name = "collision_stress_2m"
    n = 1 << 21
    say("zeros", name)
    o = Oracle(n)
    g = _buf(n)
    pr = fill(name, o, g)
    rng = np.random.default_rng(3)
    for mode in ("1", "2", "3"):
        g.set_sample_lanes(LANES[mode])
        u = rng.random(4096, dtype=np.float32)
        u[:64] = np.float32(1) - np.float32(2.0 ** -24) * np.arange(1, 65, dtype=np.float32)
        ro = o.sample(u, weights=False)
        rg = g.sample(dev(u), weights=True)
        compare_sample(rg, ro, "zeros mode " + mode, weights=False)
        got = host(rg["idx"])
        assert np.all(pr[got] > 0)
        assert np.all(host(rg["w"]) == 0.0)  # min priority is 0


# ------------------------------------------------------------ update paths

@pytest.mark.parametrize("n,B,dense", [
    (1 << 14, 40, False),          # sparse chains, 4 partitions
    (1 << 14, 3000, True),         # dense partitions
    (1 << 20, 1 << 15, False),     # bucketed large-batch path
    (1 << 12, 4096, True),         # single partition, every slot
])
def test_update_paths(n, B, dense):
    say("update paths", n, B, dense)
    rng = np.random.default_rng(n + B)
    o = Oracle(n)
    g = _buf(n, max_batch=B)
    p0 = (rng.random(n) * 2).astype(np.float32)
    o.add(n, prio=p0)
    g.add(n, prio=dev(p0))
    for step in range(4):
        if dense:
            lo = int(rng.integers(0, n - min(n, 4096) + 1))
            idx = lo + rng.integers(0, min(n, 4096), B)
        else:
            idx = rng.integers(0, n, B)
        idx[: B // 5] = idx[B // 5: 2 * (B // 5)]          # duplicates, last wins
        idx[::97] = rng.integers(n, n + 5, idx[::97].size)  # skipped
        idx[1::89] = -1
        td = rng.standard_normal(B).astype(np.float32)
        td[::53] = np.nan
        td[3::71] = np.inf
        td[5::71] = -np.inf
        o.update(idx.astype(np.int64), td)
        g.update(dev(idx, np.int64), dev(td))
        compare_trees(o, g, "update n=%d B=%d step %d" % (n, B, step))


def test_update_all_entries_one_slot():
    n, B = 1 << 16, 5000
    o = Oracle(n)
    g = _buf(n, max_batch=B)
    o.add(n)
    g.add(n)
    idx = np.full(B, 12345, np.int64)
    td = np.linspace(-3, 3, B).astype(np.float32)
    o.update(idx, td)
    g.update(dev(idx), dev(td))
    compare_trees(o, g, "one slot")


# ------------------------------------------------------------ intake and ring

@pytest.mark.parametrize("n", [2, 4, 64, 1 << 12, 1 << 13, 1 << 16])
def test_ring_intake_and_random_ops(n):
    say("ring", n)
    rng = np.random.default_rng(n)
    D = 5  # not a multiple of 4: scalar row copies
    o = Oracle(n, D)
    g = _buf(n, D, max_batch=256)
    for step in range(25):
        c = int(rng.integers(1, n + 1)) if step % 5 == 0 else int(rng.integers(1, max(2, n // 3)))
        c = min(c, n)
        st = rng.standard_normal((c, D)).astype(np.float32)
        nx = rng.standard_normal((c, D)).astype(np.float32)
        ac = rng.integers(0, 3, c).astype(np.uint32)
        rw = rng.standard_normal(c).astype(np.float32)
        dn = (rng.random(c) < 0.5).astype(np.uint8)
        prio = None if step % 2 else (rng.random(c) * 4).astype(np.float32)
        if prio is not None and step % 4 == 0:
            prio[0] = -0.0
        o.add(c, st, nx, ac, rw, dn, prio=prio)
        g.add(c, dev(st), dev(nx), dev(ac), dev(rw), dev(dn),
              prio=None if prio is None else dev(prio))
        compare_trees(o, g, "ring n=%d step %d add %d" % (n, step, c))
        B = int(rng.integers(1, 200))
        if o.total > 0:
            u = rng.random(B, dtype=np.float32)
            ro = o.sample(u, beta=0.6, rows=True)
            rg = g.sample(dev(u), beta=0.6, rows=True)
            compare_sample(rg, ro, "ring n=%d step %d sample" % (n, step), rows=True)
        idx = rng.integers(-2, n + 2, B).astype(np.int64)
        td = (rng.standard_normal(B) * 2).astype(np.float32)
        o.update(idx, td)
        g.update(dev(idx), dev(td))
        compare_trees(o, g, "ring n=%d step %d update" % (n, step))


@pytest.mark.parametrize("n,D,strides", [(1 << 10, 8, (8, 9, 12, 37)), (1 << 10, 5, (5, 8, 13)),
                                          (1 << 20, 64, (72,))])
def test_padded_gather(n, D, strides):
    """per_sample_padded against the oracle: indices and rows bit for bit, the
    padding columns +0.0 (outputs start as NaN), actions as the stored bits,
    dones as f32, weights within 1e-6."""
    say("padded", n, D, strides)
    rng = np.random.default_rng(D)
    o = Oracle(n, D)
    g = _buf(n, D, max_batch=2048)
    st = rng.standard_normal((n, D)).astype(np.float32)
    nx = rng.standard_normal((n, D)).astype(np.float32)
    ac = rng.integers(0, 3, n).astype(np.uint32)
    ac[::97] = np.uint32(0xFFFFFFF0)
    rw = rng.standard_normal(n).astype(np.float32)
    dn = (rng.random(n) < 0.1).astype(np.uint8)
    dn[::131] = 7
    p0 = rng.random(n).astype(np.float32)
    o.add(n, st, nx, ac, rw, dn, prio=p0)
    g.add(n, dev(st), dev(nx), dev(ac), dev(rw), dev(dn), prio=dev(p0))
    for stride in strides:
        for B in (1, 333, 2048):
            u = rng.random(B, dtype=np.float32)
            ro = o.sample_padded(u, stride, beta=0.4)
            out = {"idx": dev(np.full(B, -1, np.int64)),
                   "w": dev(np.full(B, np.nan, np.float32)),
                   "states": dev(np.full((B, stride), np.nan, np.float32)),
                   "next_states": dev(np.full((B, stride), np.nan, np.float32)),
                   "actions": dev(np.full(B, -1, np.int32)),
                   "rewards": dev(np.full(B, np.nan, np.float32)),
                   "dones": dev(np.full(B, np.nan, np.float32))}
            rg = g.sample_padded(dev(u), stride, beta=0.4, out=out)
            what = "padded n=%d D=%d stride=%d B=%d" % (n, D, stride, B)
            assert_bits_equal(host(rg["idx"]), ro["idx"], what + " idx")
            compare_weights(host(rg["w"]), ro["w"], what + " w")
            for key in ("states", "next_states", "actions", "rewards", "dones"):
                assert_bits_equal(host(rg[key]), ro[key], what + " " + key)


@pytest.mark.parametrize("B", [1, 333, 20000])
def test_device_masses(B):
    """per_sample_philox against the oracle (masses from Philox4x64-10 words
    offset .. offset+B-1 on both sides): indices and rows bit for bit,
    weights within 1e-6; B = 20000 takes the one-lane-per-sample sampler."""
    say("philox masses", B)
    n, D = 1 << 12, 8
    rng = np.random.default_rng(B)
    o = Oracle(n, D)
    g = _buf(n, D, max_batch=32768)
    st = rng.standard_normal((n, D)).astype(np.float32)
    nx = rng.standard_normal((n, D)).astype(np.float32)
    ac = rng.integers(0, 3, n).astype(np.uint32)
    rw = rng.standard_normal(n).astype(np.float32)
    dn = (rng.random(n) < 0.1).astype(np.uint8)
    p0 = (rng.random(n) ** 0.6).astype(np.float32)
    o.add(n, st, nx, ac, rw, dn, prio=p0)
    g.add(n, dev(st), dev(nx), dev(ac), dev(rw), dev(dn), prio=dev(p0))
    for seed, off in ((0, 0), (7, 3), (2**63 + 5, 1 << 33), (2**64 - 1, 2**64 - 4 * B - 2)):
        ro = o.sample_philox(B, seed, off, beta=0.4, rows=True)
        rg = g.sample_philox(B, seed, off, beta=0.4, rows=True)
        compare_sample(rg, ro, "philox B=%d seed=%d off=%d" % (B, seed, off), rows=True)


@pytest.mark.parametrize("size,B", [(1, 5), (1000, 333), (4096, 70000), (3 << 11, 64)])
def test_uniform_sample(size, B):
    """per_sample_uniform against the oracle: slots ((word >> 32) * size) >> 32
    and their rows, bit for bit, over partly filled rings."""
    say("uniform", size, B)
    n, D = 1 << 13, 5
    rng = np.random.default_rng(size)
    o = Oracle(n, D)
    g = _buf(n, D, max_batch=1 << 17)
    st = rng.standard_normal((size, D)).astype(np.float32)
    nx = rng.standard_normal((size, D)).astype(np.float32)
    ac = rng.integers(0, 3, size).astype(np.uint32)
    rw = rng.standard_normal(size).astype(np.float32)
    dn = (rng.random(size) < 0.1).astype(np.uint8)
    o.add(size, st, nx, ac, rw, dn)
    g.add(size, dev(st), dev(nx), dev(ac), dev(rw), dev(dn))
    for seed, off in ((3, 0), (2**64 - 1, 12345)):
        ro = o.sample_uniform(B, seed, off, rows=True)
        rg = g.sample_uniform(B, seed, off, rows=True)
        what = "uniform size=%d B=%d seed=%d" % (size, B, seed)
        assert_bits_equal(host(rg["idx"]), ro["idx"], what + " idx")
        for key in ("states", "next_states", "actions", "rewards", "dones"):
            assert_bits_equal(host(rg[key]), ro[key], what + " " + key)


@pytest.mark.parametrize("n,size,D,B", [(1 << 12, 1 << 12, 0, 300), (1 << 16, 50000, 5, 20000),
                                        (1 << 21, 1 << 21, 0, 512)])
def test_rank_based(n, size, D, B):
    """Rank-based prioritisation against the oracle: the ranking (ties by
    slot), both rank-weight trees bit for bit, and samples (indices and rows
    bit for bit, weights within 1e-6); again after an update (ranking only)
    and after more intake (rank-weight trees rebuilt)."""
    say("rank", n, size, D, B)
    rng = np.random.default_rng(size)
    o = Oracle(n, D)
    g = _buf(n, D, max_batch=max(B, 4096))
    g.rank_attach()
    first = size - min(size // 3, 1000)

    def intake(c, p):
        if D:
            st = rng.standard_normal((c, D)).astype(np.float32)
            ac = rng.integers(0, 3, c).astype(np.uint32)
            rw = rng.standard_normal(c).astype(np.float32)
            dn = (rng.random(c) < 0.1).astype(np.uint8)
            o.add(c, st, st, ac, rw, dn, prio=p)
            g.add(c, dev(st), dev(st), dev(ac), dev(rw), dev(dn), prio=None if p is None else dev(p))
        else:
            o.add(c, prio=p)
            g.add(c, prio=None if p is None else dev(p))

    intake(first, (rng.integers(0, 64, first) / 16).astype(np.float32))  # ties and zeros

    def check(what):
        o.rank_refresh()
        g.rank_refresh()
        torch.cuda.synchronize()
        assert_bits_equal(host(g.rank_order()).view(np.uint32), o.rank_order().astype(np.uint32),
                          what + " order")
        rs, rm = g.rank_trees()
        assert_bits_equal(host(rs)[1:], o.rank_sum_tree()[1:], what + " rank sum tree")
        assert_bits_equal(host(rm)[1:], o.rank_min_tree()[1:], what + " rank min tree")
        u = rng.random(B, dtype=np.float32)
        ro = o.sample_rank(u, beta=0.4, rows=D > 0)
        rg = g.sample_rank(dev(u), beta=0.4, rows=D > 0)
        compare_sample(rg, ro, what + " sample", rows=D > 0)

    check("rank n=%d first" % n)
    idx = rng.integers(0, first, 2000).astype(np.int64)
    td = rng.standard_normal(2000).astype(np.float32)
    o.update(idx, td)
    g.update(dev(idx), dev(td))
    check("rank n=%d after update" % n)
    if size > first:
        intake(size - first, None)
        check("rank n=%d after intake" % n)


def test_intake_at_extreme_running_max():
    """Intake at the running max after that max was driven to 3e38: the
    interior subtrees of each run overflow to +inf, which the pairwise adds
    and the repeated doubling of the uniform-run repair must reach alike."""
    say("intake at 3e38")
    n = 1 << 13
    rng = np.random.default_rng(7)
    o = Oracle(n, 0)
    g = _buf(n)
    p0 = rng.random(n).astype(np.float32)
    o.add(n, prio=p0)
    g.add(n, prio=dev(p0))
    big = np.full(3, 3e38, np.float32)
    o.add(3, prio=big)
    g.add(3, prio=dev(big))
    for c in (1, 2, 500, 4093, 3000):
        o.add(c)
        g.add(c)
        compare_trees(o, g, "intake %d at 3e38" % c)


def test_partial_fill_and_empty():
    from sum_tree_sampling_amd import PerError
    n = 1 << 15
    g = _buf(n)
    o = Oracle(n)
    u = dev(np.array([0.5], np.float32))
    with pytest.raises(PerError) as e:
        g.sample(u)
    assert e.value.code == -3
    # empty batches are no-ops
    g.update(dev(np.zeros(0, np.int64)), dev(np.zeros(0, np.float32)))
    g.add(0)
    compare_trees(o, g, "empty")
    o.add(777)
    g.add(777)
    compare_trees(o, g, "partial")
    assert float(host(g.scalar("min"))[0]) == 1.0
    rng = np.random.default_rng(9)
    uu = rng.random(1000, dtype=np.float32)
    compare_sample(g.sample(dev(uu)), o.sample(uu), "partial sample")
    idx = np.arange(700, 900, dtype=np.int64)  # the tail is past size and skipped
    td = np.ones(200, np.float32)
    o.update(idx, td)
    g.update(dev(idx), dev(td))
    compare_trees(o, g, "partial update")


def test_scalars_and_errors():
    from sum_tree_sampling_amd import PerError
    n = 1 << 10
    g = _buf(n, max_batch=16)
    with pytest.raises(PerError):
        g.sample(dev(np.zeros(17, np.float32)))
    with pytest.raises(PerError):
        g.add(n + 1)
    g.add(n, prio=dev(np.full(n, 0.25, np.float32)))
    assert float(host(g.scalar("total"))[0]) == 256.0
    assert float(host(g.scalar("min"))[0]) == 0.25
    assert float(host(g.scalar("max_priority"))[0]) == 1.0


def test_time_next():
    """per_time_next: the next call's kernels (one or two launches) run between
    the caller's events and give the same trees and outputs as an untimed
    call; the request is dropped after that call."""
    from sum_tree_sampling_amd import per
    n, D = 1 << 20, 8  # 256 partitions: an update of 16384 entries is bucketed
    say("time_next", n)
    rng = np.random.default_rng(11)
    bufs = [_buf(n, D, max_batch=1 << 15) for _ in range(2)]
    p0 = (rng.random(n) ** 0.6).astype(np.float32)
    rows = [rng.standard_normal((n, D)).astype(np.float32) for _ in range(2)]
    ac = rng.integers(0, 3, n).astype(np.uint32)
    rw = rng.standard_normal(n).astype(np.float32)
    dn = (rng.random(n) < 0.1).astype(np.uint8)
    for g in bufs:
        g.add(n, dev(rows[0]), dev(rows[1]), dev(ac), dev(rw), dev(dn), prio=dev(p0))
    u = dev(rng.random(777, dtype=np.float32))
    small = (dev(rng.integers(0, n, 300).astype(np.int64)),
             dev(rng.standard_normal(300).astype(np.float32)))
    large = (dev(rng.integers(0, n, 16384).astype(np.int64)),   # bucketed: two launches
             dev(rng.standard_normal(16384).astype(np.float32)))
    ops = [("sample", lambda g: g.sample(u, beta=0.4, rows=True)),
           ("update", lambda g: g.update(*small)),
           ("bucketed update", lambda g: g.update(*large)),
           ("add", lambda g: g.add(100, dev(rows[0][:100]), dev(rows[1][:100]), dev(ac[:100]),
                                   dev(rw[:100]), dev(dn[:100])))]
    for what, op in ops:
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()  # torch creates an event when it is first recorded
        b.record()
        torch.cuda.synchronize()
        per.per_time_next(a, b)
        timed = op(bufs[0])
        plain = op(bufs[1])
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        assert 0.0 < ms < 100.0, "%s: span %.4f ms" % (what, ms)
        if isinstance(timed, dict):
            for k in timed:
                assert_bits_equal(host(timed[k]), host(plain[k]), what + " " + k)
        for t0, t1, tree in ((bufs[0].sum_tree(), bufs[1].sum_tree(), "sum"),
                             (bufs[0].min_tree(), bufs[1].min_tree(), "min")):
            assert_bits_equal(host(t0), host(t1), "%s %s tree" % (what, tree))
    # a request is dropped with the call that follows it, whatever it returns
    a = torch.cuda.Event(enable_timing=True)
    a.record()
    torch.cuda.synchronize()
    per.per_time_next(a, None)
    with pytest.raises(per.PerError):  # B past max_batch
        bufs[0].update(dev(np.zeros((1 << 15) + 1, np.int64)),
                       dev(np.zeros((1 << 15) + 1, np.float32)))
    c = torch.cuda.Event(enable_timing=True)
    c.record()
    bufs[0].update(*small)  # untimed: must not record the event again
    torch.cuda.synchronize()
    assert a.elapsed_time(c) >= 0.0  # a still holds its first record, before c
    for g in bufs:
        g.close()


def test_top_deeper_than_lds():
    """2^25 leaves: 2^13 partitions, so the levels above them are rebuilt by
    the one-block top kernel through global memory before sampling."""
    n = 1 << 25
    say("deep top", n)
    rng = np.random.default_rng(25)
    o = Oracle(n)
    g = _buf(n, max_batch=2048)
    p0 = rng.random(n).astype(np.float32)
    o.add(n, prio=p0)
    g.add(n, prio=dev(p0))
    compare_trees(o, g, "2^25 fill")
    for step in range(2):
        u = rng.random(2048, dtype=np.float32)
        for mode in ("1", "2", "3"):
            g.set_sample_lanes(LANES[mode])
            compare_sample(g.sample(dev(u)), o.sample(u), "2^25 mode " + mode)
        g.set_sample_lanes(0)
        idx = rng.integers(0, n, 2048).astype(np.int64)
        td = rng.standard_normal(2048).astype(np.float32)
        o.update(idx, td)
        g.update(dev(idx), dev(td))
        u = rng.random(100, dtype=np.float32)
        compare_sample(g.sample(dev(u)), o.sample(u), "2^25 after update %d" % step)
        compare_trees(o, g, "2^25 step %d" % step)


# ------------------------------------------------------------ large trees

@pytest.mark.parametrize("L", [23, 24])
def test_large_tree_writers(L):
    """Trees of 2^23 and 2^24 leaves (2^11 and 2^12 partitions): after every
    kind of writer launch -- intake with and without priorities, a wrapping
    intake, the scanned and the bucketed update, the fused update + intake --
    both trees match the oracle bit for bit, and the samplers match in every
    layout."""
    n = 1 << L
    say("stored top", L)
    rng = np.random.default_rng(100 + L)
    o = Oracle(n)
    g = _buf(n, max_batch=65536)
    k0 = n - 3000
    p0 = (rng.random(k0) ** 0.6).astype(np.float32)
    o.add(k0, prio=p0)
    g.add(k0, prio=dev(p0))

    def check(what):
        torch.cuda.synchronize()
        assert_bits_equal(host(g.sum_tree())[1:2 * n], o.sum_tree()[1:], what + " sum tree")
        assert_bits_equal(host(g.min_tree())[1:2 * n], o.min_tree()[1:], what + " min tree")

    def sample_all(what):
        for mode in ("1", "2", "3"):
            g.set_sample_lanes(LANES[mode])
            u = rng.random(3000, dtype=np.float32)
            u[:2] = [0.0, np.nextafter(np.float32(1), np.float32(0))]
            compare_sample(g.sample(dev(u), beta=0.4), o.sample(u, beta=0.4),
                           "%s mode %s" % (what, mode))
        g.set_sample_lanes(0)

    check("fill")
    sample_all("fill")
    o.add(2000)
    g.add(2000)                                   # at the running max
    check("intake at the running max")
    pr = (rng.random(5000) * 3).astype(np.float32)
    o.add(5000, prio=pr)
    g.add(5000, prio=dev(pr))                     # wraps past the end, given priorities
    check("wrapping intake")
    for B in (200, 8192, 65536):                  # scanned, then bucketed
        idx = rng.integers(0, n, B).astype(np.int64)
        idx[: B // 8] = idx[B // 8: B // 4]
        td = (rng.standard_normal(B) * 2).astype(np.float32)
        o.update(idx, td)
        g.update(dev(idx), dev(td))
        check("update B=%d" % B)
    idx = rng.integers(0, n, 300).astype(np.int64)
    td = rng.standard_normal(300).astype(np.float32)
    o.update(idx, td)
    o.add(700)
    g.update_add(dev(idx), dev(td), 700)
    check("update + intake")
    sample_all("after the writers")
    assert np.float32(host(g.scalar("total"))[0]) == np.float32(o.sum_tree()[1])
    assert np.float32(host(g.scalar("min"))[0]) == np.float32(o.min_tree()[1])


def test_bucketed_partition_pairs():
    """A 2^23-leaf tree (2^11 partitions of 4096 leaves) updated by batches of
    ~12000 entries, which the bucketed repair takes two partitions per wave:
    pairs whose buckets fit one wave together (with repeated slots and the
    two leaves on either side of the partition boundary), pairs that do not
    (repaired one after the other), a crowded partition beside a sparse one,
    a pair with one empty partition, and the first and last partitions.  Both
    trees and the running max match the oracle bit for bit after each of
    three calls in a row (counts and overflow list cleared between them)."""
    L, S = 23, 12
    n, span = 1 << L, 1 << S
    np_ = n >> S
    rng = np.random.default_rng(2323)
    o = Oracle(n)
    g = _buf(n, max_batch=16384)
    p0 = (rng.random(n) ** 0.6).astype(np.float32)
    o.add(n, prio=p0)
    g.add(n, prio=dev(p0))

    def leaves(part, k):
        off = rng.integers(0, span, k)
        off[k // 2: k // 2 + k // 4] = off[: k // 4]  # repeated slots
        return part * span + off

    for call in range(3):
        special = {
            10: 40, 11: 30,        # 70 together: one after the other
            20: 30, 21: 30,        # 64 together with the boundary leaves: one wave
            30: 100, 31: 10,       # crowded (overflow list) beside sparse
            40: 0, 41: 20,         # one empty partition
            0: 25, 1: 25,          # the first pair
            np_ - 2: 12, np_ - 1: 33,  # the last pair
        }
        base = rng.integers(0, n, 12000)
        base = base[~np.isin(base >> S, list(special))]
        r = base.size // 8
        base[:r] = base[r: 2 * r]  # repeated slots
        parts = [base]
        for part, k in special.items():
            if k:
                parts.append(leaves(part, k))
        # the two leaves on either side of a boundary, inside a one-wave pair
        parts.append(np.array([21 * span - 1, 21 * span, 21 * span - 1, 21 * span]))
        parts.append(np.array([0, n - 1, 0]))
        idx = np.concatenate(parts).astype(np.int64)
        rng.shuffle(idx)
        td = (rng.standard_normal(idx.size) * (1 + call)).astype(np.float32)
        say("bucketed pairs call", call, "B", idx.size)
        o.update(idx, td)
        g.update(dev(idx), dev(td))
        compare_trees(o, g, "bucketed pairs call %d" % call)


# ------------------------------------------------------------ graph mode

def _rows_np(rng, c, D):
    if D == 0:
        return ()
    return (rng.standard_normal((c, D)).astype(np.float32),
            rng.standard_normal((c, D)).astype(np.float32),
            rng.integers(0, 3, c).astype(np.uint32),
            rng.standard_normal(c).astype(np.float32),
            (rng.random(c) < 0.2).astype(np.uint8))


@pytest.mark.parametrize("n,D,B,c,prio,uniform,fused", [
    (1 << 12, 8, 256, 300, False, False, False),   # one partition; the ring wraps every few replays
    (1 << 16, 5, 1024, 3000, True, False, False),  # given priorities; scalar row copies
    (1 << 20, 0, 16384, 5000, False, False, False),  # bucketed update: the overflow parity flips too
    (1 << 13, 4, 500, 700, False, True, False),    # uniform sample over a ring still filling up
    (1 << 21, 0, 512, 400, False, False, True),    # the Ape-X shard step: sample, update + intake
    (1 << 16, 5, 1024, 3000, True, False, True),   # fused, given priorities
    (1 << 23, 0, 700, 400, False, False, True),    # 2^11 partitions, fused
    (1 << 24, 0, 65536, 5000, True, False, False),  # 2^12 partitions, bucketed, given priorities
])
def test_graph_replay(n, D, B, c, prio, uniform, fused):
    """Two whole steps (intake, sample, update) issued in graph mode, first
    eagerly, then captured once in a torch CUDA graph and replayed with fresh
    inputs each time: after every replay both steps' samples and the trees
    match the oracle taken through the same steps, while the ring moves (and
    wraps) on the device only.  Leaving graph mode hands the device's ring
    state back to the host, and eager calls then carry on from it."""
    say("graph replay", n, D, B, c, prio, uniform, fused)
    rng = np.random.default_rng(n + c)
    o = Oracle(n, D)
    g = _buf(n, D, max_batch=max(B, 256))
    k0 = n // 2 + 37
    r0 = _rows_np(rng, k0, D)
    p0 = (rng.random(k0) * 3).astype(np.float32)
    o.add(k0, *r0, prio=p0)
    g.add(k0, *[dev(x) for x in r0], prio=dev(p0))
    beta = 0.5
    seeds = [(11, 0), (12, 1 << 20)]  # per captured step: fixed at capture

    def inputs():
        return dict(rows=_rows_np(rng, c, D),
                    prio=(rng.random(c) * 5).astype(np.float32) if prio else None,
                    u=rng.random(B, dtype=np.float32),
                    td=(rng.standard_normal(B) * 2).astype(np.float32))

    first = [inputs(), inputs()]
    stat = []
    for k in range(2):
        x = first[k]
        stat.append(dict(rows=[dev(a) for a in x["rows"]],
                         prio=dev(x["prio"]) if prio else None,
                         u=dev(x["u"]), td=dev(x["td"]),
                         out=g._outs(B, not uniform, D > 0)))

    def refresh(xs):
        for k in range(2):
            s, x = stat[k], xs[k]
            for t, a in zip(s["rows"], x["rows"]):
                t.copy_(dev(a))
            if prio:
                s["prio"].copy_(dev(x["prio"]))
            s["u"].copy_(dev(x["u"]))
            s["td"].copy_(dev(x["td"]))

    def issue(k):
        # a step: intake, sample, update -- or, fused: sample, update + intake
        s = stat[k]
        if not fused:
            g.add(c, *s["rows"], prio=s["prio"])
        if uniform:
            g.sample_uniform(B, seeds[k][0], seeds[k][1], rows=D > 0, out=s["out"])
        else:
            g.sample(s["u"], beta=beta, weights=True, rows=D > 0, out=s["out"])
        if fused:
            g.update_add(s["out"]["idx"], s["td"], c, *s["rows"], prio=s["prio"])
        else:
            g.update(s["out"]["idx"], s["td"])

    def oracle_and_compare(xs, what):
        for k in range(2):
            x = xs[k]
            if not fused:
                o.add(c, *x["rows"], prio=x["prio"])
            if uniform:
                ro = o.sample_uniform(B, seeds[k][0], seeds[k][1], rows=D > 0)
            else:
                ro = o.sample(x["u"], beta=beta, weights=True, rows=D > 0)
            o.update(ro["idx"], x["td"])
            if fused:
                o.add(c, *x["rows"], prio=x["prio"])
            compare_sample(stat[k]["out"], ro, "%s step %d" % (what, k), rows=D > 0,
                           weights=not uniform)
        compare_trees(o, g, what, ring=False)

    g.graph_mode(True)
    refresh(first)
    issue(0)
    issue(1)
    oracle_and_compare(first, "graph mode eager")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        issue(0)
        issue(1)
    for r in range(4):
        xs = [inputs(), inputs()]
        refresh(xs)
        graph.replay()
        oracle_and_compare(xs, "replay %d" % r)
    g.graph_mode(False)
    assert g.size == o.size and g.cursor == o.cursor, (g.size, o.size, g.cursor, o.cursor)
    xs = [inputs(), inputs()]
    refresh(xs)
    issue(0)
    issue(1)
    oracle_and_compare(xs, "eager after graph mode")
    compare_trees(o, g, "eager after graph mode")
    del graph
    say("graph replay ok")


def test_graph_mode_replay_rule():
    """Leaving graph mode after calls that flip a slot parity an odd number
    of times is reported (PER_EINVAL) yet still hands back the ring state;
    entering twice or leaving twice is refused."""
    from sum_tree_sampling_amd import PerError
    n = 1 << 12
    o = Oracle(n)
    g = _buf(n)
    g.graph_mode(True)
    with pytest.raises(PerError) as e:
        g.graph_mode(True)
    assert e.value.code == -1
    o.add(100)
    g.add(100)  # one intake: the ring parity flips once
    with pytest.raises(PerError) as e:
        g.graph_mode(False)
    assert e.value.code == -1 and "odd number" in str(e.value)
    assert g.size == o.size == 100 and g.cursor == o.cursor == 100
    with pytest.raises(PerError) as e:
        g.graph_mode(False)
    assert e.value.code == -1
    compare_trees(o, g, "after the rule check")


@pytest.mark.parametrize("n,D,B,c,prio,fill", [
    (1 << 21, 0, 512, 400, False, 1 << 21),    # the Ape-X shard step
    (1 << 12, 8, 64, 300, False, 3000),        # one partition; the ring wraps inside it
    (1 << 16, 5, 1000, 3000, True, 40000),     # given priorities; scalar row copies
    (1 << 16, 4, 2000, 5000, False, 1 << 16),  # crowded partitions; the intake spans several
    (1 << 20, 0, 16384, 700, False, 1 << 20),  # bucketed batch: enqueued as the two calls
    (1 << 16, 0, 513, 300, False, 1 << 16),    # just past two batch entries per thread
    (1 << 16, 3, 1025, 200, False, 50000),     # just past four
])
def test_update_add(n, D, B, c, prio, fill):
    """per_update_add against the oracle's update followed by its intake,
    bit for bit: batches with repeats, skipped indices, NaN / Inf TD errors
    and slots the intake overwrites at once; the running max, the ring and
    the stored rows (through a sample) after every call."""
    say("update_add", n, D, B, c, prio, fill)
    rng = np.random.default_rng(n + B + c)
    o = Oracle(n, D)
    g = _buf(n, D, max_batch=max(B, 256))
    r0 = _rows_np(rng, fill, D)
    p0 = (rng.random(fill) * 2).astype(np.float32)
    o.add(fill, *r0, prio=p0)
    g.add(fill, *[dev(x) for x in r0], prio=dev(p0))
    for step in range(6):
        size, cur = o.size, o.cursor
        idx = rng.integers(0, size, B).astype(np.int64)
        k = B // 8
        idx[:k] = (cur + rng.integers(0, c, k)) % n          # slots the intake takes next
        idx[k:2 * k] = idx[2 * k:3 * k]                       # repeats: the last one wins
        idx[3 * k] = -1
        idx[3 * k + 1] = n + 5
        # next to the run the intake takes: its boundary siblings' leaves
        near = np.array([cur - 1, cur - 2, cur + c, cur + c + 1, cur - 37, cur + c + 100])
        idx[3 * k + 2:3 * k + 8] = near % n
        rng.shuffle(idx)
        td = (rng.standard_normal(B) * 2).astype(np.float32)
        td[rng.integers(0, B, 3)] = np.nan
        if step % 2:
            td[rng.integers(0, B, 2)] = np.inf
        if step == 4:
            td[rng.integers(0, B)] = 60.0  # the batch raises the running max the intake takes
        rows = _rows_np(rng, c, D)
        pr = (rng.random(c) * 8).astype(np.float32) if prio else None
        o.update(idx, td)
        o.add(c, *rows, prio=pr)
        g.update_add(dev(idx), dev(td), c, *[dev(x) for x in rows],
                     prio=None if pr is None else dev(pr))
        compare_trees(o, g, "update_add step %d" % step)
        if D:
            u = rng.random(200, dtype=np.float32)
            compare_sample(g.sample(dev(u), rows=True), o.sample(u, rows=True),
                           "update_add step %d sample" % step, rows=True)


@pytest.mark.parametrize("lo,c", [
    (1, 4094),     # all but the partition's first and last leaf
    (2047, 2),     # across the middle
    (100, 1),      # one leaf
    (4095, 1),     # the last leaf: left siblings only
    (0, 37),       # from the first leaf: right siblings only
    (1234, 777),
    (3000, 1096),  # up to the last leaf
])
def test_update_add_boundary_siblings(lo, c):
    """A fused update and intake at the running max whose batch repairs the
    nodes the intake's climb takes as its run's boundary siblings: entries
    under every such sibling, at every height and on both sides, some under
    the same sibling or at the same leaf, plus entries inside the run
    (overwritten by the intake) and in other partitions; trees bit for bit
    with the oracle's update then intake."""
    say("update_add boundary siblings", lo, c)
    n, span, part = 1 << 16, 1 << 12, 5
    rng = np.random.default_rng(lo * 7919 + c)
    o = Oracle(n, 0)
    g = _buf(n, 0, max_batch=512)
    p0 = (rng.random(n) * 2).astype(np.float32)
    o.add(n, prio=p0)
    g.add(n, prio=dev(p0))
    for step in range(3):
        # move the ring's cursor to the run's first slot
        shift = (part * span + lo - o.cursor) % n
        if shift:
            pr = (rng.random(shift) * 2).astype(np.float32)
            o.add(shift, prio=pr)
            g.add(shift, prio=dev(pr))
        assert o.cursor == part * span + lo
        a, b = lo, lo + c - 1  # the run's first and last offset in the partition
        picks = []
        for h in range(12):
            if (a >> h) & 1:  # left sibling of height h
                s0 = ((a >> h) - 1) << h
                picks += list(rng.integers(s0, s0 + (1 << h), 1 + (h % 3 == 1)))
            if not (b >> h) & 1:  # right sibling of height h
                s0 = ((b >> h) + 1) << h
                picks += list(rng.integers(s0, s0 + (1 << h), 1 + (h % 3 == 2)))
        picks += list(rng.integers(a, b + 1, 3))           # inside the run
        picks = [part * span + x for x in picks]
        picks += picks[:4]                                  # repeats: the last one wins
        picks += list(rng.integers(0, n, 40))               # other partitions
        idx = np.array(picks, dtype=np.int64)
        rng.shuffle(idx)
        td = (rng.standard_normal(len(idx)) * 2).astype(np.float32)
        if step == 1:
            td[rng.integers(0, len(idx), 2)] = np.nan
        o.update(idx, td)
        o.add(c)
        g.update_add(dev(idx), dev(td), c)
        compare_trees(o, g, "boundary siblings lo %d c %d step %d" % (lo, c, step))


@pytest.mark.parametrize("alpha,eps", [
    (0.6, 1e-6),
    (1e-5, 1e-6),
    (3.0, 0.5),     # large results: 1e30^3 leaves the f32 range
    (1.0, 0.0),     # |td| = 0 with eps 0: y = 0
    (0.25, 1e-30),
])
def test_priority_wide_range(alpha, eps):
    """Priorities of TD errors spanning the f32 range -- log-uniform
    magnitudes from 1e-30 to 1e30 of either sign, zeros, the smallest normal
    and subnormal f32, the largest f32, NaN and infinities -- each slot
    updated once, by a bucketed batch and by a scanned one, bit for bit with
    the oracle's f32 of the f64 pow: whichever route the device's power takes,
    its f32 is the same."""
    say("priority wide range", alpha, eps)
    n = 1 << 18
    rng = np.random.default_rng(int(alpha * 1000) + int(-np.log10(eps)) if eps else 7)
    o = Oracle(n, 0, alpha=alpha, eps=eps)
    g = _buf(n, 0, max_batch=n, alpha=alpha, eps=eps)
    p0 = (rng.random(n) * 2).astype(np.float32)
    o.add(n, prio=p0)
    g.add(n, prio=dev(p0))
    mag = 10.0 ** rng.uniform(-30, 30, n)
    td = (mag * np.where(rng.random(n) < 0.5, -1.0, 1.0)).astype(np.float32)
    special = np.array([0.0, -0.0, 1.17549435e-38, 1e-45, 3.4028235e38, -3.4028235e38,
                        np.nan, np.inf, -np.inf, 1.0, -1.0, 0.5], dtype=np.float32)
    td[rng.choice(n, special.size * 8, replace=False)] = np.tile(special, 8)
    idx = rng.permutation(n).astype(np.int64)
    for lo, hi in ((0, n - 2048), (n - 2048, n)):  # the bucketed path, then the scan path
        o.update(idx[lo:hi], td[lo:hi])
        g.update(dev(idx[lo:hi]), dev(td[lo:hi]))
        compare_trees(o, g, "priority wide range alpha %g eps %g, entries %d..%d" % (alpha, eps, lo, hi))


@pytest.mark.parametrize("alpha,eps,kind", [
    (0.6, 1e-6, "near ties"),      # several entries within a few ulps of the largest |td|
    (0.6, 1e-6, "no finite td"),   # only NaN and infinite TD errors
    (0.6, 0.0, "all zero"),        # eps 0, every |td| 0: every entry at the bound
    (1e-5, 1e-6, "small alpha"),
    (3.0, 0.5, "large alpha"),
])
def test_update_add_batch_max(alpha, eps, kind):
    """The priority a fused intake at the running max takes is the max of
    the whole batch's priorities, bit for bit with the oracle's update then
    intake: near ties at the largest |td|, batches without a finite TD
    error, zero errors with eps 0, and small and large alpha."""
    say("update_add batch max", alpha, eps, kind)
    n, B, c = 1 << 16, 1500, 300
    rng = np.random.default_rng(int(alpha * 1e6) + len(kind))
    o = Oracle(n, 0, alpha=alpha, eps=eps)
    g = _buf(n, 0, max_batch=2048, alpha=alpha, eps=eps)
    p0 = (rng.random(n) * 0.01).astype(np.float32)
    o.add(n, prio=p0)
    g.add(n, prio=dev(p0))
    for step in range(4):
        idx = rng.integers(0, n, B).astype(np.int64)
        td = (rng.standard_normal(B) * 2).astype(np.float32)
        if kind == "near ties":
            top = np.float32(7.5 + step)
            k = rng.choice(B, 12, replace=False)
            # the largest |td| twice, then values 1 to 10 ulps below it, either sign
            below = (top.view(np.uint32) - np.arange(1, 11, dtype=np.uint32)).view(np.float32)
            td[k] = np.concatenate([[top, -top], below * np.where(np.arange(10) % 2, 1, -1)])
        elif kind == "no finite td":
            td[:] = np.nan
            td[rng.integers(0, B, 5)] = np.inf if step % 2 else np.nan
        elif kind == "all zero":
            td[:] = 0.0
        o.update(idx, td)
        o.add(c)
        g.update_add(dev(idx), dev(td), c)
        compare_trees(o, g, "batch max %s step %d" % (kind, step))


@pytest.mark.parametrize("alpha", [0.6, 1.0, 0.05, 7.0, 20.0])
def test_update_add_batch_max_near_running_max(alpha):
    """A fused intake at the running max when the batch's largest priority
    lies just below, at or just above the running max m0 (relative gaps from
    2^-8 down to 2^-20, both sides of the margin within which the kernel
    raises the largest |td| to alpha instead of deciding from logarithms that
    it cannot exceed m0; alpha 20 lies beyond the logarithm test's range): the
    trees, the running max and the intake's priority bit for bit with the
    oracle's update then intake."""
    say("update_add batch max near m0", alpha)
    n, B, c, eps = 1 << 14, 600, 100, 1e-6
    rng = np.random.default_rng(int(alpha * 1000) + 7)
    o = Oracle(n, 0, alpha=alpha, eps=eps)
    g = _buf(n, 0, max_batch=1024, alpha=alpha, eps=eps)
    p0 = (rng.random(n) * 0.01).astype(np.float32)
    o.add(n, prio=p0)
    g.add(n, prio=dev(p0))
    gaps = [-2.0**-8, -2.0**-11, -2.0**-12, -2.0**-13, -2.0**-14, -2.0**-20, 0.0, 2.0**-20, -2.0**-12]
    for step in range(len(gaps) + 1):
        idx = rng.integers(0, n, B).astype(np.int64)
        td = (rng.random(B) * 0.5).astype(np.float32)
        if step == 0:
            td[0] = 3.0  # the running max rises to 3^alpha
        else:
            m = float(o.max_priority)
            y = (m * (1.0 + gaps[step - 1])) ** (1.0 / alpha) - eps
            td[rng.integers(0, B)] = np.float32(y) * (1 if step % 2 else -1)
        o.update(idx, td)
        o.add(c)
        g.update_add(dev(idx), dev(td), c)
        compare_trees(o, g, "batch max near m0, alpha %g step %d" % (alpha, step))


@pytest.mark.parametrize("beta", [0.0, 0.4, 0.7, 1.0, 1.5])
@pytest.mark.parametrize("spread", ["wide, tiny min", "wide", "narrow"])
def test_is_weights_wide_range(beta, spread):
    """IS weights against the oracle's f64 form (N P_i)^-beta / (N P_min)^-beta
    in each sampler layout (B = 512, 4096, 20480 on 2^16 leaves), with the
    sampled priorities spread over 2^-20 .. 2^20 (or 1/2 .. 2) and the
    minimum priority 2^-60 or the spread's own: within 1e-6 relative always,
    and within 3e-7 for beta <= 1, the bound of the sampler's f32 route
    there (the f64 power elsewhere)."""
    say("IS weights", beta, spread)
    n = 1 << 16
    rng = np.random.default_rng(int(beta * 10) + 100 * len(spread))
    lo, hi = (-1.0, 1.0) if spread == "narrow" else (-20.0, 20.0)
    p = np.exp2(rng.uniform(lo, hi, n)).astype(np.float32)
    if spread == "wide, tiny min":
        p[rng.integers(0, n)] = np.float32(2.0**-60)
    o = Oracle(n, 0)
    g = _buf(n, 0, max_batch=1 << 15)
    o.add(n, prio=p)
    g.add(n, prio=dev(p))
    for B in (512, 4096, 20480):
        u = rng.random(B, dtype=np.float32)
        ro = o.sample(u, beta=beta)
        rg = g.sample(dev(u), beta=beta)
        what = "IS weights beta %g %s B %d" % (beta, spread, B)
        compare_sample(rg, ro, what)
        if beta <= 1.0:
            got = host(rg["w"]).astype(np.float64)
            exp = np.asarray(ro["w"], np.float64)
            rel = np.abs(got - exp) / np.abs(exp)
            assert rel.max() <= 3e-7, (what, float(rel.max()))


# ------------------------------------------------------------ full-size large buffer

def test_large_16m_full_size():
    """2^24 leaves, 2 x [2^24 x 128] f32 rows, B = 65536 with the sampler's
    default plan, two steps.  The oracle (trees only) runs both steps first,
    so that the sampled slots are known before the rows exist; the fill then
    generates every row chunk once, checks the device storage of each chunk
    against it (all five fields) and keeps the generator's rows at the
    oracle's sampled slots.  The device's steps are then checked against
    those: both trees after every operation, all indices and weights, and
    all five gathered fields of every sampled row."""
    name = "large_16m"
    s = workloads.spec(name)
    n, B, D = s["capacity"], s["batch"], s["state_dim"]
    keys = ("states", "next_states", "actions", "rewards", "dones")
    say("large: oracle steps", n, B)
    o = Oracle(n)
    pr = workloads.initial_priorities(name)
    o.add(n, prio=pr)
    snap = [(o.sum_tree().copy(), o.min_tree().copy(), o.max_priority)]
    inp = workloads.StepInputs(name)
    steps = []
    for step in range(2):
        u = inp.u()
        ro = o.sample(u, beta=s["beta"])
        td = inp.td()
        o.update(ro["idx"], td)
        snap.append((o.sum_tree().copy(), o.min_tree().copy(), o.max_priority))
        steps.append((u, td, ro))
    o.close()

    say("large: filling", n, D)
    g = _buf(n, D, max_batch=B)
    expect = [{k: None for k in keys} for _ in steps]
    chunk = 1 << 20
    for lo in range(0, n, chunk):
        say("  fill rows [%d, %d)" % (lo, lo + chunk))
        r = workloads.rows(name, lo, chunk)
        g.add(chunk, dev(r["states"]), dev(r["next_states"]), dev(r["actions"]),
              dev(r["rewards"]), dev(r["dones"]), prio=dev(pr[lo:lo + chunk]))
        torch.cuda.synchronize()
        for k in keys:
            got = host(g.storage[k][lo:lo + chunk])
            if k == "actions":
                got = got.view(np.uint32)
            assert_bits_equal(got, r[k], "storage %s rows [%d, %d)" % (k, lo, lo + chunk))
        for st, (_, _, ro) in enumerate(steps):
            idx = ro["idx"]
            sel = np.nonzero((idx >= lo) & (idx < lo + chunk))[0]
            for k in keys:
                if expect[st][k] is None:
                    expect[st][k] = np.zeros((B,) + r[k].shape[1:], r[k].dtype)
                expect[st][k][sel] = r[k][idx[sel] - lo]
        del r

    def check_trees(sn, what):
        sm, mm, mp = sn
        torch.cuda.synchronize()
        assert_bits_equal(host(g.sum_tree())[1:2 * n], sm[1:], what + " sum tree")
        assert_bits_equal(host(g.min_tree())[1:2 * n], mm[1:], what + " min tree")
        got = host(g.scalar("max_priority"))[0]
        assert np.float32(got).view(np.uint32) == np.float32(mp).view(np.uint32), (what, got, mp)

    check_trees(snap[0], "large after fill")
    for step, (u, td, ro) in enumerate(steps):
        say("large step", step)
        rg = g.sample(dev(u), beta=s["beta"], rows=True)
        compare_sample(rg, ro, "large step %d" % step)
        for k in keys:
            got = host(rg[k])
            if k == "actions":
                got = got.view(np.uint32)
            assert_bits_equal(got, expect[step][k], "large step %d gathered %s" % (step, k))
        g.update(rg["idx"], dev(td))
        check_trees(snap[step + 1], "large step %d update" % step)
