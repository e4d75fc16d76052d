"""Shared helpers of the GPU parity tests: drive the HIP path and the oracle
with the same seeded inputs and compare what they produce."""
from __future__ import annotations

import sys

import numpy as np
import torch

import workloads
from oracle import Oracle

W_RTOL = 1e-6  # IS weights: relative tolerance; everything else is bit-exact


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a, dtype=None):
    a = np.ascontiguousarray(a)
    if dtype is not None:
        a = a.astype(dtype)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).cuda()


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def assert_bits_equal(got: np.ndarray, exp: np.ndarray, what: str):
    g = np.ascontiguousarray(got).reshape(-1)
    e = np.ascontiguousarray(exp).reshape(-1)
    assert g.size == e.size and g.itemsize == e.itemsize, (what, g.shape, e.shape)
    u = {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}[g.itemsize]
    bad = np.nonzero(g.view(u) != e.view(u))[0]
    if bad.size:
        raise AssertionError("%s: %d of %d elements differ; first %s: got %s expected %s" % (
            what, bad.size, g.size, bad[:8].tolist(), g[bad[:8]].tolist(), e[bad[:8]].tolist()))


def compare_trees(o: Oracle, g, what: str, ring: bool = True):
    """Both trees and the running max bit for bit; the host's ring state too
    unless ring is False (in graph mode it counts issued calls, not replays)."""
    n = o.capacity
    torch.cuda.synchronize()
    assert_bits_equal(host(g.sum_tree())[1:2 * n], o.sum_tree()[1:], what + " sum tree")
    assert_bits_equal(host(g.min_tree())[1:2 * n], o.min_tree()[1:], what + " min tree")
    if ring:
        assert g.size == o.size and g.cursor == o.cursor, (what, g.size, o.size, g.cursor,
                                                           o.cursor)
    mp = host(g.scalar("max_priority"))[0]
    assert np.float32(mp).view(np.uint32) == np.float32(o.max_priority).view(np.uint32), \
        (what, mp, o.max_priority)


def compare_weights(got, exp, what):
    got = np.asarray(got, np.float64)
    exp = np.asarray(exp, np.float64)
    err = np.abs(got - exp)
    ok = err <= W_RTOL * np.abs(exp)
    if not ok.all():
        i = np.nonzero(~ok)[0]
        raise AssertionError("%s: %d weights off; first %s got %s exp %s" % (
            what, i.size, i[:5].tolist(), got[i[:5]].tolist(), exp[i[:5]].tolist()))


def compare_sample(res_g, res_o, what, rows=False, weights=True):
    torch.cuda.synchronize()
    assert_bits_equal(host(res_g["idx"]), res_o["idx"], what + " idx")
    if weights:
        compare_weights(host(res_g["w"]), res_o["w"], what + " w")
    if rows:
        for k in ("states", "next_states", "rewards", "dones"):
            assert_bits_equal(host(res_g[k]), res_o[k], what + " " + k)
        assert_bits_equal(host(res_g["actions"]).view(np.uint32), res_o["actions"], what + " actions")


def fill(name: str, o: Oracle | None, g, capacity=None, chunk=1 << 20):
    """Bulk fill both sides with the workload's initial priorities and rows."""
    s = workloads.spec(name)
    n = capacity or s["capacity"]
    D = g.state_dim
    pr = workloads.initial_priorities(name, capacity=n)
    for lo in range(0, n, chunk):
        c = min(chunk, n - lo)
        if n >= (1 << 22):
            say("  fill %s rows [%d, %d)" % (name, lo, lo + c))
        p = None if pr is None else pr[lo:lo + c]
        if D > 0:
            r = workloads.rows(name, lo, c, state_dim=D, capacity=n)
            if o is not None:
                if o.state_dim > 0:
                    o.add(c, r["states"], r["next_states"], r["actions"], r["rewards"],
                          r["dones"], prio=p)
                else:
                    o.add(c, prio=p)
            g.add(c, dev(r["states"]), dev(r["next_states"]), dev(r["actions"]),
                  dev(r["rewards"]), dev(r["dones"]), prio=None if p is None else dev(p))
        else:
            if o is not None:
                o.add(c, prio=p)
            g.add(c, prio=None if p is None else dev(p))
    return pr
