"""Pins that tie the CPU oracle to facts fixed by the pages and by mathematics.

Each pin_* function takes a loaded oracle library (so that the same checks can
be run against deliberately broken builds of the oracle) and raises
AssertionError when the oracle disagrees.  None of them calls the oracle to
produce its own expectation: expectations come from a hand-worked fixture,
from closed forms, from brute force over f64 cumulative sums, from a full
level-by-level rebuild in numpy, from high-precision decimal arithmetic, or
from a chi-square test.

Pages (by title):
  [Tree]  "Putting prioritized replay's segment tree on a GPU"
  [PER]   "GPU-Resident Prioritized Experience Replay"
"""
from __future__ import annotations

import decimal
import json
import math
import os

import numpy as np

import workloads
from oracle import Oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
ALPHA, EPS = workloads.ALPHA, workloads.EPS


# ---------------------------------------------------------------- helpers

def rebuild(leaves: np.ndarray):
    """Full level-by-level rebuild of both trees from their leaves
    ([Tree], "Second Port: Make the Update GPU-Shaped", step 2)."""
    n = leaves.size
    s = np.zeros(2 * n, np.float32)
    m = np.full(2 * n, np.inf, np.float32)
    s[n:] = leaves
    m[n:] = leaves
    width = n // 2
    while width >= 1:
        lo, hi = width, 2 * width
        s[lo:hi] = s[2 * lo:2 * hi:2] + s[2 * lo + 1:2 * hi:2]
        m[lo:hi] = np.minimum(m[2 * lo:2 * hi:2], m[2 * lo + 1:2 * hi:2])
        width //= 2
    return s, m


def rebuild_with_empty(leaves: np.ndarray, written: np.ndarray):
    """Rebuild where unwritten slots hold the neutral elements (0 / +inf)."""
    n = leaves.size
    sl = np.where(written, leaves, np.float32(0)).astype(np.float32)
    s, _ = rebuild(sl)
    ml = np.where(written, leaves, np.float32(np.inf)).astype(np.float32)
    _, m = rebuild(ml)
    return s, m


def assert_tree_is_rebuild(o: Oracle, written=None):
    s, m = o.sum_tree(), o.min_tree()
    n = o.capacity
    leaves = s[n:]
    if written is None:
        rs, rm = rebuild(leaves)
    else:
        rs, rm = rebuild_with_empty(leaves, written)
    assert np.array_equal(s[1:].view(np.uint32), rs[1:].view(np.uint32)), \
        "sum tree differs from the level-by-level rebuild of its leaves"
    assert np.array_equal(m[1:].view(np.uint32), rm[1:].view(np.uint32)), \
        "min tree differs from the level-by-level rebuild of its leaves"


def brute_index(leaves: np.ndarray, m: np.ndarray) -> np.ndarray:
    """Smallest j with C_j > m, C the f64 inclusive cumulative sum: proportional
    sampling written out directly ([Tree], "Sampling Is a Descent")."""
    c = np.cumsum(leaves.astype(np.float64))
    return np.searchsorted(c, m.astype(np.float64), side="right")


def f32_nearest_decimal(v: decimal.Decimal):
    """Nearest f32 to the exact value v > 0, and the distance of v to the
    nearest f32 rounding midpoint relative to v."""
    f = np.float32(float(v))
    cands = [np.nextafter(f, np.float32(0)), f, np.nextafter(f, np.float32(np.inf))]
    best = min(cands, key=lambda c: abs(decimal.Decimal(float(c)) - v))
    lo = np.nextafter(best, np.float32(0))
    hi = np.nextafter(best, np.float32(np.inf))
    mids = [(decimal.Decimal(float(best)) + decimal.Decimal(float(x))) / 2 for x in (lo, hi)]
    dist = min(abs(v - mm) for mm in mids) / v
    return best, dist


def exact_priority(td: float) -> decimal.Decimal:
    """(|td| + eps)^alpha with the sum rounded to f64 and the power exact to
    60 digits; alpha and eps are the f64 values the library receives."""
    with decimal.localcontext() as ctx:
        ctx.prec = 60
        s = decimal.Decimal(abs(float(td)) + EPS)  # the f64 sum, converted exactly
        return (decimal.Decimal(ALPHA) * s.ln()).exp()


# ---------------------------------------------------------------- pins

def pin_golden_hand_tree(lib):
    """Hand-worked 8-leaf and 4-leaf examples (tests/golden/hand_tree.json)."""
    with open(os.path.join(GOLDEN, "hand_tree.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        leaves = np.array(case["leaves"], np.float32)
        n = leaves.size
        o = Oracle(n, lib=lib)
        o.add(n, prio=leaves)
        s, m = o.sum_tree(), o.min_tree()
        assert s[1:].tolist() == case["sum_tree"][1:], case["name"]
        mt = [float("inf") if x == "inf" else x for x in case["min_tree"]]
        assert m[1:].tolist() == mt[1:], case["name"]
        u = np.array(case["masses"], np.float64) / float(case["total"])
        res = o.sample(u.astype(np.float32), beta=case["beta"])
        assert res["idx"].tolist() == case["expected_idx"], case["name"]
        exp_w = np.array(case["expected_w"], np.float64)
        assert np.allclose(res["w"], exp_w, rtol=1e-6, atol=0), case["name"]
        o.close()


def pin_a_invariant(lib):
    """P-a: after intake, wrap, updates with duplicates, invalid indices and
    NaN/Inf, both trees equal the full rebuild of their leaves."""
    rng = np.random.default_rng(11)
    n = 256
    o = Oracle(n, lib=lib)
    written = np.zeros(n, bool)
    cur = 0
    for step in range(30):
        c = int(rng.integers(1, 40))
        prio = None if step % 3 == 0 else rng.random(c).astype(np.float32) * 3
        o.add(c, prio=prio)
        written[(cur + np.arange(c)) % n] = True
        cur = (cur + c) % n
        assert_tree_is_rebuild(o, written)
        B = int(rng.integers(1, 50))
        idx = rng.integers(-3, n + 3, B)
        td = rng.standard_normal(B).astype(np.float32)
        td[rng.random(B) < 0.05] = np.nan
        td[rng.random(B) < 0.05] = np.inf
        o.update(idx, td)
        assert_tree_is_rebuild(o, written)
    o.close()


def pin_b_root_bound(lib):
    """P-b: |total - sum_f64(leaves)| <= gamma_L * sum, and the min root is the
    min over written leaves, exactly."""
    pr = workloads.initial_priorities("tiny_1k")
    n = pr.size
    o = Oracle(n, lib=lib)
    o.add(n, prio=pr)
    L = int(math.log2(n))
    S = math.fsum(float(x) for x in pr)
    u = L * 2.0 ** -24
    gamma = u / (1 - u)
    assert abs(float(o.total) - S) <= gamma * S, (o.total, S)
    assert o.min == pr.min()
    # partially filled: only written slots count for the min
    o2 = Oracle(n, lib=lib)
    o2.add(100, prio=pr[:100] + 5)
    assert o2.min == (pr[:100] + 5).min()
    assert abs(float(o2.total) - math.fsum(float(x) for x in (pr[:100] + 5))) <= \
        gamma * math.fsum(float(x) for x in (pr[:100] + 5))
    o.close()
    o2.close()


def pin_c_update_equivalence(lib):
    """P-c: sequential per-element walks == final leaves by "last batch position
    wins" + full rebuild, on duplicate-heavy batches with skipped indices."""
    rng = np.random.default_rng(12)
    n = 512
    base = (rng.random(n) + 0.1).astype(np.float32)
    o = Oracle(n, lib=lib)
    o.add(n - 37, prio=base[:n - 37])  # size = n - 37: indices >= size are skipped
    size = n - 37
    leaves = np.zeros(n, np.float32)
    leaves[:size] = base[:size]
    maxp = max(1.0, float(base[:size].max()))
    for step in range(10):
        B = 300
        distinct = rng.choice(n + 8, size=150, replace=False) - 4
        idx = np.concatenate([distinct, rng.choice(distinct, 150)])
        rng.shuffle(idx)
        idx[:3] = [size, size - 1, -1]
        td = rng.standard_normal(B).astype(np.float32)
        o.update(idx, td)
        final = {}
        for b in range(B):
            if 0 <= idx[b] < size:
                final[int(idx[b])] = b
        for slot, b in final.items():
            leaves[slot] = np.float32(math.pow(abs(float(td[b])) + EPS, ALPHA))
        for b in range(B):
            if 0 <= idx[b] < size:
                maxp = max(maxp, float(np.float32(math.pow(abs(float(td[b])) + EPS, ALPHA))))
        written = np.arange(n) < size
        rs, rm = rebuild_with_empty(leaves, written)
        assert np.array_equal(o.sum_tree()[1:].view(np.uint32), rs[1:].view(np.uint32))
        assert np.array_equal(o.min_tree()[1:].view(np.uint32), rm[1:].view(np.uint32))
        assert o.max_priority == np.float32(maxp)
    o.close()


def _dyadic_tree(rng, n):
    """Leaves k/256 (k in [0,255], many zeros) plus a last leaf that makes the
    total a power of two, so that every f32 sum and difference is exact."""
    p = rng.integers(0, 256, n).astype(np.float64) / 256.0
    p[rng.random(n) < 0.2] = 0.0
    S = p[:-1].sum()
    T = 2.0 ** math.ceil(math.log2(S + 1))
    p[-1] = T - S
    return p.astype(np.float32), T


def pin_d_dyadic_exact(lib):
    """P-d: with dyadic priorities every f32 operation of the descent is exact,
    so it must equal searchsorted(cumsum_f64, m, 'right') index for index,
    including masses placed exactly on cumulative boundaries."""
    rng = np.random.default_rng(13)
    n = 1024
    p, T = _dyadic_tree(rng, n)
    o = Oracle(n, lib=lib)
    o.add(n, prio=p)
    assert float(o.total) == T
    u = rng.random(20000, dtype=np.float32)
    m = (u * np.float32(T)).astype(np.float32)
    got = o.sample(u, weights=False)["idx"]
    assert np.array_equal(got, brute_index(p, m))
    c = np.cumsum(p.astype(np.float64))
    b = c[c < T]
    ub = (b / T).astype(np.float32)
    assert np.array_equal(ub.astype(np.float64) * T, b)  # boundaries are exact masses
    got = o.sample(ub, weights=False)["idx"]
    exp = brute_index(p, b)
    assert np.array_equal(got, exp)
    assert np.all(p[got] > 0), "a zero-priority leaf was sampled"
    o.close()


def pin_e_uniform_closed_form(lib):
    """P-e: all priorities 1 -> total = n exactly, idx = floor(u*n) and every
    IS weight is exactly 1."""
    n = 1024
    o = Oracle(n, lib=lib)
    o.add(n)  # every leaf at the initial running max 1.0
    assert float(o.total) == n and float(o.min) == 1.0
    rng = np.random.default_rng(14)
    u = rng.random(20000, dtype=np.float32)
    res = o.sample(u, beta=0.4)
    assert np.array_equal(res["idx"], np.floor(u.astype(np.float64) * n).astype(np.int64))
    assert np.all(res["w"] == 1.0)
    o.close()


def pin_f_brute_force_band(lib):
    """P-f: non-dyadic priorities: descent == f64-cumsum brute force except
    for masses within (L+1) ulp(total) of a cumulative boundary."""
    pr = workloads.initial_priorities("tiny_1k")
    n = pr.size
    o = Oracle(n, lib=lib)
    o.add(n, prio=pr)
    T = np.float32(o.total)
    rng = np.random.default_rng(15)
    u = rng.random(200000, dtype=np.float32)
    m = (u * T).astype(np.float32)
    got = o.sample(u, weights=False)["idx"]
    exp = brute_index(pr, m)
    c = np.cumsum(pr.astype(np.float64))
    band = (int(math.log2(n)) + 1) * float(np.spacing(T))
    j = np.searchsorted(c, m.astype(np.float64))
    near = np.zeros(m.size, bool)
    for dj in (-1, 0, 1):
        jj = np.clip(j + dj, 0, n - 1)
        near |= np.abs(c[jj] - m.astype(np.float64)) <= band
    bad = (got != exp) & ~near
    assert not bad.any(), "descent disagrees with brute force away from boundaries"
    assert (got != exp).sum() <= 5
    o.close()


def pin_g_chi_square(lib):
    """P-g: sampled counts match M*p_i/total (chi-square, fixed seed, p >= 1e-3);
    with 10% exact zeros no zero-priority leaf is ever returned."""
    from scipy import stats
    pr = workloads.initial_priorities("tiny_1k")
    n = pr.size
    o = Oracle(n, lib=lib)
    o.add(n, prio=pr)
    rng = np.random.default_rng(16)
    M = 1 << 20
    u = rng.random(M, dtype=np.float32)
    idx = o.sample(u, weights=False)["idx"]
    counts = np.bincount(idx, minlength=n)
    exp = M * pr.astype(np.float64) / pr.astype(np.float64).sum()
    assert exp.min() >= 5
    _, pval = stats.chisquare(counts, exp)
    assert pval >= 1e-3, pval
    o.close()
    # lognormal(0,3) with 10% zeros (the collision workload's recipe, small n)
    p = workloads.initial_priorities("collision_stress_2m", capacity=1 << 14)
    o = Oracle(1 << 14, lib=lib)
    o.add(1 << 14, prio=p)
    u = rng.random(200000, dtype=np.float32)
    u[:1000] = np.float32(1) - np.float32(2.0 ** -24) * rng.integers(1, 64, 1000).astype(np.float32)
    u[1000:2000] = np.float32(0)
    idx = o.sample(u, weights=False)["idx"]
    assert np.all(p[idx] > 0), "a zero-priority leaf was sampled"
    o.close()
    # Four leaves [x, y, z, 0] whose rounded sums let the largest mass reach the
    # zero right child; the walk must still end on a positive leaf.
    top = np.array([np.nextafter(np.float32(1), np.float32(0)),
                    np.float32(1) - np.float32(2.0 ** -23)], np.float32)
    for k in range(1500):
        x, y, z = (np.float32(10.0 ** rng.uniform(-3, 3)) for _ in range(3))
        leaves4 = np.array([x, y, z, 0], np.float32)
        o = Oracle(4, lib=lib)
        o.add(4, prio=leaves4)
        idx = o.sample(top, weights=False)["idx"]
        assert np.all(leaves4[idx] > 0), ("zero leaf sampled", leaves4)
        o.close()


def pin_h_is_weights(lib):
    """P-h: in real arithmetic w_i = (p_min / p_i)^beta: the weights must agree
    with that cancelled form within f32 rounding, equal 1 at the min-priority
    leaf and never exceed 1; w = 0 when the min priority is 0."""
    pr = workloads.initial_priorities("tiny_1k")
    n = pr.size
    o = Oracle(n, lib=lib)
    o.add(n, prio=pr)
    rng = np.random.default_rng(17)
    u = rng.random(5000, dtype=np.float32)
    for beta in (0.4, 1.0):
        res = o.sample(u, beta=beta)
        p = pr[res["idx"]].astype(np.float64)
        closed = (float(pr.min()) / p) ** beta
        assert np.all(np.abs(res["w"] - closed) <= 2.0 ** -23 * closed), beta
        assert np.all(res["w"] <= 1.0)
    j = int(np.argmin(pr))
    c = np.cumsum(pr.astype(np.float64))
    lo = c[j - 1] if j > 0 else 0.0
    um = np.float32((lo + pr[j] / 2) / float(o.total))
    res = o.sample(np.array([um], np.float32), beta=0.4)
    assert res["idx"][0] == j and res["w"][0] == 1.0
    o.close()
    z = pr.copy()
    z[5] = 0
    o = Oracle(n, lib=lib)
    o.add(n, prio=z)
    res = o.sample(u[:100], beta=0.4)
    assert np.all(res["w"] == 0.0)
    o.close()


def pin_i_gather(lib):
    """P-i: gathered rows are byte-identical to the stored rows at the sampled
    slots (storage is the ring layout of [PER], "Architecture")."""
    n, D = 1024, 8
    r = workloads.rows("tiny_1k", 0, n)
    pr = workloads.initial_priorities("tiny_1k")
    o = Oracle(n, D, lib=lib)
    o.add(n, r["states"], r["next_states"], r["actions"], r["rewards"], r["dones"], prio=pr)
    rng = np.random.default_rng(18)
    u = rng.random(777, dtype=np.float32)
    res = o.sample(u, rows=True)
    i = res["idx"]
    for key in ("states", "next_states", "actions", "rewards", "dones"):
        assert np.array_equal(res[key].view(np.uint8), r[key][i].view(np.uint8)), key
    o.close()


def pin_j_intake(lib):
    """P-j: ring intake ([PER], "Experience Insertion"): slots cursor..cursor+c-1
    (mod n) get the running max (or the given priorities), cursor and size
    wrap/saturate, the running max is monotone and equals the max written."""
    n = 64
    o = Oracle(n, lib=lib)
    assert o.max_priority == 1.0 and o.size == 0
    o.add(40)
    assert o.size == 40 and o.cursor == 40
    assert np.all(o.sum_tree()[n:n + 40] == 1.0) and np.all(o.sum_tree()[n + 40:] == 0)
    o.add(10, prio=np.full(10, 2.5, np.float32))
    assert o.max_priority == 2.5 and o.cursor == 50
    o.update(np.array([3]), np.array([100.0], np.float32))
    big = np.float32(math.pow(100.0 + EPS, ALPHA))
    assert o.max_priority == big
    o.add(30)  # wraps: slots 50..63 and 0..15
    leaves = o.sum_tree()[n:]
    assert o.cursor == 16 and o.size == 64
    assert np.all(leaves[50:] == big) and np.all(leaves[:16] == big)
    assert np.all(leaves[40:50] == 2.5) and np.all(leaves[16:40] == 1.0)
    o.add(64, prio=np.full(64, 0.5, np.float32))
    assert o.cursor == 16 and o.max_priority == big
    assert np.all(o.sum_tree()[n:] == 0.5)
    # a given -0.0 priority is stored as +0.0 (no negative zero in either tree)
    o.add(2, prio=np.array([-0.0, 0.0], np.float32))
    assert o.sum_tree()[n + 16].view(np.uint32) == 0
    assert o.min_tree()[n + 16].view(np.uint32) == 0 and o.min_tree()[1].view(np.uint32) == 0
    o.close()


def pin_k_priority_decimal(lib):
    """P-k: leaf priorities equal the f32 nearest to (|td| + eps)^alpha computed
    to 60 digits ([PER], "Priority update" and "Error Handling & Fallback"):
    NaN gives eps^alpha, +/-Inf the running max at batch start."""
    rng = np.random.default_rng(19)
    n = 4096
    o = Oracle(n, lib=lib)
    o.add(n, prio=np.full(n, 0.25, np.float32))
    td = np.concatenate([rng.standard_normal(3000), rng.laplace(0, 1, 1000) * 30,
                         [0.0, -0.0, 1e-30, 1e30, 3e38]]).astype(np.float32)
    idx = np.arange(td.size)
    o.update(idx, td)
    leaves = o.sum_tree()[n:]
    ambiguous = 0
    for k, t in enumerate(td):
        v = exact_priority(float(t))
        best, dist = f32_nearest_decimal(v)
        if dist < 2.0 ** -50:
            ambiguous += 1
            continue
        assert leaves[k].view(np.uint32) == best.view(np.uint32), (k, t, leaves[k], best)
    assert ambiguous <= 2
    m0 = o.max_priority
    o.update(np.array([7, 8, 9]), np.array([np.nan, np.inf, -np.inf], np.float32))
    leaves = o.sum_tree()[n:]
    best, _ = f32_nearest_decimal(exact_priority(0.0))
    assert leaves[7] == best
    assert leaves[8] == m0 and leaves[9] == m0
    assert o.max_priority == m0
    o.close()
    # Inf takes the max at batch start, not the max raised earlier in the batch.
    o = Oracle(8, lib=lib)
    o.add(8, prio=np.full(8, 0.5, np.float32))
    o.update(np.array([0, 1]), np.array([1e3, np.inf], np.float32))
    big, _ = f32_nearest_decimal(exact_priority(1e3))
    leaves = o.sum_tree()[8:]
    assert leaves[0] == big and leaves[1] == 1.0 and o.max_priority == big
    o.close()


def pin_l_padded_gather(lib):
    """P-l: the direct-to-trainer gather ("True Single-Graph Implementation
    Plan", Tasks 2 and 3) writes each stored state row into the first D
    columns of a destination row of out_stride floats and exactly +0.0 after
    them, actions as the stored 32 bits read as i32, rewards as stored and
    dones as the stored byte's value in f32; its indices are those of the
    plain sample for the same masses.  out_stride < D is refused."""
    n, D = 1024, 8
    r = workloads.rows("tiny_1k", 0, n)
    pr = workloads.initial_priorities("tiny_1k")
    acts = r["actions"].copy()
    acts[::97] = np.uint32(0xFFFFFFF0)  # high bit set: must come back as the same bits
    dones = r["dones"].copy()
    dones[::131] = 7  # a byte other than 0 / 1 keeps its value
    o = Oracle(n, D, lib=lib)
    o.add(n, r["states"], r["next_states"], acts, r["rewards"], dones, prio=pr)
    u = np.random.default_rng(21).random(500, dtype=np.float32)
    plain = o.sample(u, rows=False)
    for stride in (8, 9, 12, 37):
        res = o.sample_padded(u, stride)
        i = res["idx"]
        assert np.array_equal(i, plain["idx"])
        assert np.array_equal(res["w"].view(np.uint32), plain["w"].view(np.uint32))
        for key, src in (("states", r["states"]), ("next_states", r["next_states"])):
            out = res[key]
            assert out.shape == (500, stride)
            assert np.array_equal(out[:, :D].view(np.uint32), src[i].view(np.uint32)), key
            assert np.all(out[:, D:].view(np.uint32) == 0), key
        assert np.array_equal(res["actions"].view(np.uint32), acts[i])
        assert np.array_equal(res["rewards"].view(np.uint32), r["rewards"][i].view(np.uint32))
        assert np.array_equal(res["dones"], dones[i].astype(np.float32))
    try:
        o.sample_padded(u, D - 1)
    except ValueError:
        pass
    else:
        raise AssertionError("out_stride < state_dim accepted")
    o.close()


def _numpy_stream(seed, j0, count):
    """Words j0 .. j0+count-1 of a seed's stream from numpy's own Philox4x64-10
    (numpy increments its 256-bit counter before each block, so a counter one
    below block j0 // 4 makes its first block that one)."""
    M = 2**64 - 1
    blk = j0 // 4
    ctr = [M, M, M, M] if blk == 0 else [blk - 1, 0, 0, 0]
    g = np.random.Philox(key=np.array([seed, 0], np.uint64), counter=np.array(ctr, np.uint64))
    words = g.random_raw(count + j0 % 4 + 4)
    return [int(x) for x in words[j0 % 4:j0 % 4 + count]]


def pin_m_device_masses(lib):
    """P-m: the device-side generator ("GPU-Resident Prioritized Experience
    Replay", section "Sampling Kernels": masses and uniform indices come from
    a generator on the GPU) is Philox4x64-10 (Salmon et al., SC 2011): its
    words equal numpy's independent Philox4x64-10 implementation; the
    sample with generated masses equals the plain sample given the same
    masses; uniform indices are the multiply-shift of the word's high half
    into [0, size) and pass a chi-square test."""
    o = Oracle(1024, 8, lib=lib)
    for seed, j0 in ((0, 0), (1, 5), (12345, 1 << 20), (2**64 - 1, 3), (77, (1 << 40) + 2)):
        ref = _numpy_stream(seed, j0, 11)
        got = [o.stream_word(seed, j0 + k) for k in range(11)]
        assert got == ref, (seed, j0)
    r = workloads.rows("tiny_1k", 0, 1024)
    pr = workloads.initial_priorities("tiny_1k")
    o.add(1024, r["states"], r["next_states"], r["actions"], r["rewards"], r["dones"], prio=pr)
    seed, off, B = 99, 4097, 777
    words = _numpy_stream(seed, off, B)
    u = np.array([(x >> 40) * 2.0**-24 for x in words], np.float32)
    assert np.all(u >= 0) and np.all(u < 1)
    a = o.sample(u, beta=0.4, rows=True)
    b = o.sample_philox(B, seed, off, beta=0.4, rows=True)
    for key in ("idx", "w", "states", "next_states", "actions", "rewards", "dones"):
        assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), key
    o.close()
    # uniform indices over a size that is not a power of two
    o = Oracle(1024, lib=lib)
    o.add(1000)
    B = 1 << 18
    res = o.sample_uniform(B, 5, 0)["idx"]
    ref = [((x >> 32) * 1000) >> 32 for x in _numpy_stream(5, 0, 64)]
    assert res[:64].tolist() == ref
    assert res.min() >= 0 and res.max() < 1000
    counts = np.bincount(res, minlength=1000)
    chi2 = float(((counts - B / 1000) ** 2 / (B / 1000)).sum())
    import scipy.stats
    assert scipy.stats.chi2.sf(chi2, 999) > 1e-3, chi2
    o.close()


def pin_n_rank_based(lib):
    """P-n: rank-based prioritisation ("GPU-Resident Prioritized Experience
    Replay", section "Sampling Kernels", rank-based): the order is the filled
    slots by descending priority with ties by ascending slot (numpy lexsort);
    the rank weights are f32((r+1)^-alpha) (numpy f64 power) under a tree
    equal to the rebuild of its leaves; with alpha = 0 every rank is equally
    likely and sample == order[floor(u * size)]; the IS weights equal
    (rank / size)^(alpha * beta) up to f32 rounding; rank frequencies follow
    r^-alpha (chi-square)."""
    n = 1024
    rng = np.random.default_rng(31)
    p = rng.integers(0, 50, 900).astype(np.float32) / 8  # many ties and zeros
    for alpha in (0.7, 0.0):
        o = Oracle(n, alpha=alpha, lib=lib)
        o.add(900, prio=p)
        o.rank_refresh()
        order = o.rank_order()
        ref = np.lexsort((np.arange(900), -p.astype(np.float64)))
        assert np.array_equal(order, ref)
        rs, rm = o.rank_sum_tree(), o.rank_min_tree()
        w = np.zeros(n, np.float32)
        w[:900] = (np.arange(1, 901, dtype=np.float64) ** -alpha).astype(np.float32)
        assert np.array_equal(rs[n:].view(np.uint32), w.view(np.uint32))
        es, em = rebuild_with_empty(w, np.arange(n) < 900)
        assert np.array_equal(rs[1:].view(np.uint32), es[1:].view(np.uint32))
        assert np.array_equal(rm[1:].view(np.uint32), em[1:].view(np.uint32))
        if alpha == 0.0:
            o.close()
            continue
        u = rng.random(20000, dtype=np.float32)
        res = o.sample_rank(u, beta=0.5)
        rank = np.argsort(order)[res["idx"]] + 1  # 1-based rank of each sampled slot
        expw = (rank / 900.0) ** (alpha * 0.5)
        assert np.allclose(res["w"], expw, rtol=1e-6, atol=0)
        M = 1 << 18
        res = o.sample_rank(rng.random(M, dtype=np.float32), weights=False)
        counts = np.bincount(np.argsort(order)[res["idx"]], minlength=900).astype(np.float64)
        prob = np.arange(1, 901, dtype=np.float64) ** -alpha
        expc = M * prob / prob.sum()
        keep = expc >= 5
        chi2 = float((((counts - expc) ** 2) / expc)[keep].sum())
        import scipy.stats
        assert scipy.stats.chi2.sf(chi2, int(keep.sum()) - 1) > 1e-3, chi2
        o.close()
    # alpha = 0 over a full power-of-two ring: uniform over ranks, exactly
    o = Oracle(n, alpha=0.0, lib=lib)
    o.add(n, prio=rng.random(n).astype(np.float32))
    o.rank_refresh()
    u = (rng.integers(0, 1 << 20, 5000) / float(1 << 20)).astype(np.float32)
    res = o.sample_rank(u, beta=0.4)
    assert np.array_equal(res["idx"], o.rank_order()[np.floor(u.astype(np.float64) * n).astype(np.int64)])
    assert np.all(res["w"] == 1.0)
    o.close()


ALL_PINS = [pin_golden_hand_tree, pin_a_invariant, pin_b_root_bound, pin_c_update_equivalence,
            pin_d_dyadic_exact, pin_e_uniform_closed_form, pin_f_brute_force_band,
            pin_g_chi_square, pin_h_is_weights, pin_i_gather, pin_j_intake,
            pin_k_priority_decimal, pin_l_padded_gather, pin_m_device_masses,
            pin_n_rank_based]
