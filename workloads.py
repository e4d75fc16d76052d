"""Seeded synthetic inputs for the prioritized-replay workloads.

This module only draws random numbers in the shapes and distributions of the
workloads.  It holds none of the sum-tree method's arithmetic (no tree, no
descent, no priority transform of TD errors, no weights), and it imports
neither the HIP package nor the oracle; both of them are fed from here.

Every workload draws from numpy's PCG64 seeded by SeedSequence(seed), spawned
once, in a fixed order, into independent streams:
    0 initial priorities, 1 zero mask, 2 rows (one child per 2^16-row chunk),
    3 (reserved), 4 uniforms u per step, 5 TD errors per step,
    6 update-index construction per step.
Per-step arrays are always drawn one step at a time, so step s holds the same
values however many steps a caller asks for.

Workloads (capacity n, batch B, state_dim D):
  tiny_1k              n=2^10, B=32,    D=8,   priorities U(0.01,1)^0.6
  apex_shard_2m        n=2^21, B=512,   D=0,   priorities (|N(0,1)|+1e-6)^0.6,
                       td ~ Laplace(0,1), 400-transition intake per step
  dqn_1m               n=2^20, B=1024,  D=64,  filled at the running max priority
  collision_stress_2m  n=2^21, B=4096,  D=0,   priorities lognormal(0,3) with
                       exactly round(0.1 n) zeros; update indices are 2048
                       distinct slots plus 2048 repeats of them, shuffled
  large_16m            n=2^24, B=65536, D=128, priorities U(0,1)^0.6
Rows: states / next_states ~ N(0,1) f32, actions uniform in {0,1,2} (u32),
rewards ~ N(0,1) f32, dones ~ Bernoulli(0.01) (u8).
"""
from __future__ import annotations

import numpy as np

ROW_CHUNK = 1 << 16

WORKLOADS = {
    "tiny_1k": dict(capacity=1 << 10, batch=32, state_dim=8, intake=0, td="normal",
                    prio="uniform_0.01_1_pow", seed=1001, beta=0.4, weights=True),
    "apex_shard_2m": dict(capacity=1 << 21, batch=512, state_dim=0, intake=400,
                          td="laplace", prio="absnormal_pow", seed=1002, beta=0.4,
                          weights=False),
    "dqn_1m": dict(capacity=1 << 20, batch=1024, state_dim=64, intake=0, td="normal",
                   prio=None, seed=1003, beta=0.4, weights=True),
    "collision_stress_2m": dict(capacity=1 << 21, batch=4096, state_dim=0, intake=0,
                                td="normal", prio="lognormal3_zeros", seed=1004,
                                beta=0.4, weights=False, unique=2048),
    "large_16m": dict(capacity=1 << 24, batch=65536, state_dim=128, intake=0, td="normal",
                      prio="uniform_pow", seed=1005, beta=0.4, weights=True),
}

ALPHA = 0.6
EPS = 1e-6

_N_STREAMS = 7


def spec(name: str) -> dict:
    s = dict(WORKLOADS[name])
    s["name"] = name
    return s


def _streams(seed: int):
    return np.random.SeedSequence(seed).spawn(_N_STREAMS)


def _rng(ss):
    return np.random.Generator(np.random.PCG64(ss))


def initial_priorities(name: str, capacity: int | None = None, seed: int | None = None):
    """f32 priorities for the initial bulk fill, or None (fill at the running max)."""
    s = spec(name)
    n = capacity or s["capacity"]
    ss = _streams(seed if seed is not None else s["seed"])
    rng = _rng(ss[0])
    kind = s["prio"]
    if kind is None:
        return None
    if kind == "uniform_0.01_1_pow":
        p = rng.uniform(0.01, 1.0, n) ** 0.6
    elif kind == "absnormal_pow":
        p = (np.abs(rng.standard_normal(n)) + 1e-6) ** 0.6
    elif kind == "lognormal3_zeros":
        p = np.exp(3.0 * rng.standard_normal(n))
        zr = _rng(ss[1])
        nz = int(round(0.1 * n))
        p[zr.choice(n, size=nz, replace=False)] = 0.0
    elif kind == "uniform_pow":
        p = rng.random(n) ** 0.6
    else:
        raise KeyError(kind)
    return p.astype(np.float32)


def row_chunk(name: str, k: int, state_dim: int | None = None, seed: int | None = None,
              capacity: int | None = None) -> dict:
    """Rows [k*ROW_CHUNK, (k+1)*ROW_CHUNK) of the transition storage (clipped to capacity)."""
    s = spec(name)
    D = s["state_dim"] if state_dim is None else state_dim
    n = capacity or s["capacity"]
    nchunks = (n + ROW_CHUNK - 1) // ROW_CHUNK
    if not 0 <= k < nchunks:
        raise IndexError(k)
    rows = min(ROW_CHUNK, n - k * ROW_CHUNK)
    child = _streams(seed if seed is not None else s["seed"])[2].spawn(nchunks)[k]
    rng = _rng(child)
    return dict(
        states=rng.standard_normal((rows, D), dtype=np.float32),
        next_states=rng.standard_normal((rows, D), dtype=np.float32),
        actions=rng.integers(0, 3, rows, dtype=np.uint32),
        rewards=rng.standard_normal(rows, dtype=np.float32),
        dones=(rng.random(rows) < 0.01).astype(np.uint8),
    )


def rows(name: str, start: int, count: int, **kw) -> dict:
    """Rows [start, start+count) assembled from their chunks."""
    out = None
    pos = 0
    k0 = start // ROW_CHUNK
    k1 = (start + count - 1) // ROW_CHUNK
    for k in range(k0, k1 + 1):
        c = row_chunk(name, k, **kw)
        lo = max(start, k * ROW_CHUNK) - k * ROW_CHUNK
        hi = min(start + count, (k + 1) * ROW_CHUNK) - k * ROW_CHUNK
        if out is None:
            out = {key: np.empty((count,) + v.shape[1:], v.dtype) for key, v in c.items()}
        for key, v in c.items():
            out[key][pos:pos + hi - lo] = v[lo:hi]
        pos += hi - lo
    return out


class StepInputs:
    """Per-step uniforms, TD errors and (for the collision workload) update indices."""

    def __init__(self, name: str, seed: int | None = None, batch: int | None = None,
                 capacity: int | None = None):
        s = spec(name)
        self.spec = s
        self.B = batch or s["batch"]
        self.n = capacity or s["capacity"]
        ss = _streams(seed if seed is not None else s["seed"])
        self._u = _rng(ss[4])
        self._td = _rng(ss[5])
        self._dup = _rng(ss[6])

    def u(self) -> np.ndarray:
        """B uniforms in [0, 1) (f32)."""
        return self._u.random(self.B, dtype=np.float32)

    def td(self) -> np.ndarray:
        if self.spec["td"] == "laplace":
            return self._td.laplace(0.0, 1.0, self.B).astype(np.float32)
        return self._td.standard_normal(self.B, dtype=np.float32)

    def update_idx(self) -> np.ndarray:
        """Constructed update indices: U distinct uniform slots plus B-U repeats, shuffled."""
        U = self.spec.get("unique", self.B)
        distinct = self._dup.choice(self.n, size=U, replace=False)
        rep = self._dup.choice(distinct, size=self.B - U, replace=True)
        idx = np.concatenate([distinct, rep]).astype(np.int64)
        self._dup.shuffle(idx)
        return idx
