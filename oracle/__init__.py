"""CPU oracle for the prioritized-replay sum tree (ctypes binding of pero.c).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the CPU-baseline leg of the benchmark may import this module.  It shares no
code with the HIP library and must never be used as a fallback for it.

Every call is a thin marshalling wrapper around the plain C loops in pero.c;
the arithmetic and its page citations live there.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pero.c")
_LIB = os.path.join(_HERE, "libpero.so")

# Plain C: every f32 operation is one IEEE round-to-nearest step.
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile pero.c into libpero.so next to it (gcc)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _bind(path: str):
    lib = ctypes.CDLL(path)
    i64, i32, f64, f32, vp = (ctypes.c_int64, ctypes.c_int32, ctypes.c_double,
                              ctypes.c_float, ctypes.c_void_p)
    lib.pero_create.restype = vp
    lib.pero_create.argtypes = [i64, i32, f64, f64]
    lib.pero_destroy.restype = None
    lib.pero_destroy.argtypes = [vp]
    lib.pero_add.restype = ctypes.c_int
    lib.pero_add.argtypes = [vp, i64, vp, vp, vp, vp, vp, vp]
    lib.pero_update.restype = ctypes.c_int
    lib.pero_update.argtypes = [vp, i64, vp, vp]
    lib.pero_sample.restype = ctypes.c_int
    lib.pero_sample.argtypes = [vp, i64, vp, f64, vp, vp, vp, vp, vp, vp, vp]
    lib.pero_sample_padded.restype = ctypes.c_int
    lib.pero_stream_word.restype = ctypes.c_uint64
    lib.pero_stream_word.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
    lib.pero_sample_philox.restype = ctypes.c_int
    lib.pero_sample_philox.argtypes = [vp, i64, ctypes.c_uint64, ctypes.c_uint64, f64, vp, vp, vp,
                                       vp, vp, vp, vp]
    lib.pero_sample_uniform.restype = ctypes.c_int
    lib.pero_sample_uniform.argtypes = [vp, i64, ctypes.c_uint64, ctypes.c_uint64, vp, vp, vp,
                                        vp, vp, vp]
    lib.pero_sample_padded.argtypes = [vp, i64, vp, f64, vp, vp, vp, vp, i64, vp, vp, vp]
    for name in ("pero_total", "pero_min", "pero_max_priority"):
        getattr(lib, name).restype = f32
        getattr(lib, name).argtypes = [vp]
    for name in ("pero_size", "pero_cursor", "pero_capacity"):
        getattr(lib, name).restype = i64
        getattr(lib, name).argtypes = [vp]
    lib.pero_state_dim.restype = i32
    lib.pero_state_dim.argtypes = [vp]
    lib.pero_rank_refresh.restype = ctypes.c_int
    lib.pero_rank_refresh.argtypes = [vp]
    lib.pero_sample_rank.restype = ctypes.c_int
    lib.pero_sample_rank.argtypes = [vp, i64, vp, f64, vp, vp, vp, vp, vp, vp, vp]
    lib.pero_rank_order.restype = ctypes.POINTER(i64)
    lib.pero_rank_order.argtypes = [vp]
    for name in ("pero_rank_sum_tree", "pero_rank_min_tree"):
        getattr(lib, name).restype = ctypes.POINTER(f32)
        getattr(lib, name).argtypes = [vp]
    for name in ("pero_sum_tree", "pero_min_tree"):
        getattr(lib, name).restype = ctypes.POINTER(f32)
        getattr(lib, name).argtypes = [vp]
    return lib


def load(path: str | None = None):
    """Load the compiled oracle (building it if absent)."""
    global _lib
    if path is not None:
        return _bind(path)
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(_LIB)
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype)


class Oracle:
    """Host-memory sum + min tree with ring storage, driven one element at a time."""

    def __init__(self, capacity: int, state_dim: int = 0, alpha: float = 0.6,
                 eps: float = 1e-6, lib=None):
        self._lib = lib if lib is not None else load()
        h = self._lib.pero_create(int(capacity), int(state_dim), float(alpha), float(eps))
        if not h:
            raise ValueError("pero_create rejected capacity=%r state_dim=%r"
                             % (capacity, state_dim))
        self._h = h
        self.capacity = int(capacity)
        self.state_dim = int(state_dim)

    def close(self):
        if getattr(self, "_h", None):
            self._lib.pero_destroy(self._h)
            self._h = None

    __del__ = close

    def add(self, count, states=None, next_states=None, actions=None, rewards=None,
            dones=None, prio=None):
        args = [_c(states, np.float32), _c(next_states, np.float32), _c(actions, np.uint32),
                _c(rewards, np.float32), _c(dones, np.uint8), _c(prio, np.float32)]
        rc = self._lib.pero_add(self._h, int(count), *[_ptr(a) for a in args])
        if rc != 0:
            raise ValueError("pero_add failed rc=%d" % rc)

    def update(self, idx, td):
        idx = _c(idx, np.int64)
        td = _c(td, np.float32)
        assert idx.shape == td.shape
        rc = self._lib.pero_update(self._h, idx.size, _ptr(idx), _ptr(td))
        if rc != 0:
            raise ValueError("pero_update failed rc=%d" % rc)

    def sample(self, u, beta=0.4, weights=True, rows=False):
        u = _c(u, np.float32)
        B = u.size
        idx = np.empty(B, np.int64)
        w = np.empty(B, np.float32) if weights else None
        D = self.state_dim
        outs = [None] * 5
        if rows and D > 0:
            outs = [np.empty((B, D), np.float32), np.empty((B, D), np.float32),
                    np.empty(B, np.uint32), np.empty(B, np.float32), np.empty(B, np.uint8)]
        rc = self._lib.pero_sample(self._h, B, _ptr(u), float(beta), _ptr(idx), _ptr(w),
                                   *[_ptr(o) for o in outs])
        if rc == -3:
            raise RuntimeError("sample from an empty buffer")
        if rc != 0:
            raise ValueError("pero_sample failed rc=%d" % rc)
        res = {"idx": idx}
        if weights:
            res["w"] = w
        if rows and D > 0:
            res.update(states=outs[0], next_states=outs[1], actions=outs[2],
                       rewards=outs[3], dones=outs[4])
        return res

    def stream_word(self, seed, j):
        """Word j of the Philox4x64-10 stream of a seed."""
        return int(self._lib.pero_stream_word(int(seed) & (2**64 - 1), int(j) & (2**64 - 1)))

    def _rows(self, B, rows):
        D = self.state_dim
        if rows and D > 0:
            return [np.empty((B, D), np.float32), np.empty((B, D), np.float32),
                    np.empty(B, np.uint32), np.empty(B, np.float32), np.empty(B, np.uint8)]
        return [None] * 5

    def _result(self, idx, w, outs, rows):
        res = {"idx": idx}
        if w is not None:
            res["w"] = w
        if rows and self.state_dim > 0:
            res.update(states=outs[0], next_states=outs[1], actions=outs[2],
                       rewards=outs[3], dones=outs[4])
        return res

    def sample_philox(self, B, seed, offset, beta=0.4, weights=True, rows=False):
        """pero_sample_philox: masses from words offset .. offset+B-1 of the stream."""
        idx = np.empty(B, np.int64)
        w = np.empty(B, np.float32) if weights else None
        outs = self._rows(B, rows)
        rc = self._lib.pero_sample_philox(self._h, B, int(seed) & (2**64 - 1),
                                          int(offset) & (2**64 - 1), float(beta), _ptr(idx),
                                          _ptr(w), *[_ptr(o) for o in outs])
        if rc == -3:
            raise RuntimeError("sample from an empty buffer")
        if rc != 0:
            raise ValueError("pero_sample_philox failed rc=%d" % rc)
        return self._result(idx, w, outs, rows)

    def sample_uniform(self, B, seed, offset, rows=False):
        """pero_sample_uniform: slots uniform over [0, size) from the stream."""
        idx = np.empty(B, np.int64)
        outs = self._rows(B, rows)
        rc = self._lib.pero_sample_uniform(self._h, B, int(seed) & (2**64 - 1),
                                           int(offset) & (2**64 - 1), _ptr(idx),
                                           *[_ptr(o) for o in outs])
        if rc == -3:
            raise RuntimeError("sample from an empty buffer")
        if rc != 0:
            raise ValueError("pero_sample_uniform failed rc=%d" % rc)
        return self._result(idx, None, outs, rows)

    def sample_padded(self, u, out_stride, beta=0.4, weights=True, rows=True):
        """pero_sample_padded: rows [B, out_stride] f32 zero past state_dim,
        actions i32, rewards f32, dones f32."""
        u = _c(u, np.float32)
        B = u.size
        idx = np.empty(B, np.int64)
        w = np.empty(B, np.float32) if weights else None
        outs = [None] * 5
        if rows and self.state_dim > 0:
            outs = [np.full((B, out_stride), np.nan, np.float32),
                    np.full((B, out_stride), np.nan, np.float32),
                    np.empty(B, np.int32), np.empty(B, np.float32), np.empty(B, np.float32)]
        rc = self._lib.pero_sample_padded(self._h, B, _ptr(u), float(beta), _ptr(idx), _ptr(w),
                                          _ptr(outs[0]), _ptr(outs[1]), int(out_stride),
                                          *[_ptr(o) for o in outs[2:]])
        if rc == -3:
            raise RuntimeError("sample from an empty buffer")
        if rc != 0:
            raise ValueError("pero_sample_padded failed rc=%d" % rc)
        res = {"idx": idx}
        if weights:
            res["w"] = w
        if rows and self.state_dim > 0:
            res.update(states=outs[0], next_states=outs[1], actions=outs[2],
                       rewards=outs[3], dones=outs[4])
        return res

    @property
    def total(self):
        return self._lib.pero_total(self._h)

    @property
    def min(self):
        return self._lib.pero_min(self._h)

    @property
    def max_priority(self):
        return self._lib.pero_max_priority(self._h)

    @property
    def size(self):
        return self._lib.pero_size(self._h)

    @property
    def cursor(self):
        return self._lib.pero_cursor(self._h)

    def sum_tree(self) -> np.ndarray:
        """Copy of the 2n-entry sum tree (index 0 unused)."""
        p = self._lib.pero_sum_tree(self._h)
        return np.ctypeslib.as_array(p, shape=(2 * self.capacity,)).copy()

    def min_tree(self) -> np.ndarray:
        p = self._lib.pero_min_tree(self._h)
        return np.ctypeslib.as_array(p, shape=(2 * self.capacity,)).copy()

    def rank_refresh(self):
        """pero_rank_refresh: rank the filled slots, rebuild the rank-weight tree."""
        if self._lib.pero_rank_refresh(self._h) != 0:
            raise MemoryError("pero_rank_refresh failed")

    def rank_order(self) -> np.ndarray:
        """Slots by rank (descending priority, ties by slot), as of the refresh."""
        p = self._lib.pero_rank_order(self._h)
        return np.ctypeslib.as_array(p, shape=(self.capacity,))[:self.size].copy()

    def rank_sum_tree(self) -> np.ndarray:
        p = self._lib.pero_rank_sum_tree(self._h)
        return np.ctypeslib.as_array(p, shape=(2 * self.capacity,)).copy()

    def rank_min_tree(self) -> np.ndarray:
        p = self._lib.pero_rank_min_tree(self._h)
        return np.ctypeslib.as_array(p, shape=(2 * self.capacity,)).copy()

    def sample_rank(self, u, beta=0.4, weights=True, rows=False):
        """pero_sample_rank: rank-based sample as of the last refresh."""
        u = _c(u, np.float32)
        B = u.size
        idx = np.empty(B, np.int64)
        w = np.empty(B, np.float32) if weights else None
        outs = self._rows(B, rows)
        rc = self._lib.pero_sample_rank(self._h, B, _ptr(u), float(beta), _ptr(idx), _ptr(w),
                                        *[_ptr(o) for o in outs])
        if rc == -3:
            raise RuntimeError("rank sample before a refresh, or from an empty buffer")
        if rc != 0:
            raise ValueError("pero_sample_rank failed rc=%d" % rc)
        return self._result(idx, w, outs, rows)
