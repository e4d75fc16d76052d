"""Thin Python binding of the C ABI in include/per.h (libper.so, HIP, gfx950).

Functions carry the C names and only marshal arguments: device tensors are
passed as their data pointers and the stream as torch's current HIP stream.
Every step of the work runs in the library's kernels; there is no host or
CPU fallback, and loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libper.so")

PER_OK, PER_EINVAL, PER_ENOSPC, PER_EEMPTY, PER_EHIP = 0, -1, -2, -3, -4

_lib = None


class PerError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("per error %d: %s" % (code, msg))
        self.code = code


_U64 = (1 << 64) - 1

def load(path: str | None = None) -> ctypes.CDLL:
    """Load libper.so (raises if it is missing: build it with build.build())."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError("libper.so not built at %s; run sum_tree_sampling_amd.build.build()" % p)
    lib = ctypes.CDLL(p)
    i64, i32, f64, vp, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_double, ctypes.c_void_p, ctypes.c_size_t
    u64 = ctypes.c_uint64
    c_int = ctypes.c_int
    sig = {
        "per_workspace_bytes": (c_int, [i64, i64, ctypes.POINTER(sz)]),
        "per_create": (c_int, [ctypes.POINTER(vp), i64, i32, i64, f64, f64, vp, sz, vp, vp, vp,
                               vp, vp, vp]),
        "per_destroy": (c_int, [vp]),
        "per_add": (c_int, [vp, i64, vp, vp, vp, vp, vp, vp, vp]),
        "per_update": (c_int, [vp, i64, vp, vp, vp]),
        "per_update_static": (c_int, [vp, i64, vp, vp, vp]),
        "per_set_sample_lanes": (c_int, [vp, i32]),
        "per_time_next": (c_int, [vp, vp]),
        "per_update_add": (c_int, [vp, i64, vp, vp, i64, vp, vp, vp, vp, vp, vp, vp]),
        "per_sample": (c_int, [vp, i64, vp, f64, vp, vp, vp, vp, vp, vp, vp, vp]),
        "per_sample_padded": (c_int, [vp, i64, vp, f64, vp, vp, vp, vp, i64, vp, vp, vp, vp]),
        "per_sample_philox": (c_int, [vp, i64, u64, u64, f64, vp, vp, vp, vp, vp, vp, vp, vp]),
        "per_sample_uniform": (c_int, [vp, i64, u64, u64, vp, vp, vp, vp, vp, vp, vp]),
        "per_rank_workspace_bytes": (c_int, [i64, ctypes.POINTER(sz)]),
        "per_rank_attach": (c_int, [vp, vp, sz]),
        "per_rank_refresh": (c_int, [vp, vp]),
        "per_sample_rank": (c_int, [vp, i64, vp, f64, vp, vp, vp, vp, vp, vp, vp, vp]),
        "per_rank_ptrs": (c_int, [vp, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                  ctypes.POINTER(vp)]),
        "per_flush": (c_int, [vp, vp]),
        "per_graph_mode": (c_int, [vp, i32, vp]),
        "per_total": (c_int, [vp, vp, vp]),
        "per_min": (c_int, [vp, vp, vp]),
        "per_max_priority": (c_int, [vp, vp, vp]),
        "per_size": (i64, [vp]),
        "per_cursor": (i64, [vp]),
        "per_capacity": (i64, [vp]),
        "per_state_dim": (i32, [vp]),
        "per_tree_ptrs": (c_int, [vp, ctypes.POINTER(vp), ctypes.POINTER(vp)]),
        "per_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _check(rc: int) -> None:
    if rc != PER_OK:
        raise PerError(rc, load().per_last_error().decode())


def _p(t) -> int | None:
    """Data pointer of a device tensor (None passes NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not (t.is_cuda and t.is_contiguous()):
        raise ValueError("expected a contiguous device tensor")
    return t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream=None) -> int:
    """hipStream_t of `stream`, or of torch's current stream on the current device."""
    if stream is None:
        if _raw_stream is not None:
            return _raw_stream(torch.cuda.current_device())
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# ---------------------------------------------------------------- C names

def per_workspace_bytes(capacity: int, max_batch: int) -> int:
    out = ctypes.c_size_t(0)
    _check(load().per_workspace_bytes(int(capacity), int(max_batch), ctypes.byref(out)))
    return out.value


def per_create(capacity, state_dim, max_batch, alpha, eps, ws, ws_bytes=None, states=None,
               next_states=None, actions=None, rewards=None, dones=None, stream=None) -> int:
    h = ctypes.c_void_p(0)
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else int(ws_bytes)
    _check(load().per_create(ctypes.byref(h), int(capacity), int(state_dim), int(max_batch),
                             float(alpha), float(eps), _p(ws), nbytes, _p(states),
                             _p(next_states), _p(actions), _p(rewards), _p(dones),
                             _stream(stream)))
    return h.value


def per_destroy(h: int) -> None:
    _check(load().per_destroy(h))


def per_add(h, count, states=None, next_states=None, actions=None, rewards=None, dones=None,
            prio=None, stream=None) -> None:
    _check(load().per_add(h, int(count), _p(states), _p(next_states), _p(actions), _p(rewards),
                          _p(dones), _p(prio), _stream(stream)))


def per_update(h, B, idx, td, stream=None) -> None:
    _check(load().per_update(h, int(B), _p(idx), _p(td), _stream(stream)))


def per_update_static(h, B, idx, td, stream=None) -> None:
    _check(load().per_update_static(h, int(B), _p(idx), _p(td), _stream(stream)))


def per_set_sample_lanes(h, lanes) -> None:
    _check(load().per_set_sample_lanes(h, int(lanes)))


def per_time_next(start=None, stop=None) -> None:
    """Time the next call's kernels: start / stop are torch.cuda.Event
    (created with enable_timing=True) or raw hipEvent_t handles."""
    _check(load().per_time_next(_event(start), _event(stop)))


def _event(e):
    if e is None:
        return None
    if isinstance(e, int):
        return e
    return e.cuda_event if hasattr(e, "cuda_event") else int(e)


def per_update_add(h, B, idx, td, count, states=None, next_states=None, actions=None,
                   rewards=None, dones=None, prio=None, stream=None) -> None:
    _check(load().per_update_add(h, int(B), _p(idx), _p(td), int(count), _p(states),
                                 _p(next_states), _p(actions), _p(rewards), _p(dones), _p(prio),
                                 _stream(stream)))


def per_sample(h, B, u, beta, idx_out, w_out=None, states_out=None, next_states_out=None,
               actions_out=None, rewards_out=None, dones_out=None, stream=None) -> None:
    _check(load().per_sample(h, int(B), _p(u), float(beta), _p(idx_out), _p(w_out),
                             _p(states_out), _p(next_states_out), _p(actions_out),
                             _p(rewards_out), _p(dones_out), _stream(stream)))


def per_sample_padded(h, B, u, beta, idx_out, w_out=None, states_out=None, next_states_out=None,
                      out_stride=0, actions_out=None, rewards_out=None, dones_out=None,
                      stream=None) -> None:
    _check(load().per_sample_padded(h, int(B), _p(u), float(beta), _p(idx_out), _p(w_out),
                                    _p(states_out), _p(next_states_out), int(out_stride),
                                    _p(actions_out), _p(rewards_out), _p(dones_out),
                                    _stream(stream)))


def per_sample_philox(h, B, seed, offset, beta, idx_out, w_out=None, states_out=None,
                      next_states_out=None, actions_out=None, rewards_out=None, dones_out=None,
                      stream=None) -> None:
    _check(load().per_sample_philox(h, int(B), int(seed) & _U64, int(offset) & _U64, float(beta),
                                    _p(idx_out), _p(w_out), _p(states_out), _p(next_states_out),
                                    _p(actions_out), _p(rewards_out), _p(dones_out),
                                    _stream(stream)))


def per_sample_uniform(h, B, seed, offset, idx_out, states_out=None, next_states_out=None,
                       actions_out=None, rewards_out=None, dones_out=None, stream=None) -> None:
    _check(load().per_sample_uniform(h, int(B), int(seed) & _U64, int(offset) & _U64,
                                     _p(idx_out), _p(states_out), _p(next_states_out),
                                     _p(actions_out), _p(rewards_out), _p(dones_out),
                                     _stream(stream)))


def per_rank_workspace_bytes(capacity) -> int:
    out = ctypes.c_size_t(0)
    _check(load().per_rank_workspace_bytes(int(capacity), ctypes.byref(out)))
    return out.value


def per_rank_attach(h, ws, nbytes) -> None:
    _check(load().per_rank_attach(h, _p(ws), int(nbytes)))


def per_rank_refresh(h, stream=None) -> None:
    _check(load().per_rank_refresh(h, _stream(stream)))


def per_sample_rank(h, B, u, beta, idx_out, w_out=None, states_out=None, next_states_out=None,
                    actions_out=None, rewards_out=None, dones_out=None, stream=None) -> None:
    _check(load().per_sample_rank(h, int(B), _p(u), float(beta), _p(idx_out), _p(w_out),
                                  _p(states_out), _p(next_states_out), _p(actions_out),
                                  _p(rewards_out), _p(dones_out), _stream(stream)))


def per_rank_ptrs(h):
    o, s, m = ctypes.c_void_p(0), ctypes.c_void_p(0), ctypes.c_void_p(0)
    _check(load().per_rank_ptrs(h, ctypes.byref(o), ctypes.byref(s), ctypes.byref(m)))
    return o.value, s.value, m.value


def per_flush(h, stream=None) -> None:
    _check(load().per_flush(h, _stream(stream)))


def per_graph_mode(h, on, stream=None) -> None:
    _check(load().per_graph_mode(h, 1 if on else 0, _stream(stream)))


def per_total(h, out, stream=None) -> None:
    _check(load().per_total(h, _p(out), _stream(stream)))


def per_min(h, out, stream=None) -> None:
    _check(load().per_min(h, _p(out), _stream(stream)))


def per_max_priority(h, out, stream=None) -> None:
    _check(load().per_max_priority(h, _p(out), _stream(stream)))


def per_size(h) -> int:
    return load().per_size(h)


def per_cursor(h) -> int:
    return load().per_cursor(h)


def per_capacity(h) -> int:
    return load().per_capacity(h)


def per_state_dim(h) -> int:
    return load().per_state_dim(h)


def per_tree_ptrs(h):
    s, m = ctypes.c_void_p(0), ctypes.c_void_p(0)
    _check(load().per_tree_ptrs(h, ctypes.byref(s), ctypes.byref(m)))
    return s.value, m.value


def per_last_error() -> str:
    return load().per_last_error().decode()


# ---------------------------------------------------------------- convenience

class PerBuffer:
    """Device memory (torch) plus a handle.  Actions are stored as 32-bit
    words (torch.int32 holds the u32 bit patterns unchanged)."""

    def __init__(self, capacity: int, state_dim: int = 0, max_batch: int = 4096,
                 alpha: float = 0.6, eps: float = 1e-6, device="cuda", stream=None):
        self.capacity, self.state_dim, self.max_batch = int(capacity), int(state_dim), int(max_batch)
        self.device = torch.device(device)
        nbytes = per_workspace_bytes(capacity, max_batch)
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self.storage = None
        if state_dim > 0:
            self.storage = dict(
                states=torch.empty((capacity, state_dim), dtype=torch.float32, device=self.device),
                next_states=torch.empty((capacity, state_dim), dtype=torch.float32, device=self.device),
                actions=torch.empty(capacity, dtype=torch.int32, device=self.device),
                rewards=torch.empty(capacity, dtype=torch.float32, device=self.device),
                dones=torch.empty(capacity, dtype=torch.uint8, device=self.device),
            )
        st = self.storage or {}
        self.h = per_create(capacity, state_dim, max_batch, alpha, eps, self.ws, nbytes,
                            st.get("states"), st.get("next_states"), st.get("actions"),
                            st.get("rewards"), st.get("dones"), stream)
        sp, mp = per_tree_ptrs(self.h)
        base = self.ws.data_ptr()
        f = self.ws.view(torch.float32)
        n2 = 2 * self.capacity
        self._sum = f[(sp - base) // 4:(sp - base) // 4 + n2]
        self._min = f[(mp - base) // 4:(mp - base) // 4 + n2]

    def close(self):
        if getattr(self, "h", None):
            per_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def size(self) -> int:
        return per_size(self.h)

    @property
    def cursor(self) -> int:
        return per_cursor(self.h)

    def graph_mode(self, on: bool, stream=None) -> None:
        """Enter / leave graph mode (per_graph_mode): calls issued in it may
        be captured and replayed; leaving waits for the stream."""
        per_graph_mode(self.h, on, stream)

    def sum_tree(self, stream=None) -> torch.Tensor:
        """Device view of the [2n] sum tree (index 0 unused), flushed first."""
        per_flush(self.h, stream)
        return self._sum

    def min_tree(self, stream=None) -> torch.Tensor:
        per_flush(self.h, stream)
        return self._min

    def add(self, count, states=None, next_states=None, actions=None, rewards=None, dones=None,
            prio=None, stream=None):
        per_add(self.h, count, states, next_states, actions, rewards, dones, prio, stream)

    def update(self, idx, td, stream=None):
        per_update(self.h, idx.numel(), idx, td, stream)

    def update_static(self, idx, td, stream=None):
        """per_update_static: per_update with its scratch in the library's
        static device array (allocates nothing)."""
        per_update_static(self.h, idx.numel(), idx, td, stream)

    def set_sample_lanes(self, lanes: int) -> None:
        """per_set_sample_lanes: 64, 16 or 1 lanes per sample; 0 = automatic."""
        per_set_sample_lanes(self.h, lanes)

    def update_add(self, idx, td, count, states=None, next_states=None, actions=None,
                   rewards=None, dones=None, prio=None, stream=None):
        """per_update_add: update(idx, td), then add(count, ...), in one launch."""
        per_update_add(self.h, idx.numel(), idx, td, count, states, next_states, actions,
                       rewards, dones, prio, stream)

    def sample(self, u, beta=0.4, weights=True, rows=False, out=None, stream=None):
        B = u.numel()
        if out is None:
            out = {"idx": torch.empty(B, dtype=torch.int64, device=self.device)}
            if weights:
                out["w"] = torch.empty(B, dtype=torch.float32, device=self.device)
            if rows:
                D = self.state_dim
                out.update(
                    states=torch.empty((B, D), dtype=torch.float32, device=self.device),
                    next_states=torch.empty((B, D), dtype=torch.float32, device=self.device),
                    actions=torch.empty(B, dtype=torch.int32, device=self.device),
                    rewards=torch.empty(B, dtype=torch.float32, device=self.device),
                    dones=torch.empty(B, dtype=torch.uint8, device=self.device))
        per_sample(self.h, B, u, beta, out["idx"], out.get("w"), out.get("states"),
                   out.get("next_states"), out.get("actions"), out.get("rewards"),
                   out.get("dones"), stream)
        return out

    def _outs(self, B, weights, rows):
        out = {"idx": torch.empty(B, dtype=torch.int64, device=self.device)}
        if weights:
            out["w"] = torch.empty(B, dtype=torch.float32, device=self.device)
        if rows:
            D = self.state_dim
            out.update(
                states=torch.empty((B, D), dtype=torch.float32, device=self.device),
                next_states=torch.empty((B, D), dtype=torch.float32, device=self.device),
                actions=torch.empty(B, dtype=torch.int32, device=self.device),
                rewards=torch.empty(B, dtype=torch.float32, device=self.device),
                dones=torch.empty(B, dtype=torch.uint8, device=self.device))
        return out

    def sample_philox(self, B, seed, offset, beta=0.4, weights=True, rows=False, out=None,
                      stream=None):
        """per_sample_philox: masses from stream words offset .. offset+B-1."""
        out = out or self._outs(B, weights, rows)
        per_sample_philox(self.h, B, seed, offset, beta, out["idx"], out.get("w"),
                          out.get("states"), out.get("next_states"), out.get("actions"),
                          out.get("rewards"), out.get("dones"), stream)
        return out

    def sample_uniform(self, B, seed, offset, rows=False, out=None, stream=None):
        """per_sample_uniform: B slots uniform over [0, size) from the stream."""
        out = out or self._outs(B, False, rows)
        per_sample_uniform(self.h, B, seed, offset, out["idx"], out.get("states"),
                           out.get("next_states"), out.get("actions"), out.get("rewards"),
                           out.get("dones"), stream)
        return out

    def rank_attach(self):
        """Allocate and attach the rank-based workspace (torch-owned)."""
        nbytes = per_rank_workspace_bytes(self.capacity)
        self.rank_ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
        off = (-self.rank_ws.data_ptr()) % 256
        self._rank_ws = self.rank_ws[off:off + nbytes]
        per_rank_attach(self.h, self._rank_ws, nbytes)

    def rank_refresh(self, stream=None):
        per_rank_refresh(self.h, stream)

    def _rank_view(self, ptr, count, dtype):
        base = self._rank_ws.data_ptr()
        item = torch.empty((), dtype=dtype).element_size()
        return self._rank_ws[ptr - base:ptr - base + count * item].view(dtype)

    def rank_order(self) -> torch.Tensor:
        """Device view of the ranking (slot of each rank, int32 bits of u32)."""
        o, _, _ = per_rank_ptrs(self.h)
        return self._rank_view(o, self.size, torch.int32)

    def rank_trees(self):
        """Device views of the two rank-weight trees (2n f32 each)."""
        _, s, m = per_rank_ptrs(self.h)
        return (self._rank_view(s, 2 * self.capacity, torch.float32),
                self._rank_view(m, 2 * self.capacity, torch.float32))

    def sample_rank(self, u, beta=0.4, weights=True, rows=False, out=None, stream=None):
        """per_sample_rank: rank-based sample as of the last refresh."""
        out = out or self._outs(u.numel(), weights, rows)
        per_sample_rank(self.h, u.numel(), u, beta, out["idx"], out.get("w"), out.get("states"),
                        out.get("next_states"), out.get("actions"), out.get("rewards"),
                        out.get("dones"), stream)
        return out

    def sample_padded(self, u, out_stride, beta=0.4, weights=True, out=None, stream=None):
        """per_sample_padded: state rows [B, out_stride] zero past state_dim,
        actions i32, rewards f32, dones f32 (the trainer's input layout)."""
        B = u.numel()
        if out is None:
            out = {"idx": torch.empty(B, dtype=torch.int64, device=self.device)}
            if weights:
                out["w"] = torch.empty(B, dtype=torch.float32, device=self.device)
            if self.state_dim > 0:
                out.update(
                    states=torch.empty((B, out_stride), dtype=torch.float32, device=self.device),
                    next_states=torch.empty((B, out_stride), dtype=torch.float32,
                                            device=self.device),
                    actions=torch.empty(B, dtype=torch.int32, device=self.device),
                    rewards=torch.empty(B, dtype=torch.float32, device=self.device),
                    dones=torch.empty(B, dtype=torch.float32, device=self.device))
        per_sample_padded(self.h, B, u, beta, out["idx"], out.get("w"), out.get("states"),
                          out.get("next_states"), out_stride, out.get("actions"),
                          out.get("rewards"), out.get("dones"), stream)
        return out

    def scalar(self, which: str, stream=None) -> torch.Tensor:
        out = torch.empty(1, dtype=torch.float32, device=self.device)
        {"total": per_total, "min": per_min, "max_priority": per_max_priority}[which](
            self.h, out, stream)
        return out
