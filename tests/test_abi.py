"""The C ABI library loads, exports every entry point include/per.h declares,
and rejects bad arguments on the host before touching a device."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "per.h")
LIB = os.path.join(ROOT, "sum_tree_sampling_amd", "libper.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(per_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from sum_tree_sampling_amd import build
        build.build()
    from sum_tree_sampling_amd import per
    return per.load()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for must in ("per_workspace_bytes", "per_create", "per_destroy", "per_add", "per_update",
                 "per_sample", "per_total", "per_min", "per_max_priority", "per_size",
                 "per_cursor", "per_tree_ptrs", "per_last_error"):
        assert must in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (per_\w+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_binding_names_match_header():
    import sum_tree_sampling_amd as pkg
    for name in declared_functions():
        assert hasattr(pkg, name), name


def test_workspace_bytes_validation(lib):
    from sum_tree_sampling_amd import per
    n = 1 << 21
    b = per.per_workspace_bytes(n, 512)
    assert b >= 2 * 2 * n * 4
    for cap in (0, 1, 3, 1000, (1 << 30) + 1, 1 << 31, -8):
        with pytest.raises(per.PerError) as e:
            per.per_workspace_bytes(cap, 512)
        assert e.value.code == per.PER_EINVAL
    for mb in (0, -1, (1 << 24) + 1):
        with pytest.raises(per.PerError) as e:
            per.per_workspace_bytes(1024, mb)
        assert e.value.code == per.PER_EINVAL
    assert per.per_workspace_bytes(2, 1) > 0
    assert per.per_workspace_bytes(1 << 30, 1 << 24) > (1 << 33)


def _create(lib, **kw):
    args = dict(capacity=1024, state_dim=0, max_batch=64, alpha=0.6, eps=1e-6,
                ws=0x10000, ws_bytes=1 << 20, states=None, next_states=None, actions=None,
                rewards=None, dones=None)
    args.update(kw)
    h = ctypes.c_void_p(0)
    rc = lib.per_create(ctypes.byref(h), args["capacity"], args["state_dim"], args["max_batch"],
                        args["alpha"], args["eps"], args["ws"], args["ws_bytes"], args["states"],
                        args["next_states"], args["actions"], args["rewards"], args["dones"],
                        None)
    return rc, h.value


@pytest.mark.parametrize("kw,code", [
    (dict(capacity=1000), -1),
    (dict(capacity=1), -1),
    (dict(max_batch=0), -1),
    (dict(state_dim=-1), -1),
    (dict(alpha=0.0), -1),
    (dict(alpha=float("nan")), -1),
    (dict(eps=-1.0), -1),
    (dict(eps=float("inf")), -1),
    (dict(ws=None), -1),
    (dict(ws=0x10004), -1),
    (dict(ws_bytes=100), -2),
    (dict(state_dim=8), -1),                      # storage missing
    (dict(state_dim=0, states=0x20000), -1),      # storage without state_dim
    (dict(state_dim=8, states=0x20004, next_states=0x30000, actions=0x40000,
          rewards=0x50000, dones=0x60000), -1),   # misaligned rows
])
def test_create_rejects_on_host(lib, kw, code):
    rc, h = _create(lib, **kw)
    assert rc == code and not h
    assert lib.per_last_error().decode()


def test_null_handle_is_rejected(lib):
    assert lib.per_add(None, 1, None, None, None, None, None, None, None) == -1
    assert lib.per_update(None, 1, 0x1000, 0x1000, None) == -1
    assert lib.per_sample(None, 1, 0x1000, 0.4, 0x1000, None, None, None, None, None, None,
                          None) == -1
    assert lib.per_sample_padded(None, 1, 0x1000, 0.4, 0x1000, None, None, None, 8, None, None,
                                 None, None) == -1
    assert lib.per_sample_philox(None, 1, 1, 0, 0.4, 0x1000, None, None, None, None, None, None,
                                 None) == -1
    assert lib.per_sample_uniform(None, 1, 1, 0, 0x1000, None, None, None, None, None, None) == -1
    assert lib.per_rank_attach(None, 0x1000, 1 << 20) == -1
    assert lib.per_rank_refresh(None, None) == -1
    assert lib.per_sample_rank(None, 1, 0x1000, 0.4, 0x1000, None, None, None, None, None, None,
                               None) == -1
    assert lib.per_graph_mode(None, 1, None) == -1
    assert lib.per_update_add(None, 1, 0x1000, 0x1000, 1, None, None, None, None, None, None,
                              None) == -1
    assert lib.per_total(None, 0x1000, None) == -1
    assert lib.per_update_static(None, 1, 0x1000, 0x1000, None) == -1
    assert lib.per_set_sample_lanes(None, 0) == -1
    assert lib.per_time_next(None, None) == 0
    assert lib.per_destroy(None) == -1
    assert lib.per_size(None) == -1 and lib.per_cursor(None) == -1


PROBE_HEADER = os.path.join(ROOT, "include", "per_probe.h")
PROBE_LIB = os.path.join(ROOT, "sum_tree_sampling_amd", "libper_probe.so")


def test_probe_library_exports_and_checks():
    """libper_probe.so exports what include/per_probe.h declares and rejects
    bad arguments on the host (no launch is made for them)."""
    if not os.path.exists(PROBE_LIB):
        from sum_tree_sampling_amd import build
        build.build()
    text = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(per_probe_[a-z_]+)\s*\(", text)))
    assert names == ["per_probe_chain", "per_probe_empty", "per_probe_launch_cost"]
    out = subprocess.run(["nm", "-D", "--defined-only", PROBE_LIB], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (per_probe_\w+)$", out, flags=re.M))
    assert set(names) <= exported
    lib = ctypes.CDLL(PROBE_LIB)
    lib.per_probe_empty.argtypes = [ctypes.c_int64, ctypes.c_void_p]
    lib.per_probe_chain.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_void_p, ctypes.c_void_p]
    assert lib.per_probe_empty(0, None) == -1
    assert lib.per_probe_chain(None, 1024, 10, 0x1000, None) == -1
    assert lib.per_probe_chain(0x1000, 1000, 10, 0x1000, None) == -1   # not a power of two
    assert lib.per_probe_chain(0x1000, 1024, 0, 0x1000, None) == -1
    assert lib.per_probe_chain(0x1000, 1 << 31, 10, 0x1000, None) == -1
    lib.per_probe_launch_cost.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                          ctypes.POINTER(ctypes.c_double)]
    us = ctypes.c_double(0.0)
    assert lib.per_probe_launch_cost(3000, 256, 0, None) == -1
    assert lib.per_probe_launch_cost(50, 256, 0, ctypes.byref(us)) == -1     # under 100
    assert lib.per_probe_launch_cost(3050, 256, 1, ctypes.byref(us)) == -1   # not whole graphs
    assert lib.per_probe_launch_cost(3000, 100, 0, ctypes.byref(us)) == -1   # no such block


STAMPS_HEADER = os.path.join(ROOT, "include", "per_stamps.h")
STAMPS_LIB = os.path.join(ROOT, "sum_tree_sampling_amd", "libper_stamps.so")


def test_stamps_library_exports_and_checks(lib):
    """libper_stamps.so exports what include/per.h and include/per_stamps.h
    declare and rejects bad arguments on the host; libper.so carries no
    stamps."""
    if not os.path.exists(STAMPS_LIB):
        from sum_tree_sampling_amd import build
        build.build()
    text = re.sub(r"/\*.*?\*/", "", open(STAMPS_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(per_(?:sample_)?stamps_[a-z_]+)\s*\(", text)))
    assert names == ["per_sample_stamps_clear", "per_sample_stamps_read", "per_stamps_clear",
                     "per_stamps_read"]

    def exported(path):
        out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                             check=True).stdout
        return set(re.findall(r"\bT (per_\w+)$", out, flags=re.M))

    stamped = exported(STAMPS_LIB)
    for name in declared_functions() + names:
        assert name in stamped, name
    assert not [n for n in exported(LIB) if "stamps" in n]
    sl = ctypes.CDLL(STAMPS_LIB)
    sl.per_stamps_read.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p]
    buf = (ctypes.c_ulonglong * 4)()
    assert sl.per_stamps_read(None, 4, None) == -1
    assert sl.per_stamps_read(buf, -1, None) == -1
    assert sl.per_stamps_read(buf, 4096 * 16 + 1, None) == -1
    sl.per_sample_stamps_read.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p]
    assert sl.per_sample_stamps_read(None, 4, None) == -1
    assert sl.per_sample_stamps_read(buf, 4096 * 8 + 1, None) == -1
