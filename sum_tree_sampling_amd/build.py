"""Compile the HIP library (libper.so), the latency probe (libper_probe.so)
and the library's phase-stamped measurement build (libper_stamps.so) for
gfx950, in-tree, with hipcc."""
from __future__ import annotations

import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libper.so")
SOURCES = ["per_api.hip", "tree_kernels.hip", "sample_kernels.hip", "rank_kernels.hip"]
PROBE_SRC = os.path.join(HERE, "probe", "latency_probe.hip")
PROBE_LIB = os.path.join(HERE, "libper_probe.so")
STAMPS_LIB = os.path.join(HERE, "libper_stamps.so")
STAMPED = ("tree_kernels.hip", "sample_kernels.hip")  # sources whose kernels carry stamps

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# IEEE f32 arithmetic as written: no contraction into FMA, no fast-math, no
# flush-to-zero of denormals; packed-FP32 instructions disabled.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-kernarg-preload-count=5",
    "-Wall", "-Wno-unused-function",
]


# The compiler's per-kernel resource report, read to refuse kernels that use
# scratch memory: a kernel on the path keeps its values in registers and LDS
# (a helper left out of line, or an array indexed through a pointer, would
# silently move them to per-lane scratch in device memory).
RESOURCE_FLAG = "-Rpass-analysis=kernel-resource-usage"


def scratch_users(report: str) -> list:
    """Kernels of a resource report with a nonzero ScratchSize."""
    out, name = [], None
    for ln in report.splitlines():
        m = re.search(r"Function Name: (\S+)", ln)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", ln)
        if m and name and int(m.group(1)) > 0:
            out.append((name, int(m.group(1))))
    return out


def _compile(src: str, obj: str, defines: tuple = ()) -> None:
    cmd = [HIPCC, *FLAGS, *["-D" + d for d in defines], RESOURCE_FLAG, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed on %s" % src)
    users = scratch_users(r.stderr)
    if users:
        raise RuntimeError("kernels of %s use scratch memory: %s" % (
            os.path.basename(src), ", ".join("%s (%d B/lane)" % u for u in users)))
    # the host pass does not know the packed-fp32 feature; that note is expected
    # and the resource report (remarks with their source excerpts) is read above
    noise = [ln for ln in r.stderr.splitlines()
             if "packed-fp32-ops" not in ln and "remark:" not in ln
             and not re.match(r"^\s*\d*\s*\|", ln) and ln.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")


def build() -> str:
    """Compile every source and link libper.so, libper_probe.so and
    libper_stamps.so (libper.so with PER_PHASE_STAMPS in the STAMPED sources)
    next to this file."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    srcs = [os.path.join(CSRC, s) for s in SOURCES] + [PROBE_SRC]
    objs = [os.path.join(objdir, os.path.basename(s).replace(".hip", ".o")) for s in srcs]
    stamped = {f.replace(".hip", ".o"): os.path.join(objdir, f.replace(".hip", "_stamps.o"))
               for f in STAMPED}
    jobs = [(s, o, ()) for s, o in zip(srcs, objs)]
    jobs += [(os.path.join(CSRC, f), stamped[f.replace(".hip", ".o")], ("PER_PHASE_STAMPS",))
             for f in STAMPED]
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        list(ex.map(lambda job: _compile(*job), jobs))
    lib_objs = objs[:-1]
    stamps_objs = [stamped.get(os.path.basename(o), o) for o in lib_objs]
    for lib, lib_objs in ((LIB, lib_objs), (PROBE_LIB, objs[-1:]), (STAMPS_LIB, stamps_objs)):
        tmp = lib + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *lib_objs]
        subprocess.check_call(cmd)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build())
