"""Build libpa.so (the HIP kernels and the C ABI) and libpa_probe.so (bandwidth
probes used by the benchmark) in-tree for gfx950.

Usage: python -m paged_kv_gqa_pa_amd.build   (or build() from Python)
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libpa.so")
# The same library with device-side precondition checks (PA_DEVICE_CHECKS).
DEBUG_OUT = os.path.join(HERE, "libpa_debug.so")
DEBUG_FLAGS = ["-DPA_DEVICE_CHECKS=1"]
PROBE_OUT = os.path.join(HERE, "libpa_probe.so")
OBJDIR = os.path.join(HERE, "_build")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

SOURCES = ["pa_api.hip", "pa_cache.hip", "pa_decode.hip", "pa_verify.hip", "pa_prefill.hip",
           "pa_plan.hip"]
PROBE_SOURCES = ["probe.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-mcode-object-version=5",
    # no packed fp32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    path = os.path.join(ROCM, "bin", "hipcc")
    return path if os.path.exists(path) else shutil.which("hipcc") or "hipcc"


def _fresh(obj: str, src: str) -> bool:
    """With PA_BUILD_INCREMENTAL=1 in the environment, an object newer than its source
    and every header is reused (a development shortcut; build() compiles everything
    otherwise)."""
    if os.environ.get("PA_BUILD_INCREMENTAL") != "1" or not os.path.exists(obj):
        return False
    deps = [os.path.join(CSRC, src)] + [os.path.join(CSRC, h) for h in os.listdir(CSRC)
                                        if h.endswith(".h")]
    deps.append(os.path.join(HERE, "..", "include", "pa.h"))
    return all(os.path.getmtime(obj) > os.path.getmtime(d) for d in deps if os.path.exists(d))


def _compile(src: str, extra, objdir: str = None) -> str:
    objdir = objdir or OBJDIR
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    if _fresh(obj, src) and (not extra or objdir != OBJDIR):
        return obj
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-I", os.path.join(HERE, "..", "include"),
           "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    # --no-undefined: a kernel whose host stub was not emitted fails here, not at load time.
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = True, extra_flags=()) -> str:
    """Compile every HIP source, link libpa.so, libpa_debug.so (device checks) and
    libpa_probe.so; returns libpa's path.  PA_BUILD_SKIP_DEBUG=1 in the environment
    leaves the debug library out (a development shortcut)."""
    dbg_dir = os.path.join(OBJDIR, "debug")
    os.makedirs(dbg_dir, exist_ok=True)
    jobs_list = [(s, list(extra_flags), OBJDIR) for s in SOURCES + PROBE_SOURCES]
    with_debug = os.environ.get("PA_BUILD_SKIP_DEBUG") != "1"
    if with_debug:
        jobs_list += [(s, list(extra_flags) + DEBUG_FLAGS, dbg_dir) for s in SOURCES]
    jobs = min(len(jobs_list), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs_list))
    n = len(SOURCES)
    _link(objs[:n], OUT)
    _link(objs[n:n + len(PROBE_SOURCES)], PROBE_OUT)
    if with_debug:
        _link(objs[n + len(PROBE_SOURCES):], DEBUG_OUT)
    if verbose:
        print(f"built {OUT}, {PROBE_OUT}" + (f" and {DEBUG_OUT}" if with_debug else ""))
    return OUT


if __name__ == "__main__":
    build(verbose=True, extra_flags=sys.argv[1:])
