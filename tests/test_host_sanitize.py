"""The C ABI's host-side validation under AddressSanitizer and UBSan, on the CPU.

Every HIP source of the library is compiled with the sanitizers on the host
pass only (device code is built as usual, at -O1: it never runs here), linked
with tests/sanitize_abi.cpp, and run: every entry point is called with invalid arguments (and, with no GPU
visible, with valid ones, which then fail at the HIP layer).  The run must
exit 0 with no sanitizer report.
"""
import concurrent.futures as cf
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_gqa_pa_amd", "csrc")
SOURCES = ["pa_api.hip", "pa_cache.hip", "pa_decode.hip", "pa_verify.hip", "pa_prefill.hip",
           "pa_plan.hip"]
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_host_validation_under_sanitizers(tmp_path):
    def compile_one(src):
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *SAN,
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, src), "-o", obj]
        return obj, subprocess.run(cmd, capture_output=True, text=True)

    with cf.ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 1)) as ex:
        results = list(ex.map(compile_one, SOURCES))
    for obj, res in results:
        assert res.returncode == 0, res.stderr[-3000:]
    objs = [obj for obj, _ in results]
    exe = str(tmp_path / "sanitize_abi")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", *SAN,
           "-I", os.path.join(ROOT, "include"), "-x", "hip",
           os.path.join(ROOT, "tests", "sanitize_abi.cpp"), "-x", "none", *objs, "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = res.stdout + res.stderr
    print(out[-4000:])
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert "OK: 0 failure(s)" in out
