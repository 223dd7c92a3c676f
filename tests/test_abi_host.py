"""Host-side checks of the C ABI that need no GPU.

The library must load, export every function include/pa.h declares, and
reject invalid arguments on the host before anything would be launched (these
calls pass NULL or dummy pointers that are never dereferenced).
"""
import ctypes
import os
import re

import pytest

from paged_kv_gqa_pa_amd import _lib as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "pa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(pa_\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_function():
    lib = pa.lib()
    names = declared_functions()
    assert set(names) >= {"pa_decode", "pa_verify", "pa_reshape_and_cache"}
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(pa.EXPORTED) == names


def test_version_and_default_split():
    lib = pa.lib()
    assert lib.pa_version() >= 100
    # vector-ALU decode (fp32, bf16 groups below 4): 64 positions per KV head within [128, 512]
    assert lib.pa_default_split_tokens(1, 16, 8, 128, pa.PA_BF16) == 512
    assert lib.pa_default_split_tokens(1, 6, 2, 128, pa.PA_BF16) == 128
    assert lib.pa_default_split_tokens(1, 2, 1, 64, pa.PA_F32) == 128
    assert lib.pa_default_split_tokens(1, 96, 16, 128, pa.PA_F32) == 512
    # matrix-core kernel (verify, int8, bf16 groups of 4+): 1024 per KV head within [2048, 4096]
    assert lib.pa_default_split_tokens(5, 16, 8, 128, pa.PA_BF16) == 4096
    assert lib.pa_default_split_tokens(1, 12, 2, 128, pa.PA_INT8) == 2048
    assert lib.pa_default_split_tokens(1, 12, 2, 128, pa.PA_BF16) == 2048
    assert lib.pa_default_split_tokens(2, 4, 1, 64, pa.PA_BF16) == 2048
    # it never depends on the batch: the same for any num_seqs / lengths, by signature


def test_workspace_size():
    lib = pa.lib()
    st = lib.pa_default_split_tokens(1, 16, 8, 128, pa.PA_BF16)
    # one piece covers the context: no workspace
    assert lib.pa_workspace_size(64, 1, 16, 8, 128, st, pa.PA_BF16, 0) == 0
    assert lib.pa_workspace_size(64, 1, 16, 8, 128, st + 1, pa.PA_BF16, 0) > 0
    n = lib.pa_workspace_size(8, 1, 12, 2, 128, 32768, pa.PA_INT8, 512)
    pieces = 32768 // 512
    rows = 8 * 12
    o = rows * pieces * 128 * 4
    lse = rows * pieces * 4
    rnd = lambda x: (x + 255) // 256 * 256
    assert n == rnd(o) + rnd(lse)
    # invalid sizes give 0
    assert lib.pa_workspace_size(8, 1, 12, 5, 128, 100, pa.PA_BF16, 0) == 0
    assert lib.pa_workspace_size(8, 1, 12, 2, 128, 100, pa.PA_BF16, 24) == 0


def _decode_status(**kw):
    lib = pa.lib()
    a = dict(out=None, q=None, k=None, v=None, ks=None, vs=None, bt=None, cl=None, N=4, Hq=2,
             Hkv=1, D=64, bs=16, NB=16, MB=4, ML=64, scale=0.125, qd=pa.PA_F32, kd=pa.PA_F32,
             split=0, ws=None, wsb=0, stream=None)
    a.update(kw)
    st = lib.pa_decode(a["out"], a["q"], a["k"], a["v"], a["ks"], a["vs"], a["bt"], a["cl"],
                       a["N"], a["Hq"], a["Hkv"], a["D"], a["bs"], a["NB"], a["MB"], a["ML"],
                       ctypes.c_float(a["scale"]), a["qd"], a["kd"], a["split"], a["ws"],
                       a["wsb"], a["stream"])
    return st, lib.pa_last_error().decode()


FAKE = 0x1000  # aligned non-null dummy address; never dereferenced on these paths


@pytest.mark.parametrize("kw,status", [
    (dict(Hq=3, Hkv=2), pa.PA_ERR_INVALID_ARG),
    (dict(D=96), pa.PA_ERR_UNSUPPORTED),
    (dict(bs=32), pa.PA_ERR_UNSUPPORTED),
    (dict(split=24), pa.PA_ERR_INVALID_ARG),
    (dict(split=4096 + 16), pa.PA_ERR_INVALID_ARG),
    (dict(ML=65), pa.PA_ERR_INVALID_ARG),
    (dict(qd=pa.PA_F32, kd=pa.PA_BF16), pa.PA_ERR_UNSUPPORTED),
    (dict(qd=7), pa.PA_ERR_INVALID_ARG),
    (dict(N=-1), pa.PA_ERR_INVALID_ARG),
    (dict(Hq=40, Hkv=1), pa.PA_ERR_INVALID_ARG),   # nulls reported before group size
    (dict(scale=float("nan")), pa.PA_ERR_INVALID_ARG),
    (dict(), pa.PA_ERR_INVALID_ARG),                # null pointers
])
def test_decode_rejects_invalid_arguments(kw, status):
    st, msg = _decode_status(**kw)
    assert st == status, msg
    assert msg


def test_decode_group_size_and_workspace_checked_before_launch():
    ptrs = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, cl=FAKE)
    st, msg = _decode_status(Hq=40, Hkv=1, **ptrs)
    assert st == pa.PA_ERR_UNSUPPORTED, msg
    # a long context needs a workspace: missing -> PA_ERR_WORKSPACE
    st, msg = _decode_status(ML=64, MB=4, split=16, **ptrs)
    assert st == pa.PA_ERR_WORKSPACE, msg
    # int8 needs scales
    st, msg = _decode_status(qd=pa.PA_BF16, kd=pa.PA_INT8, **ptrs)
    assert st == pa.PA_ERR_INVALID_ARG and "scale" in msg
    # zero sequences is a no-op
    st, msg = _decode_status(N=0)
    assert st == pa.PA_OK, msg


def test_empty_packed_calls_need_no_arrays():
    """Variable-length verify and prefill with no query rows read and write nothing:
    NULL q and out are accepted (an empty tensor has no storage); a negative or too
    large total is still rejected first."""
    lib = pa.lib()
    for name in ("pa_verify_varlen", "pa_prefill"):
        fn = getattr(lib, name)

        def call(total, out=None, q=None):
            args = [out, q, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, 3, total, 5, 4, 2, 128,
                    16, 64, 8, 128, ctypes.c_float(0.1), pa.PA_BF16, pa.PA_BF16]
            if name == "pa_verify_varlen":
                args += [0, None, 0]
            return fn(*args, None)

        assert call(0) == pa.PA_OK, lib.pa_last_error().decode()
        assert call(-1) == pa.PA_ERR_INVALID_ARG
        assert call(16) == pa.PA_ERR_INVALID_ARG            # > num_seqs * max_query_tokens
        assert call(4) == pa.PA_ERR_INVALID_ARG             # rows to compute, NULL arrays


def test_cache_write_rejects_invalid_arguments():
    lib = pa.lib()

    def call(**kw):
        a = dict(key=FAKE, value=FAKE, kc=FAKE, vc=FAKE, slots=FAKE, T=4, H=2, D=128, NB=8,
                 bs=16, dt=pa.PA_BF16)
        a.update(kw)
        return lib.pa_reshape_and_cache(a["key"], a["value"], a["kc"], a["vc"], a["slots"],
                                        a["T"], a["H"], a["D"], a["NB"], a["bs"], a["dt"], None)

    assert call(D=80) == pa.PA_ERR_UNSUPPORTED
    assert call(bs=8) == pa.PA_ERR_UNSUPPORTED
    assert call(dt=9) == pa.PA_ERR_INVALID_ARG
    assert call(key=None) == pa.PA_ERR_INVALID_ARG
    assert call(key=FAKE + 4) == pa.PA_ERR_INVALID_ARG
    assert call(T=-1) == pa.PA_ERR_INVALID_ARG
    assert call(T=0, key=None) == pa.PA_OK


def test_probe_library_exports_and_rejects_bad_arguments():
    """The bandwidth-probe library loads, exports what include/pa_probe.h declares and
    rejects invalid arguments before launching anything."""
    from paged_kv_gqa_pa_amd import _probe
    src = open(os.path.join(ROOT, "include", "pa_probe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(pa_probe_\w+)\s*\(", src, flags=re.M)))
    assert names == sorted(_probe.EXPORTED)
    lib = _probe.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert lib.pa_probe_stream_read(None, 1024, 0, None, None) == -1
    assert lib.pa_probe_stream_read(ctypes.c_void_p(4096), 1000, 0, ctypes.c_void_p(4096), None) == -1
    assert b"multiple of 16" in lib.pa_probe_last_error()
    d = ctypes.c_void_p(4096)
    # row_bytes 64 is not built
    assert lib.pa_probe_tile_read(d, d, d, d, 1, 1, 4, 4, 64, 16, 64, 4, d, None) == -1
    # waves 16 is not built
    assert lib.pa_probe_tile_read(d, d, d, d, 1, 1, 4, 4, 256, 16, 64, 16, d, None) == -1


def test_plan_size_and_invalid_arguments():
    """Plan sizes follow the layout (16 header ints, one row per (sequence, piece) unit of
    4 + split/16 rounded up to 4 ints); invalid calls are refused before any launch."""
    lib = pa.lib()
    # batch-64 decode: one 512-token piece per sequence -> 64 rows of 4 + 32 ints
    assert lib.pa_plan_size(64, 1, 16, 8, 128, 512, pa.PA_BF16, 0) == 4 * (16 + 64 * 36)
    # 8 sequences of 32768 in 2048-token pieces (int8 default) -> 128 rows of 4 + 128 ints
    assert lib.pa_plan_size(8, 1, 12, 2, 128, 32768, pa.PA_INT8, 0) == 4 * (16 + 128 * 132)
    # split 48 -> 3 entries, padded to 4
    assert lib.pa_plan_size(2, 1, 2, 1, 64, 100, pa.PA_F32, 48) == 4 * (16 + 2 * 3 * 8)
    # more than 8192 units, or invalid sizes: 0
    assert lib.pa_plan_size(9000, 1, 2, 1, 64, 16, pa.PA_F32, 0) == 0
    assert lib.pa_plan_size(4, 1, 3, 2, 64, 16, pa.PA_F32, 0) == 0
    d = ctypes.c_void_p(FAKE)
    need = lib.pa_plan_size(4, 1, 2, 1, 64, 64, pa.PA_F32, 16)
    # plan buffer too small / missing
    assert lib.pa_plan(d, d, 4, 1, 2, 1, 64, 4, 64, pa.PA_F32, 16, d, need - 4, None) == pa.PA_ERR_INVALID_ARG
    assert lib.pa_plan(d, d, 4, 1, 2, 1, 64, 4, 64, pa.PA_F32, 16, None, need, None) == pa.PA_ERR_INVALID_ARG
    # table too narrow for max_context_len
    assert lib.pa_plan(d, d, 4, 1, 2, 1, 64, 3, 64, pa.PA_F32, 16, d, need, None) == pa.PA_ERR_INVALID_ARG
    # null tables
    assert lib.pa_plan(None, d, 4, 1, 2, 1, 64, 4, 64, pa.PA_F32, 16, d, need, None) == pa.PA_ERR_INVALID_ARG
    # planned decode with a null plan
    ptrs = [d] * 8
    st = lib.pa_decode_planned(*ptrs, 4, 2, 1, 64, 16, 16, 4, 64, ctypes.c_float(0.125),
                               pa.PA_F32, pa.PA_F32, 16, d, 1 << 20, None, need, None)
    assert st == pa.PA_ERR_INVALID_ARG
    # planned decode with a plan smaller than the call's sizes need
    st = lib.pa_decode_planned(*ptrs, 4, 2, 1, 64, 16, 16, 4, 64, ctypes.c_float(0.125),
                               pa.PA_F32, pa.PA_F32, 16, d, 1 << 20, d, need - 16, None)
    assert st == pa.PA_ERR_INVALID_ARG and b"work plan" in lib.pa_last_error()


def test_prefill_plan_size_and_invalid_arguments():
    lib = pa.lib()
    # 16 sequences x 512 tokens, 16/8 heads: 1024 rows per sequence in tiles of the workgroup's rows
    n = lib.pa_prefill_plan_size(16, 512, 16, 8)
    assert n > 0 and (n // 4 - 16) % 8 == 0
    units = (n // 4 - 16) // 8
    assert units % 16 == 0 and 1024 % (units // 16) == 0
    assert lib.pa_prefill_plan_size(16, 512, 15, 8) == 0        # q_heads not a multiple
    assert lib.pa_prefill_plan_size(100000, 512, 16, 8) == 0    # too many units
    d = ctypes.c_void_p(FAKE)
    assert lib.pa_prefill_plan(d, d, 16, 8192, 512, 16, 8, 64, d, n - 4, None) == pa.PA_ERR_INVALID_ARG
    assert lib.pa_prefill_plan(d, d, 16, 9000, 512, 16, 8, 64, d, n, None) == pa.PA_ERR_INVALID_ARG
    assert lib.pa_prefill_plan(None, d, 16, 8192, 512, 16, 8, 64, d, n, None) == pa.PA_ERR_INVALID_ARG
