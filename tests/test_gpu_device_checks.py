"""The debug library (libpa_debug.so, device-side precondition checks).

Clean calls leave its status word at 0 and give the release library's bits;
each kind of violated precondition sets its bit.  Every violation used here is
one the kernels clamp (table entries into the pool, lengths to the table,
slots skipped, offsets clamped), so no access leaves the buffers: the checks
only report what the release build silently tolerates.
"""
import contextlib
import os

import numpy as np
import pytest
import torch

import oracle
from paged_kv_gqa_pa_amd import _lib as pa
from tests.gpu_util import TOL, DevCase, dev, max_abs_err
from tests.test_gpu_decode import _random_case
from tests.test_gpu_verify import _random_verify_case

pytestmark = pytest.mark.gpu

DEBUG_LIB = os.path.join(os.path.dirname(pa.LIB_PATH), "libpa_debug.so")


def _say(*a):
    print("[case]", *a, flush=True)


@contextlib.contextmanager
def _library(path):
    """Route the binding's calls to the library at `path` for the block."""
    saved_lib, saved_path = pa._lib, pa.LIB_PATH
    pa._lib, pa.LIB_PATH = None, path
    try:
        pa._load()
        yield
    finally:
        pa._lib, pa.LIB_PATH = saved_lib, saved_path


def _status():
    torch.cuda.synchronize()
    return pa.device_check_status(clear=True)


def test_release_library_reports_no_checks():
    with _library(os.path.join(os.path.dirname(pa.LIB_PATH), "libpa.so")):
        with pytest.raises(pa.PAError) as ei:
            pa.device_check_status()
        assert ei.value.status == pa.PA_ERR_UNSUPPORTED


def test_clean_calls_report_nothing_and_match_release_bits():
    _say("debug library: clean decode / verify / prefill / cache write")
    rng = np.random.default_rng(61)
    case = _random_case(rng, [1, 17, 300, 700], Hkv=2, G=2, D=128, tag="bf16", poison=True)
    vcase = _random_verify_case(rng, [9, 300, 517], Hkv=2, G=6, D=128, T=5, poison=True,
                                kv="int8")
    outs = {}
    for name in ("libpa.so", "libpa_debug.so"):
        with _library(os.path.join(os.path.dirname(pa.LIB_PATH), name)):
            dc, dv = DevCase(case), DevCase(vcase)
            if name == "libpa_debug.so":
                _status()
            o1 = torch.empty_like(dc.q)
            pa.decode(o1, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens,
                      case.scale, case.max_context_len, split_tokens=64)
            o2 = torch.empty_like(dv.q)
            pa.verify(o2, dv.q, dv.k_cache, dv.v_cache, dv.block_tables, dv.context_lens,
                      vcase.scale, vcase.max_context_len, dv.k_scale, dv.v_scale, split_tokens=64)
            qp = dv.q.reshape(-1, *dv.q.shape[2:])
            o3 = torch.empty_like(qp)
            qs = dev((np.arange(4) * 5).astype(np.int32))
            pa.prefill(o3, qp, dv.k_cache, dv.v_cache, dv.block_tables, dv.context_lens, qs,
                       vcase.scale, 5, dv.k_scale, dv.v_scale)
            torch.cuda.synchronize()
            outs[name] = [o.view(torch.int16).clone() for o in (o1, o2, o3)]
            if name == "libpa_debug.so":
                assert _status() == 0
    for a, b in zip(outs["libpa.so"], outs["libpa_debug.so"]):
        assert torch.equal(a, b)


def _decode_case(rng):
    case = _random_case(rng, [20, 300, 45], Hkv=2, G=2, D=128, tag="bf16", nb=64)
    return case, DevCase(case)


def test_table_entry_out_of_range_is_reported():
    _say("debug library: table entry out of range")
    rng = np.random.default_rng(62)
    case, dc = _decode_case(rng)
    with _library(DEBUG_LIB):
        _status()
        bt = case.block_tables.copy()
        bt[1, 3] = case.spec.num_blocks + 5          # read: position 48..63 < 300
        out = torch.empty_like(dc.q)
        pa.decode(out, dc.q, dc.k_cache, dc.v_cache, dev(bt), dc.context_lens, case.scale,
                  case.max_context_len)
        flags = _status()
        assert flags & pa.PA_CHECK_TABLE_ENTRY, flags
        # the sequences whose tables are valid are unaffected
        want = oracle.decode(case.q, case.k_cache, case.v_cache, case.block_tables,
                             case.context_lens, case.scale, "bf16", "bf16")
        got = out.double().cpu().numpy()
        assert np.isfinite(got).all()
        assert max_abs_err(out[[0, 2]], want[[0, 2]], TOL["bf16"]) < TOL["bf16"]
        # an entry past the context (never read) is not reported
        bt2 = case.block_tables.copy()
        bt2[0, 5] = 10 ** 6
        pa.decode(out, dc.q, dc.k_cache, dc.v_cache, dev(bt2), dc.context_lens, case.scale,
                  case.max_context_len)
        assert _status() == 0


def test_context_lengths_are_reported():
    _say("debug library: context lengths past the table and past max_context_len")
    rng = np.random.default_rng(63)
    case, dc = _decode_case(rng)
    with _library(DEBUG_LIB):
        _status()
        out = torch.empty_like(dc.q)
        lens = case.context_lens.copy()
        lens[2] = case.block_tables.shape[1] * 16 + 40          # past the table
        pa.decode(out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dev(lens), case.scale,
                  case.max_context_len)
        assert _status() & pa.PA_CHECK_CONTEXT_TABLE
        # within the table but past max_context_len: positions past the grid's pieces
        pa.decode(out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens,
                  case.scale, 128, split_tokens=64)
        flags = _status()
        assert flags & pa.PA_CHECK_CONTEXT_MAX and not flags & pa.PA_CHECK_CONTEXT_TABLE, flags


def test_cache_slot_out_of_range_is_reported():
    _say("debug library: cache slot out of range")
    rng = np.random.default_rng(64)
    case, dc = _decode_case(rng)
    with _library(DEBUG_LIB):
        _status()
        nb = case.spec.num_blocks
        key = torch.randn((3, 2, 128), device="cuda").bfloat16()
        slots = dev(np.array([5, nb * 16 + 3, -1], np.int64))
        before = dc.k_cache.clone()
        pa.reshape_and_cache(key, key, dc.k_cache, dc.v_cache, slots)
        assert _status() & pa.PA_CHECK_SLOT
        # only slot 5 was written
        diff = (dc.k_cache.view(torch.int16) != before.view(torch.int16)).reshape(2, nb * 16, 128)
        assert diff.any(dim=(0, 2)).nonzero().flatten().tolist() == [5]


def test_query_offsets_are_reported():
    _say("debug library: decreasing query offsets")
    rng = np.random.default_rng(65)
    vcase = _random_verify_case(rng, [30, 40, 50], Hkv=2, G=2, D=128, T=4, poison=True)
    dv = DevCase(vcase)
    qp = dv.q.reshape(-1, *dv.q.shape[2:])
    with _library(DEBUG_LIB):
        _status()
        out = torch.empty_like(qp)
        qs = dev(np.array([0, 4, 2, 12], np.int32))      # sequence 1 ends before it starts
        pa.verify_varlen(out, qp, dv.k_cache, dv.v_cache, dv.block_tables, dv.context_lens, qs,
                         vcase.scale, vcase.max_context_len, 4)
        assert _status() & pa.PA_CHECK_QUERY_START
        pa.prefill(out, qp, dv.k_cache, dv.v_cache, dv.block_tables, dv.context_lens, qs,
                   vcase.scale, 4)
        assert _status() & pa.PA_CHECK_QUERY_START


def test_append_quant_slot_out_of_range_is_reported():
    _say("debug library: requantizing append, slot out of range")
    rng = np.random.default_rng(66)
    case = _random_case(rng, [20, 40], Hkv=2, G=6, D=128, tag="int8")
    dc = DevCase(case)
    nb = case.spec.num_blocks
    new = torch.randn((2, 2, 128), device="cuda").bfloat16()
    good = int(case.block_tables[0, 1]) * 16 + 3          # position 19 of sequence 0
    slots = dev(np.array([good, nb * 16 + 5], np.int64))
    with _library(DEBUG_LIB):
        _status()
        before = dc.k_scale.clone()
        out = torch.empty_like(dc.q)
        pa.decode_append_quant(out, dc.q, new, new, dc.k_cache, dc.v_cache, dc.k_scale, dc.v_scale,
                               slots, dc.block_tables, dc.context_lens, case.scale,
                               case.max_context_len)
        assert _status() & pa.PA_CHECK_SLOT
        # only sequence 0's block has a new scale
        changed = (dc.k_scale != before).nonzero().tolist()
        assert all(blk == good // 16 for _, blk in changed), changed
