"""Visibility, not value, decides which keys count, on the GPU as in the oracle.

A NaN in a key row at a visible position makes every row that sees it NaN; rows
that do not see it (verify and prefill rows before it, other sequences) keep
their values.  The kernels mask positions by index only, so a kernel that
skipped non-finite scores would fail here.
"""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_gqa_pa_amd import _lib as pa
from tests.gpu_util import TOL, DevCase, dev, host_f64, max_abs_err
from tests.test_gpu_decode import _random_case
from tests.test_gpu_verify import _random_verify_case

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _nan_key(case, b, pos):
    """NaN in dimension 3 of K at position pos of sequence b, every KV head."""
    phys = case.block_tables[b, pos // 16]
    row = case.k_cache[:, phys, pos % 16]
    row[:, 3] = np.array(np.nan, np.float32).astype(row.dtype) if row.dtype == np.float32 \
        else np.uint16(0x7FC0)


def _check(out, want, tol):
    got = host_f64(out)
    nan_want = np.isnan(want)
    assert nan_want.any(), "the case must reach a NaN"
    assert np.array_equal(np.isnan(got), nan_want), "NaN where the oracle has NaN, nowhere else"
    err = max_abs_err(np.where(nan_want, 0.0, got), np.where(nan_want, 0.0, want), tol)
    assert err < tol, err


@pytest.mark.parametrize("tag,G", [("f32", 2), ("bf16", 2), ("bf16", 6)])
@pytest.mark.parametrize("split", [0, 64])
def test_decode_visible_nan_key(tag, G, split):
    _say("decode visible NaN key", tag, "G", G, "split", split)
    rng = np.random.default_rng(900 + G)
    case = _random_case(rng, [5, 100, 333, 700], Hkv=2, G=G, D=128, tag=tag, poison=True)
    _nan_key(case, 1, 37)
    _nan_key(case, 3, 699)    # the last position
    dc = DevCase(case)
    out = torch.empty_like(dc.q)
    pa.decode(out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, case.scale,
              case.max_context_len, split_tokens=split)
    torch.cuda.synchronize()
    want = oracle.decode(case.q, case.k_cache, case.v_cache, case.block_tables,
                         case.context_lens, case.scale, case.spec.q_dtype, tag)
    assert np.isnan(want[1]).all() and np.isnan(want[3]).all() and np.isfinite(want[[0, 2]]).all()
    _check(out, want, TOL[tag])


@pytest.mark.parametrize("split", [0, 64])
def test_verify_visible_nan_key(split):
    """Key L - T + 2 is NaN: tokens 2.. of that sequence see it, tokens 0 and 1 do not."""
    _say("verify visible NaN key split", split)
    rng = np.random.default_rng(910)
    T = 5
    case = _random_verify_case(rng, [40, 300, 517], Hkv=2, G=2, D=128, T=T, poison=True)
    _nan_key(case, 1, 300 - T + 2)
    dc = DevCase(case)
    out = torch.empty_like(dc.q)
    pa.verify(out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, case.scale,
              case.max_context_len, split_tokens=split)
    torch.cuda.synchronize()
    want = oracle.verify(case.q, case.k_cache, case.v_cache, case.block_tables,
                         case.context_lens, case.scale, "bf16", "bf16")
    assert np.isnan(want[1, 2:]).all() and np.isfinite(want[1, :2]).all()
    _check(out, want, TOL["bf16"])


def test_prefill_visible_nan_key():
    """A chunk of 40 tokens: rows from the NaN key's own token on are NaN."""
    _say("prefill visible NaN key")
    rng = np.random.default_rng(920)
    T = 40
    case = _random_verify_case(rng, [90, 300], Hkv=2, G=2, D=128, T=T, poison=True)
    _nan_key(case, 1, 300 - T + 10)
    qp = np.ascontiguousarray(case.q.reshape(-1, *case.q.shape[2:]))
    qs = np.array([0, T, 2 * T], np.int32)
    dc = DevCase(case)
    q = dev(qp)
    out = torch.empty_like(q)
    pa.prefill(out, q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, dev(qs),
               case.scale, T)
    torch.cuda.synchronize()
    want = oracle.verify_varlen(qp, case.k_cache, case.v_cache, case.block_tables,
                                case.context_lens, qs, case.scale, "bf16", "bf16")
    assert np.isnan(want[T + 10:]).all() and np.isfinite(want[:T + 10]).all()
    _check(out, want, TOL["bf16"])
