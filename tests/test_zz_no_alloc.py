"""pa_decode_noalloc (split-K partials in the library's fixed device array) against
pa_decode with a caller workspace: the same kernels, so the same bits.

Two calls in a row on one GPU, the second with a smaller input, each compared
with pa_decode on the same arguments and with the oracle; sizes whose partials
do not fit the array are refused before anything is launched.
"""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_gqa_pa_amd import _lib as pa
from paged_kv_gqa_pa_amd import workloads as wl
from tests.gpu_util import TOL, DevCase, dev, max_abs_err

pytestmark = pytest.mark.gpu

SCRATCH = 16 << 20   # PA_NOALLOC_SCRATCH_BYTES in include/pa.h


def _say(*a):
    print("[case]", *a, flush=True)


def _both(dc, sel, split, max_len):
    """(pa_decode_noalloc output, pa_decode output) for sequences `sel`."""
    case = dc.case
    q = dc.q[sel].contiguous()
    bt, cl = dc.block_tables[sel].contiguous(), dc.context_lens[sel].contiguous()
    need = pa.workspace_size(q.shape[0], 1, q.shape[1], dc.k_cache.shape[0],
                             dc.k_cache.shape[3], max_len, dc.k_cache.dtype, split)
    assert 0 < need <= SCRATCH, need   # the scratch array is really used
    a = torch.full_like(q, float("nan"))
    pa.decode_noalloc(a, q, dc.k_cache, dc.v_cache, bt, cl, case.scale, max_len, dc.k_scale,
                      dc.v_scale, split_tokens=split)
    b = torch.full_like(q, float("nan"))
    pa.decode(b, q, dc.k_cache, dc.v_cache, bt, cl, case.scale, max_len, dc.k_scale, dc.v_scale,
              split_tokens=split)
    torch.cuda.synchronize()
    return a, b


def _oracle(case, sel):
    return oracle.decode(case.q[sel], case.k_cache, case.v_cache, case.block_tables[sel],
                         case.context_lens[sel], case.scale, case.spec.q_dtype,
                         case.spec.kv_dtype, case.k_scale, case.v_scale)


@pytest.mark.parametrize("name,split,first,second", [
    ("qwen2_1p5b_bf16", 64, slice(0, 32), slice(3, 8)),      # matrix-core kernel, G = 6
    ("batch64_28layer_bf16", 128, slice(0, 64), slice(10, 13)),  # vector-ALU kernel, G = 2
    ("long_ctx_int8", 2048, slice(0, 8), slice(2, 4)),        # int8, 16 pieces per sequence
])
def test_noalloc_equals_decode_two_calls(name, split, first, second):
    case = wl.build_case(name, poison=True)
    dc = DevCase(case)
    for sel in (first, second):
        _say("decode_noalloc", name, "split", split, "seqs", sel.start, sel.stop)
        a, b = _both(dc, sel, split, case.max_context_len)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "same bits as pa_decode"
        tol = TOL[case.spec.kv_dtype]
        assert max_abs_err(a, _oracle(case, sel), tol) < tol


def test_noalloc_refuses_oversized_partials():
    """64 sequences x 16 heads x 256 pieces of partials (> 16 MiB): refused on the host."""
    _say("decode_noalloc oversize")
    case = wl.build_case("tiny_fp32")
    dc = DevCase(case)
    q = torch.zeros((64, 16, 64), dtype=torch.float32, device="cuda")
    kc = torch.zeros((8, 16, 16, 64), dtype=torch.float32, device="cuda")
    bt = torch.zeros((64, 2048), dtype=torch.int32, device="cuda")
    cl = torch.zeros(64, dtype=torch.int32, device="cuda")
    need = pa.workspace_size(64, 1, 16, 8, 64, 32768, torch.float32, 128)
    assert need > SCRATCH
    out = torch.empty_like(q)
    with pytest.raises(pa.PAError) as ei:
        pa.decode_noalloc(out, q, kc, kc, bt, cl, 0.125, 32768, split_tokens=128)
    assert ei.value.status == pa.PA_ERR_WORKSPACE
    # the same library state still serves a fitting call
    a, b = _both(dc, slice(0, 4), 16, case.max_context_len)
    assert torch.equal(a, b)
