"""GPU parity of pa_verify_varlen (per-sequence query counts over packed rows)."""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_gqa_pa_amd import _lib as pa
from paged_kv_gqa_pa_amd import workloads as wl
from tests.gpu_util import TOL, DevCase, dev, host_bits, max_abs_err
from tests.test_gpu_verify import EDGE, _random_verify_case

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _packed(case, counts):
    """Rows 0..T_b-1 of each sequence's q, packed; context lengths moved so that the
    sequence's T_b new tokens are its last positions (the rest of the cache is unchanged)."""
    T = case.q.shape[1]
    counts = np.asarray(counts, np.int64)
    qs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = [case.q[b, :int(c)] for b, c in enumerate(counts)]
    D, Hq = case.q.shape[3], case.q.shape[2]
    qp = np.concatenate(rows, axis=0) if qs[-1] else np.zeros((0, Hq, D), case.q.dtype)
    lens = np.maximum(case.context_lens.astype(np.int64) - T + counts, 0).astype(np.int32)
    return np.ascontiguousarray(qp), qs, lens


def _run(case, dc, qp, qs, lens, T, split=0, out=None):
    q = dev(qp)
    out = torch.empty_like(q) if out is None else out
    pa.verify_varlen(out, q, dc.k_cache, dc.v_cache, dc.block_tables, dev(lens), dev(qs),
                     case.scale, int(case.max_context_len), T, dc.k_scale, dc.v_scale,
                     split_tokens=split)
    torch.cuda.synchronize()
    return out


def _want(case, qp, qs, lens):
    return oracle.verify_varlen(qp, case.k_cache, case.v_cache, case.block_tables, lens, qs,
                                case.scale, "bf16", case.spec.kv_dtype, case.k_scale, case.v_scale)


@pytest.mark.parametrize("kv", ["bf16", "int8"])
@pytest.mark.parametrize("G,T", [(2, 5), (3, 5), (8, 2), (1, 16), (16, 1), (6, 5), (8, 5), (16, 4)])
@pytest.mark.parametrize("D", [64, 128])
def test_varlen_edges(G, T, D, kv):
    """Counts 0..T per sequence (with lengths from 0 up), poisoned cache tails, one
    piece and many pieces (the merge over packed rows)."""
    _say("verify varlen edges", kv, "G", G, "T", T, "D", D)
    rng = np.random.default_rng(2000 + 10 * G + T + D)
    case = _random_verify_case(rng, EDGE, Hkv=2, G=G, D=D, T=T, poison=True, kv=kv)
    dc = DevCase(case)
    counts = rng.integers(0, T + 1, size=len(EDGE))
    counts[:3] = [0, T, 1]
    qp, qs, lens = _packed(case, counts)
    want = _want(case, qp, qs, lens)
    for split in (0, 32):
        err = max_abs_err(_run(case, dc, qp, qs, lens, T, split), want)
        assert err < TOL[kv], (split, err)


@pytest.mark.parametrize("kv", ["bf16", "int8"])
def test_varlen_equal_counts_is_verify_bitwise(kv):
    """Every sequence with T tokens: the same bits as pa_verify."""
    _say("verify varlen == verify", kv)
    rng = np.random.default_rng(11)
    T = 5
    case = _random_verify_case(rng, [40, 300, 517, 5, 1029], Hkv=2, G=3, D=128, T=T, kv=kv)
    dc = DevCase(case)
    qp, qs, lens = _packed(case, [T] * 5)
    for split in (0, 64):
        out = torch.empty_like(dc.q)
        pa.verify(out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, case.scale,
                  case.max_context_len, dc.k_scale, dc.v_scale, split_tokens=split)
        got = _run(case, dc, qp, qs, lens, T, split)
        assert host_bits(got).tobytes() == host_bits(out.reshape(-1, *out.shape[2:])).tobytes()


def test_varlen_speculative_workload():
    """The 64-sequence speculative workload with 1..5 tokens per sequence."""
    _say("verify varlen spec_verify_bf16, counts 1..5")
    case = wl.build_case("spec_verify_bf16", poison=True)
    dc = DevCase(case)
    pa.reshape_and_cache(dc.new_k, dc.new_v, dc.k_cache, dc.v_cache, dc.slot_mapping)
    torch.cuda.synchronize()
    case.k_cache, case.v_cache = oracle.reshape_and_cache(case.new_k, case.new_v, case.k_cache,
                                                          case.v_cache, case.slot_mapping)
    rng = np.random.default_rng(5)
    counts = rng.integers(1, 6, size=case.spec.num_seqs)
    qp, qs, lens = _packed(case, counts)
    err = max_abs_err(_run(case, dc, qp, qs, lens, 5), _want(case, qp, qs, lens))
    assert err < TOL["bf16"], err


def test_varlen_many_sequences_and_untouched_rows():
    """70 sequences (the merge looks the sequence up across two chunks of offsets); rows of
    out past the last sequence are not written."""
    _say("verify varlen 70 sequences split 64")
    rng = np.random.default_rng(70)
    T = 4
    lens = rng.integers(0, 400, size=70)
    case = _random_verify_case(rng, lens, Hkv=2, G=2, D=64, T=T)
    dc = DevCase(case)
    counts = rng.integers(0, T + 1, size=70)
    qp, qs, lens = _packed(case, counts)
    extra = 3
    qx = np.concatenate([qp, np.zeros((extra,) + qp.shape[1:], qp.dtype)])
    out = torch.full((qx.shape[0],) + qx.shape[1:], 7.0, dtype=torch.bfloat16, device="cuda")
    q = dev(qx)
    pa.verify_varlen(out, q, dc.k_cache, dc.v_cache, dc.block_tables, dev(lens), dev(qs),
                     case.scale, int(case.max_context_len), T, split_tokens=64)
    torch.cuda.synchronize()
    want = _want(case, qp, qs, lens)
    assert max_abs_err(out[:qp.shape[0]], want) < TOL["bf16"]
    assert (out[qp.shape[0]:].float() == 7.0).all()


def test_varlen_invalid_arguments():
    rng = np.random.default_rng(4)
    case = _random_verify_case(rng, [20, 30], Hkv=1, G=4, D=128, T=4)
    dc = DevCase(case)
    qp, qs, lens = _packed(case, [4, 4])
    case96 = _random_verify_case(rng, [20, 30], Hkv=1, G=4, D=96, T=4)
    q96, qs96, lens96 = _packed(case96, [4, 4])
    with pytest.raises(pa.PAError) as ei:      # head_dim 96 is not built
        _run(case96, DevCase(case96), q96, qs96, lens96, 4)
    assert ei.value.status == pa.PA_ERR_UNSUPPORTED
    # a larger max_query_tokens than any sequence uses (5 x 4 heads = 20 rows: two row
    # tiles) gives the same rows
    assert max_abs_err(_run(case, dc, qp, qs, lens, 5), _want(case, qp, qs, lens)) < TOL["bf16"]
    with pytest.raises(pa.PAError) as ei:      # 8 packed rows > 2 sequences x 3 tokens
        _run(case, dc, qp, qs, lens, 3)
    assert ei.value.status == pa.PA_ERR_INVALID_ARG
