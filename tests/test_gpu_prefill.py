"""GPU parity of pa_prefill (chunked prefill over the paged cache) against the oracle.

The oracle is the variable-length verify definition (sequence b's T_b new tokens
are its last positions; token t sees 0 .. L_b - T_b + t) at prefill sizes.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from paged_kv_gqa_pa_amd import _lib as pa
from tests.gpu_util import TOL, DevCase, dev, max_abs_err
from tests.test_gpu_verify import _random_verify_case
from tests.test_gpu_verify_varlen import _packed

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _pack(case, counts, lens):
    """The first counts[b] query tokens of each sequence, packed, with context lengths lens
    (at most the lengths the case's cache holds)."""
    counts = np.asarray(counts, np.int64)
    qs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    qp = np.concatenate([case.q[b, :int(c)] for b, c in enumerate(counts)], axis=0)
    lens = np.asarray(lens, np.int32)
    assert (lens <= case.context_lens).all()
    return np.ascontiguousarray(qp), qs, lens


def _prefill(case, dc, qp, qs, lens, T, out=None):
    q = dev(qp)
    out = torch.empty_like(q) if out is None else out
    pa.prefill(out, q, dc.k_cache, dc.v_cache, dc.block_tables, dev(lens), dev(qs), case.scale, T,
               dc.k_scale, dc.v_scale)
    torch.cuda.synchronize()
    return out


def _want(case, qp, qs, lens):
    return oracle.verify_varlen(qp, case.k_cache, case.v_cache, case.block_tables, lens, qs,
                                case.scale, "bf16", case.spec.kv_dtype, case.k_scale, case.v_scale)


LENS = [0, 1, 15, 16, 17, 64, 65, 130, 333, 700]


@pytest.mark.parametrize("kv", ["bf16", "int8"])
@pytest.mark.parametrize("G", [1, 2, 6, 16])
@pytest.mark.parametrize("D", [64, 128])
def test_prefill_edges(G, D, kv):
    """Counts from 0 to past the context, tile boundaries of 64 rows, poisoned tails."""
    _say("prefill edges", kv, "G", G, "D", D)
    rng = np.random.default_rng(3000 + G + D)
    T = 90
    case = _random_verify_case(rng, LENS, Hkv=2, G=G, D=D, T=T, poison=True, kv=kv)
    dc = DevCase(case)
    counts = [0, 3, 15, 16, 17, 64, 65, 90, 33, 90]    # sequence 1: 3 tokens, 1 position
    qp, qs, lens = _pack(case, counts, LENS)
    err = max_abs_err(_prefill(case, dc, qp, qs, lens, T), _want(case, qp, qs, lens))
    assert err < TOL[kv], err


@pytest.mark.parametrize("kv", ["bf16", "int8"])
@pytest.mark.parametrize("scale", [-0.3, -1.0 / np.sqrt(128), 0.0, 1.5])
def test_prefill_scales(scale, kv):
    """Negative, zero and large softmax scales: the bf16 path carries a negative scale
    in q's sign and takes the row maximum over the raw scores; a zero scale gives the
    mean of the visible V rows; a large one makes the running maximum jump (rescales)."""
    _say("prefill scale", scale, kv)
    rng = np.random.default_rng(4100)
    T = 70
    case = dataclasses.replace(
        _random_verify_case(rng, [90, 300, 80, 700], Hkv=2, G=2, D=128, T=T, poison=True, kv=kv),
        scale=float(scale))
    dc = DevCase(case)
    qp, qs, lens = _packed(case, [70, 5, 17, 33])
    err = max_abs_err(_prefill(case, dc, qp, qs, lens, T), _want(case, qp, qs, lens))
    assert err < TOL[kv], err


@pytest.mark.parametrize("kv", ["bf16", "int8"])
def test_prefill_agrees_with_varlen_verify(kv):
    """Where verify's row limit allows (T_b * G <= 16), both kernels meet the oracle and
    each other."""
    _say("prefill vs verify_varlen", kv)
    rng = np.random.default_rng(9)
    T, G = 5, 3
    case = _random_verify_case(rng, [40, 300, 517, 5, 1029], Hkv=2, G=G, D=128, T=T, kv=kv)
    dc = DevCase(case)
    qp, qs, lens = _packed(case, [5, 1, 0, 4, 5])
    got = _prefill(case, dc, qp, qs, lens, T)
    ver = torch.empty_like(got)
    pa.verify_varlen(ver, dev(qp), dc.k_cache, dc.v_cache, dc.block_tables, dev(lens), dev(qs),
                     case.scale, int(case.max_context_len), T, dc.k_scale, dc.v_scale)
    torch.cuda.synchronize()
    want = _want(case, qp, qs, lens)
    assert max_abs_err(got, want) < TOL[kv]
    assert max_abs_err(ver, want) < TOL[kv]


def test_prefill_chunk_of_512_tokens():
    """Four sequences, a 512-token chunk after 0..1500 prior positions, 16 query / 8 KV
    heads, head_dim 128, bf16."""
    _say("prefill 4 x 512 tokens, 16/8 heads, D=128")
    rng = np.random.default_rng(512)
    T = 512
    prior = np.array([0, 100, 777, 1500])
    case = _random_verify_case(rng, prior + T, Hkv=8, G=2, D=128, T=T, poison=True)
    dc = DevCase(case)
    qp, qs, lens = _packed(case, [T] * 4)
    err = max_abs_err(_prefill(case, dc, qp, qs, lens, T), _want(case, qp, qs, lens))
    assert err < TOL["bf16"], err


def test_prefill_untouched_rows_and_invalid_arguments():
    _say("prefill untouched rows, invalid arguments")
    rng = np.random.default_rng(4)
    T = 20
    case = _random_verify_case(rng, [50, 30, 200], Hkv=1, G=4, D=64, T=T)
    dc = DevCase(case)
    qp, qs, lens = _packed(case, [20, 0, 7])
    qx = np.concatenate([qp, np.zeros((2,) + qp.shape[1:], qp.dtype)])
    out = torch.full((qx.shape[0],) + qx.shape[1:], 5.0, dtype=torch.bfloat16, device="cuda")
    q = dev(qx)
    pa.prefill(out, q, dc.k_cache, dc.v_cache, dc.block_tables, dev(lens), dev(qs), case.scale, T)
    torch.cuda.synchronize()
    assert max_abs_err(out[:qp.shape[0]], _want(case, qp, qs, lens)) < TOL["bf16"]
    assert (out[qp.shape[0]:].float() == 5.0).all()
    with pytest.raises(pa.PAError) as ei:       # 29 packed rows > 3 sequences x 9 tokens
        pa.prefill(out, q, dc.k_cache, dc.v_cache, dc.block_tables, dev(lens), dev(qs),
                   case.scale, 9)
    assert ei.value.status == pa.PA_ERR_INVALID_ARG
    q32 = q.float()
    with pytest.raises(pa.PAError) as ei:       # fp32 query: not built
        pa.prefill(q32.clone(), q32, dc.k_cache.float(), dc.v_cache.float(), dc.block_tables,
                   dev(lens), dev(qs), case.scale, T)
    assert ei.value.status == pa.PA_ERR_UNSUPPORTED


def _prefill_plan(case, dc, qs, lens, T):
    sp = case.spec
    return pa.make_prefill_plan(dev(lens), dev(qs), int(qs[-1]), T, sp.q_heads, sp.kv_heads,
                                case.block_tables.shape[1])


@pytest.mark.parametrize("kv", ["bf16", "int8"])
@pytest.mark.parametrize("G", [1, 2, 6])
def test_planned_prefill_equals_unplanned_bitwise(G, kv):
    """The prefill plan only reorders the start of row tiles: same bits, and the oracle."""
    _say("planned prefill", kv, "G", G)
    rng = np.random.default_rng(4000 + G)
    T = 90
    case = _random_verify_case(rng, LENS, Hkv=2, G=G, D=128, T=T, poison=True, kv=kv)
    dc = DevCase(case)
    counts = [0, 3, 15, 16, 17, 64, 65, 90, 33, 90]
    qp, qs, lens = _pack(case, counts, LENS)
    base = _prefill(case, dc, qp, qs, lens, T)
    plan = _prefill_plan(case, dc, qs, lens, T)
    got = torch.empty_like(base)
    pa.prefill(got, dev(qp), dc.k_cache, dc.v_cache, dc.block_tables, dev(lens), dev(qs),
               case.scale, T, dc.k_scale, dc.v_scale, plan=plan)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), base.view(torch.int16))
    assert max_abs_err(got, _want(case, qp, qs, lens)) < TOL[kv]


def test_prefill_plan_contents_exact():
    """One row per (sequence, row tile) unit with its offsets and lengths, ordered by the
    positions the tile's last row sees (256 buckets), longest first."""
    _say("prefill plan contents")
    rng = np.random.default_rng(77)
    T, G = 300, 2
    prior = np.array([0, 700, 5, 1500, 64, 333])
    case = _random_verify_case(rng, prior + T, Hkv=2, G=G, D=64, T=T)
    dc = DevCase(case)
    counts = [300, 1, 0, 299, 128, 77]
    qp, qs, lens = _packed(case, counts)
    plan = _prefill_plan(case, dc, qs, lens, T)
    torch.cuda.synchronize()
    p = plan.cpu().numpy().view(np.int32)
    N = len(counts)
    maxb = case.block_tables.shape[1]
    rows_per_tile = int(p[3])
    tiles = -(-T * G // rows_per_tile)
    assert list(p[:8]) == [0x50414E32, N, tiles, rows_per_tile, int(qs[-1]), T, maxb, G]
    rows = p[16:16 + N * tiles * 8].reshape(N * tiles, 8)
    seen = set()
    width = max(1, -(-(maxb * 16 + 1) // 255))
    buckets = []
    for r in rows:
        b, t, q0, Tb, L, key = (int(x) for x in r[:6])
        assert (b, t) not in seen
        seen.add((b, t))
        assert q0 == int(qs[b]) and Tb == counts[b] and L == int(lens[b])
        R = Tb * G
        if t * rows_per_tile >= R:
            want = -1
        else:
            tl = (min(t * rows_per_tile + rows_per_tile, R) - 1) // G
            want = min(max(L - Tb + tl + 1, 0), L)
        assert key == want, (b, t)
        buckets.append(0 if key < 0 else 1 + min(key // width, 254))
    assert len(seen) == N * tiles
    assert (np.diff(buckets) <= 0).all(), "tiles must be ordered longest first"


def test_prefill_plan_for_other_sizes_is_ignored():
    _say("prefill plan for other sizes")
    rng = np.random.default_rng(78)
    T = 40
    case = _random_verify_case(rng, [50, 130, 200], Hkv=2, G=3, D=128, T=T)
    dc = DevCase(case)
    qp, qs, lens = _packed(case, [40, 7, 33])
    base = _prefill(case, dc, qp, qs, lens, T)
    big = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    sp = case.spec
    # a plan for a larger query count (another tile count)
    pa.make_prefill_plan(dev(lens), dev(qs), int(qs[-1]), 300, sp.q_heads, sp.kv_heads,
                         case.block_tables.shape[1], plan=big)
    got = torch.empty_like(base)
    pa.prefill(got, dev(qp), dc.k_cache, dc.v_cache, dc.block_tables, dev(lens), dev(qs),
               case.scale, T, plan=big)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), base.view(torch.int16))
    big.fill_(0x33)
    pa.prefill(got, dev(qp), dc.k_cache, dc.v_cache, dc.block_tables, dev(lens), dev(qs),
               case.scale, T, plan=big)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), base.view(torch.int16))
    small = torch.zeros(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(pa.PAError) as ei:
        pa.prefill(got, dev(qp), dc.k_cache, dc.v_cache, dc.block_tables, dev(lens), dev(qs),
                   case.scale, T, plan=small)
    assert ei.value.status == pa.PA_ERR_INVALID_ARG
