"""Work plans (pa_plan and the *_planned calls) on the GPU.

A plan only reorders the start of work units whose arithmetic is fixed by the
unit, so a planned call must give the unplanned call's bits exactly, and both
meet the oracle.  The plan's own contents are integer indexing (sequence,
piece, length, tile count, copied table entries): checked exactly against the
definition computed here on the host.
"""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_gqa_pa_amd import _lib as pa
from tests.gpu_util import TOL, DevCase, dev, host_bits, max_abs_err
from tests.test_gpu_decode import _random_case
from tests.test_gpu_verify import _random_verify_case

pytestmark = pytest.mark.gpu

TDT = {"f32": torch.float32, "bf16": torch.bfloat16, "int8": torch.int8}
HEADER, ROW_HEAD, MAGIC = 16, 4, 0x50414E31


def _say(*a):
    print("[case]", *a, flush=True)


def _plan(dc, kv, split, T=1, max_len=None):
    case = dc.case
    sp = case.spec
    return pa.make_plan(dc.block_tables, dc.context_lens, sp.q_heads, sp.kv_heads, sp.head_dim,
                        case.max_context_len if max_len is None else max_len, TDT[kv],
                        num_query_tokens=T, split_tokens=split)


def _decode(dc, split, plan=None):
    case = dc.case
    out = torch.empty_like(dc.q)
    pa.decode(out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, case.scale,
              case.max_context_len, dc.k_scale, dc.v_scale, split_tokens=split, plan=plan)
    torch.cuda.synchronize()
    return out


def _same_bits(a, b):
    return np.array_equal(host_bits(a), host_bits(b))


LENS = [0, 1, 15, 16, 17, 33, 64, 65, 200, 511, 512, 513, 777, 1000, 7, 300]


def test_plan_contents_exact():
    """Header, one row per (sequence, piece) unit, rows sorted by tile count, copied table
    entries equal to the table's."""
    _say("plan contents, 16 sequences, split 64")
    rng = np.random.default_rng(41)
    case = _random_case(rng, LENS, Hkv=2, G=3, D=128, tag="bf16")
    dc = DevCase(case)
    split = 64
    plan = _plan(dc, "bf16", split)
    torch.cuda.synchronize()
    p = plan.cpu().numpy().view(np.int32)
    N = len(LENS)
    max_pieces = -(-case.max_context_len // split)
    sb = split // 16
    stride = ROW_HEAD + (sb + 3) // 4 * 4
    maxb = case.block_tables.shape[1]
    assert list(p[:5]) == [MAGIC, N, max_pieces, split, maxb]
    snake_units, snake_rounds = int(p[5]), int(p[6])
    assert (p[7:HEADER] == 0).all()
    rows = p[HEADER:HEADER + N * max_pieces * stride].reshape(N * max_pieces, stride)
    seen = set()
    for row in rows:
        b, piece, L, tiles = (int(x) for x in row[:4])
        assert (b, piece) not in seen
        seen.add((b, piece))
        want_L = int(case.context_lens[b])
        assert L == want_L
        npieces = max(1, -(-want_L // split))
        want_tiles = min(max(-(-want_L // 16) - piece * sb, 0), sb) if piece < npieces else -1
        assert tiles == want_tiles, (b, piece)
        ids = row[ROW_HEAD:ROW_HEAD + sb]
        for i in range(sb):
            want = case.block_tables[b, piece * sb + i] if i < tiles else 0
            assert ids[i] == want, (b, piece, i)
    assert len(seen) == N * max_pieces
    _check_order(rows[:, 3], snake_units, snake_rounds)


def _check_order(keys, snake_units, snake_rounds):
    """Longest first, except that the first snake_rounds rounds of snake_units units
    alternate: even rounds longest first, odd rounds shortest first; every unit of a round
    is at least as long as every unit of the next."""
    U = len(keys)
    S = snake_units if snake_units > 0 else U
    bounds = list(range(0, U, S)) + [U]
    for r in range(len(bounds) - 1):
        part = keys[bounds[r]:bounds[r + 1]]
        if snake_units > 0 and r < snake_rounds and r % 2 == 1:
            assert (np.diff(part) >= 0).all(), r
        else:
            assert (np.diff(part) <= 0).all(), r
        if r + 2 < len(bounds):
            assert part.min() >= keys[bounds[r + 1]:bounds[r + 2]].max(), r


@pytest.mark.parametrize("kv,G,T", [("bf16", 2, 1), ("f32", 1, 1), ("bf16", 6, 1), ("int8", 6, 1),
                                    ("bf16", 2, 5)])
def test_plan_order_for_each_kernel(kv, G, T):
    """The vector-ALU decode keeps two workgroups per CU (snaked rounds of CUs / kv_heads
    units); the matrix-core kernel one (plain longest-first)."""
    _say("plan order", kv, "G", G, "T", T)
    rng = np.random.default_rng(42 + G + T)
    lens = rng.integers(1, 513, size=200).astype(np.int32)
    case = (_random_case(rng, lens, Hkv=8, G=G, D=128, tag=kv) if T == 1 else
            _random_verify_case(rng, lens, Hkv=8, G=G, D=128, T=T, kv=kv))
    dc = DevCase(case)
    plan = _plan(dc, kv, 0, T=T)
    torch.cuda.synchronize()
    p = plan.cpu().numpy().view(np.int32)
    split, max_pieces = int(p[3]), int(p[2])
    stride = ROW_HEAD + (split // 16 + 3) // 4 * 4
    U = len(lens) * max_pieces
    rows = p[HEADER:HEADER + U * stride].reshape(U, stride)
    snake_units, snake_rounds = int(p[5]), int(p[6])
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    vector_kernel = T == 1 and kv != "int8" and G < 4
    if vector_kernel:                       # two or more workgroups per CU
        assert snake_units == -(-cus // 8) and snake_rounds >= 2
    elif kv == "bf16":                      # 128 KiB of LDS: one workgroup per CU
        assert snake_units == 0
    if snake_units:
        assert snake_units == -(-cus // 8) and snake_rounds >= 2
    _check_order(rows[:, 3], snake_units, snake_rounds)


@pytest.mark.parametrize("tag", ["f32", "bf16", "int8"])
@pytest.mark.parametrize("G", [1, 2, 6, 16])
@pytest.mark.parametrize("D", [64, 128])
def test_planned_decode_equals_unplanned_bitwise(tag, G, D):
    _say("planned decode", tag, "G", G, "D", D)
    rng = np.random.default_rng(500 + G + D)
    case = _random_case(rng, LENS, Hkv=2, G=G, D=D, tag=tag)
    dc = DevCase(case)
    want = oracle.decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens,
                         case.scale, case.spec.q_dtype, tag, case.k_scale, case.v_scale)
    for split in (0, 64, 512):
        plan = _plan(dc, tag, split)
        base = _decode(dc, split)
        got = _decode(dc, split, plan)
        assert _same_bits(got, base), split
        assert max_abs_err(got, want) < TOL[tag], split


@pytest.mark.parametrize("kv", ["bf16", "int8"])
@pytest.mark.parametrize("G,T", [(2, 5), (3, 5), (1, 16), (6, 5), (8, 5)])
def test_planned_verify_equals_unplanned_bitwise(kv, G, T):
    _say("planned verify", kv, "G", G, "T", T)
    rng = np.random.default_rng(600 + G + T)
    case = _random_verify_case(rng, [5, 16, 17, 300, 1029, 64, 3, 700], Hkv=2, G=G, D=128, T=T,
                               poison=True, kv=kv)
    dc = DevCase(case)
    want = oracle.verify(case.q, case.k_cache, case.v_cache, case.block_tables,
                         case.context_lens, case.scale, "bf16", kv, case.k_scale, case.v_scale)
    for split in (0, 256):
        outs = []
        for plan in (None, _plan(dc, kv, split, T=T)):
            o = torch.empty_like(dc.q)
            pa.verify(o, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens,
                      case.scale, case.max_context_len, dc.k_scale, dc.v_scale,
                      split_tokens=split, plan=plan)
            torch.cuda.synchronize()
            outs.append(o)
        assert _same_bits(outs[1], outs[0]), split
        assert max_abs_err(outs[1], want) < TOL[kv], split


@pytest.mark.parametrize("tag,G", [("bf16", 2), ("f32", 3), ("bf16", 6)])
def test_planned_append_equals_unplanned_bitwise(tag, G):
    """Cache write + decode through the plan: caches and outputs equal the unplanned call's."""
    _say("planned append", tag, "G", G)
    rng = np.random.default_rng(700 + G)
    case = _random_case(rng, [1, 16, 17, 200, 512, 513, 40], Hkv=2, G=G, D=128, tag=tag)
    N, Hkv, D = len(case.context_lens), 2, 128
    # each sequence's new token is its last position
    last = case.context_lens.astype(np.int64) - 1
    slots = case.block_tables[np.arange(N), last // 16].astype(np.int64) * 16 + last % 16
    nk = rng.standard_normal((N, Hkv, D), dtype=np.float32)
    nv = rng.standard_normal((N, Hkv, D), dtype=np.float32)
    from paged_kv_gqa_pa_amd import workloads as wl
    nk, nv = wl.encode(nk, tag), wl.encode(nv, tag)
    res = []
    for use_plan in (False, True):
        dc = DevCase(case)
        plan = _plan(dc, tag, 128) if use_plan else None
        out = torch.empty_like(dc.q)
        pa.decode_append(out, dc.q, dev(nk), dev(nv), dc.k_cache, dc.v_cache, dev(slots),
                         dc.block_tables, dc.context_lens, case.scale, case.max_context_len,
                         split_tokens=128, plan=plan)
        torch.cuda.synchronize()
        res.append((out, dc.k_cache, dc.v_cache))
    for a, b in zip(res[0], res[1]):
        assert _same_bits(a, b)


def test_plan_for_other_sizes_is_ignored():
    """A plan whose header does not match the call (other batch, other piece length) is
    detected on the device: the call runs in the natural order with the same bits."""
    _say("mismatched plans fall back to the natural order")
    rng = np.random.default_rng(77)
    case = _random_case(rng, LENS, Hkv=2, G=2, D=128, tag="bf16")
    dc = DevCase(case)
    base = _decode(dc, 64)
    big = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    sp = case.spec
    # a plan for the first 9 sequences only
    pa.make_plan(dc.block_tables[:9].contiguous(), dc.context_lens[:9].contiguous(), sp.q_heads,
                 sp.kv_heads, sp.head_dim, case.max_context_len, torch.bfloat16,
                 split_tokens=64, plan=big)
    assert _same_bits(_decode(dc, 64, big), base)
    # a plan for another piece length
    pa.make_plan(dc.block_tables, dc.context_lens, sp.q_heads, sp.kv_heads, sp.head_dim,
                 case.max_context_len, torch.bfloat16, split_tokens=32, plan=big)
    assert _same_bits(_decode(dc, 64, big), base)
    # garbage in the plan buffer
    big.fill_(0x5A)
    assert _same_bits(_decode(dc, 64, big), base)


def test_plan_invalid_arguments():
    _say("plan invalid arguments")
    rng = np.random.default_rng(78)
    case = _random_case(rng, LENS, Hkv=2, G=2, D=128, tag="bf16")
    dc = DevCase(case)
    plan = _plan(dc, "bf16", 64)
    out = torch.empty_like(dc.q)
    with pytest.raises(pa.PAError) as ei:          # buffer too small for split 16
        pa.decode(out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens,
                  case.scale, case.max_context_len, split_tokens=16, plan=plan)
    assert ei.value.status == pa.PA_ERR_INVALID_ARG
    with pytest.raises(pa.PAError) as ei:          # 9000 sequences x 1 piece > 8192 units
        pa.make_plan(torch.zeros((9000, 1), dtype=torch.int32, device="cuda"),
                     torch.zeros(9000, dtype=torch.int32, device="cuda"), 4, 2, 128, 16,
                     torch.bfloat16)
    assert ei.value.status == pa.PA_ERR_UNSUPPORTED


def test_plan_and_decode_in_a_graph_follow_new_lengths():
    """Captured plan + planned decode: each replay plans from the buffers' current lengths
    and tables, and matches the unplanned decode of those lengths."""
    _say("graph of plan + planned decode, lengths changed between replays")
    rng = np.random.default_rng(79)
    lens_a = np.array([300, 17, 512, 1, 90, 256, 0, 450], np.int32)
    case = _random_case(rng, lens_a, Hkv=2, G=2, D=128, tag="bf16")
    dc = DevCase(case)
    sp = case.spec
    plan = torch.empty(pa.plan_size(len(lens_a), 1, sp.q_heads, sp.kv_heads, sp.head_dim,
                                    512, torch.bfloat16, 0), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(dc.q)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        pa.make_plan(dc.block_tables, dc.context_lens, sp.q_heads, sp.kv_heads, sp.head_dim, 512,
                     torch.bfloat16, plan=plan)
        pa.decode(out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens,
                  case.scale, 512, plan=plan)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pa.make_plan(dc.block_tables, dc.context_lens, sp.q_heads, sp.kv_heads, sp.head_dim, 512,
                     torch.bfloat16, plan=plan)
        pa.decode(out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens,
                  case.scale, 512, plan=plan)
    for lens in (lens_a, np.minimum(lens_a[::-1] + 5, lens_a.max()).astype(np.int32), lens_a):
        lens = np.minimum(lens, [-(-int(L) // 16) * 16 for L in lens_a]).astype(np.int32)
        dc.context_lens.copy_(torch.from_numpy(lens))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = torch.empty_like(out)
        pa.decode(ref, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens,
                  case.scale, 512)
        torch.cuda.synchronize()
        assert _same_bits(out, ref), lens
