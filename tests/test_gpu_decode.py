"""GPU parity of pa_reshape_and_cache and pa_decode against the fp64 oracle.

Every case prints what it runs before touching the GPU.  Tolerances: max-abs
1e-4 for fp32, 2e-2 for bf16 output (bf16 and int8 caches); cache writes and
placement / batch invariance are bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_gqa_pa_amd import _lib as pa
from paged_kv_gqa_pa_amd import workloads as wl
from tests.gpu_util import TOL, DevCase, dev, host_bits, max_abs_err

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _decode(dc, split_tokens=0, max_len=None, q=None, block_tables=None, k_cache=None,
            v_cache=None, context_lens=None):
    case = dc.case
    q = dc.q if q is None else q
    out = torch.empty_like(q)
    pa.decode(out, q, dc.k_cache if k_cache is None else k_cache,
              dc.v_cache if v_cache is None else v_cache,
              dc.block_tables if block_tables is None else block_tables,
              dc.context_lens if context_lens is None else context_lens, case.scale,
              case.max_context_len if max_len is None else max_len, dc.k_scale, dc.v_scale,
              split_tokens=split_tokens)
    torch.cuda.synchronize()
    return out


def _oracle_decode(case, q=None):
    return oracle.decode(case.q if q is None else q, case.k_cache, case.v_cache,
                         case.block_tables, case.context_lens, case.scale, case.spec.q_dtype,
                         case.spec.kv_dtype, case.k_scale, case.v_scale)


@pytest.mark.parametrize("split", [0, 16, 32, 48])
def test_tiny_fp32_parity(split):
    _say("tiny_fp32 poison split", split)
    case = wl.build_case("tiny_fp32", poison=True)
    dc = DevCase(case)
    out = _decode(dc, split)
    err = max_abs_err(out, _oracle_decode(case))
    assert err < TOL["f32"], err


@pytest.mark.parametrize("split", [0, 64, 128])
def test_qwen2_layer_bf16_parity(split):
    _say("qwen2_1p5b_bf16 split", split)
    case = wl.build_case("qwen2_1p5b_bf16", poison=True)
    dc = DevCase(case)
    out = _decode(dc, split)
    err = max_abs_err(out, _oracle_decode(case))
    assert err < TOL["bf16"], err


@pytest.mark.parametrize("layer", [0, 27])
def test_batch64_cache_write_then_decode(layer):
    """Full-size batch-64 layer: write the new token, compare whole caches, decode."""
    _say("batch64_28layer_bf16 layer", layer)
    case = wl.build_case("batch64_28layer_bf16", layer=layer)
    dc = DevCase(case)
    pa.reshape_and_cache(dc.new_k, dc.new_v, dc.k_cache, dc.v_cache, dc.slot_mapping)
    torch.cuda.synchronize()
    want_k, want_v = oracle.reshape_and_cache(case.new_k, case.new_v, case.k_cache,
                                              case.v_cache, case.slot_mapping)
    assert host_bits(dc.k_cache).tobytes() == want_k.tobytes()
    assert host_bits(dc.v_cache).tobytes() == want_v.tobytes()
    case.k_cache, case.v_cache = want_k, want_v
    out = _decode(dc)
    err = max_abs_err(out, _oracle_decode(case))
    assert err < TOL["bf16"], err


def test_long_ctx_int8_parity():
    _say("long_ctx_int8 default split")
    case = wl.build_case("long_ctx_int8")
    dc = DevCase(case)
    out = _decode(dc)
    err = max_abs_err(out, _oracle_decode(case))
    assert err < TOL["int8"], err


def test_long_ctx_int8_poison_and_small_split():
    """Two long-context sequences cut to lengths that end inside a block; their table
    rows end there (-1 after), the tails and every block no row uses are poisoned
    (code 127, unused blocks with scale 1e30); 256-position pieces."""
    _say("long_ctx_int8 poison, first 2 seqs cut to 32763 / 20003, split 256")
    case = wl.build_case("long_ctx_int8")
    lens = np.array([32768 - 5, 20000 + 3], np.int32)
    table = case.block_tables[:2].copy()
    for b, L in enumerate(lens):
        table[b, -(-int(L) // 16):] = -1
    kc, vc = case.k_cache.copy(), case.v_cache.copy()
    ks, vs = case.k_scale.copy(), case.v_scale.copy()
    spare, tails = wl.poison_int8(kc, ks, table, lens)
    wl.poison_int8(vc, vs, table, lens)
    assert spare >= 16384 - 2048 - 1251 and tails == 2
    q = np.ascontiguousarray(case.q[:2])
    out = torch.empty_like(dev(q))
    pa.decode(out, dev(q), dev(kc), dev(vc), dev(table), dev(lens), case.scale,
              case.max_context_len, dev(ks), dev(vs), split_tokens=256)
    torch.cuda.synchronize()
    want = oracle.decode(q, kc, vc, table, lens, case.scale, "bf16", "int8", ks, vs)
    err = max_abs_err(out, want, TOL["int8"])
    assert err < TOL["int8"], err


def test_placement_invariance_bitwise():
    _say("placement invariance qwen2_1p5b_bf16")
    case = wl.build_case("qwen2_1p5b_bf16")
    dc = DevCase(case)
    base = _decode(dc, 64)
    relabel = np.random.default_rng(11).permutation(case.spec.num_blocks).astype(np.int32)
    kc2 = np.empty_like(case.k_cache)
    vc2 = np.empty_like(case.v_cache)
    kc2[:, relabel] = case.k_cache
    vc2[:, relabel] = case.v_cache
    t = case.block_tables
    t2 = np.where(t >= 0, relabel[np.maximum(t, 0)], -1).astype(np.int32)
    moved = _decode(dc, 64, block_tables=dev(t2), k_cache=dev(kc2), v_cache=dev(vc2))
    assert torch.equal(base.view(torch.int16), moved.view(torch.int16))


def test_batch_invariance_bitwise():
    """A sequence alone gives the same bits as inside the batch (fixed piece length)."""
    _say("batch invariance qwen2_1p5b_bf16")
    case = wl.build_case("qwen2_1p5b_bf16")
    dc = DevCase(case)
    full = _decode(dc, 128)
    for b in (0, 5, 31):
        one = torch.empty_like(dc.q[b:b + 1])
        pa.decode(one, dc.q[b:b + 1].contiguous(), dc.k_cache, dc.v_cache,
                  dc.block_tables[b:b + 1].contiguous(), dc.context_lens[b:b + 1].contiguous(),
                  case.scale, int(case.context_lens[b]), split_tokens=128)
        torch.cuda.synchronize()
        assert torch.equal(one.view(torch.int16), full[b:b + 1].view(torch.int16)), b


def test_split_invariance_fp32():
    _say("split invariance fp32")
    rng = np.random.default_rng(5)
    lens = np.array([1, 15, 16, 17, 100, 257, 600], np.int32)
    case = _random_case(rng, lens, Hkv=2, G=3, D=128, tag="f32")
    dc = DevCase(case)
    want = _oracle_decode(case)
    outs = []
    for split in (16, 64, 256, 512, 1024):
        o = _decode(dc, split)
        assert max_abs_err(o, want) < TOL["f32"], split
        outs.append(o.double().cpu().numpy())
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() < 1e-6


def _random_case(rng, lens, Hkv, G, D, tag, qtag=None, nb=None, poison=False):
    """A PagedCase-like object with random contents for the given lengths; with
    `poison`, the blocks no sequence uses and the tails of partial last blocks hold
    NaN (int8: code 127, and scale 1e30 for the unused blocks)."""
    qtag = qtag or ("f32" if tag == "f32" else "bf16")
    lens = np.asarray(lens, np.int32)
    maxb = max(1, -(-int(lens.max()) // 16))
    need = int(sum(-(-int(L) // 16) for L in lens))
    nb = nb or need + 3
    table = wl.assign_blocks(lens, rng.permutation(nb).astype(np.int32), maxb)
    N = len(lens)
    k32 = rng.standard_normal((Hkv, nb, 16, D), dtype=np.float32)
    v32 = rng.standard_normal((Hkv, nb, 16, D), dtype=np.float32)
    ks = vs = None
    if tag == "int8":
        kc, ks = wl.quantize_int8_blocks(k32)
        vc, vs = wl.quantize_int8_blocks(v32)
        if poison:
            wl.poison_int8(kc, ks, table, lens)
            wl.poison_int8(vc, vs, table, lens)
    else:
        kc, vc = wl.encode(k32, tag), wl.encode(v32, tag)
        if poison:
            wl.poison_float(kc, tag, table, lens)
            wl.poison_float(vc, tag, table, lens)
    q = wl.encode(rng.standard_normal((N, Hkv * G, D), dtype=np.float32), qtag)
    spec = wl.Spec("random", 0, N, Hkv * G, Hkv, D, nb, qtag, tag, max(16, int(lens.max())))
    return wl.PagedCase(spec=spec, layer=0, context_lens=lens, block_tables=table, q=q,
                        k_cache=kc, v_cache=vc, k_scale=ks, v_scale=vs,
                        new_k=np.zeros((0, Hkv, D), kc.dtype), new_v=np.zeros((0, Hkv, D), kc.dtype),
                        slot_mapping=np.zeros(0, np.int64), scale=1.0 / np.sqrt(D))


EDGE_LENS = [0, 1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 200, 511, 512, 513, 1000]


@pytest.mark.parametrize("tag", ["f32", "bf16", "int8"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 3, 4, 5, 6, 7, 8, 16])
def test_edge_lengths_all_shapes(tag, D, G):
    _say("edge lengths", tag, "D", D, "G", G)
    rng = np.random.default_rng(100 + G + D)
    case = _random_case(rng, EDGE_LENS, Hkv=2, G=G, D=D, tag=tag, poison=True)
    dc = DevCase(case)
    want = _oracle_decode(case)
    for split in (0, 32):
        out = _decode(dc, split)
        err = max_abs_err(out, want, TOL[tag])
        assert err < TOL[tag], (split, err)
        got = out.float().cpu().numpy()
        assert (got[0] == 0).all(), "empty context must give zeros"
    if tag != "int8":
        # one position: the output is that position's V row exactly
        vrow = oracle.widen(case.v_cache[:, case.block_tables[1, 0], 0, :], tag)   # [Hkv, D]
        got = out.double().cpu().numpy()[1]
        assert np.array_equal(got, np.repeat(vrow, G, axis=0))


@pytest.mark.parametrize("tag,G", [("f32", 2), ("bf16", 2), ("bf16", 6), ("int8", 2), ("int8", 6)])
@pytest.mark.parametrize("scale", [-0.3, 0.0, 1.5])
def test_decode_scales(tag, G, scale):
    """Negative, zero and large softmax scales on both decode kernels (vector ALUs:
    f32 and bf16 groups below 4; matrix cores: bf16 groups of 4 or more and int8)."""
    _say("decode scale", scale, tag, "G", G)
    rng = np.random.default_rng(500 + G)
    case = _random_case(rng, [1, 17, 100, 333, 700], Hkv=2, G=G, D=128, tag=tag)
    case.scale = float(scale)
    dc = DevCase(case)
    want = _oracle_decode(case)
    for split in (0, 64):
        out = _decode(dc, split)
        assert max_abs_err(out, want) < TOL[tag], (split, max_abs_err(out, want))


def test_equal_keys_give_mean_of_v():
    _say("equal keys")
    rng = np.random.default_rng(9)
    case = _random_case(rng, [37, 300], Hkv=1, G=4, D=128, tag="f32")
    case.k_cache[...] = case.k_cache[0, 0, 0]
    dc = DevCase(case)
    out = _decode(dc, 64)
    for b, L in enumerate(case.context_lens):
        rows = oracle.gather_context(case.v_cache, case.block_tables[b], int(L), 0, "f32")
        assert np.abs(out[b].double().cpu().numpy() - rows.mean(0)).max() < 1e-5


def test_poisoned_tail_and_spare_blocks_bitwise():
    _say("poison vs clean bf16")
    clean = wl.build_case("qwen2_1p5b_bf16")
    dirty = wl.build_case("qwen2_1p5b_bf16", poison=True)
    a = _decode(DevCase(clean), 0)
    b = _decode(DevCase(dirty), 0)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def _stored(rng, shape, tag):
    if tag == "int8":
        return rng.integers(-127, 128, size=shape, dtype=np.int8)
    return wl.encode(rng.standard_normal(shape, dtype=np.float32), tag)


@pytest.mark.parametrize("tag,D", [("f32", 64), ("bf16", 128), ("int8", 128), ("int8", 64)])
def test_cache_write_skips_negative_slots_and_touches_nothing_else(tag, D):
    _say("cache write", tag, D)
    rng = np.random.default_rng(17)
    Hkv, nb = 3, 9
    kc = _stored(rng, (Hkv, nb, 16, D), tag)
    vc = _stored(rng, (Hkv, nb, 16, D), tag)
    key = _stored(rng, (7, Hkv, D), tag)
    val = _stored(rng, (7, Hkv, D), tag)
    slots = np.array([3, -1, 16 * nb - 1, 40, -7, 0, 77], np.int64)
    dk, dv = dev(kc), dev(vc)
    pa.reshape_and_cache(dev(key), dev(val), dk, dv, dev(slots))
    torch.cuda.synchronize()
    wk, wv = oracle.reshape_and_cache(key, val, kc, vc, slots)
    assert host_bits(dk).tobytes() == wk.tobytes()
    assert host_bits(dv).tobytes() == wv.tobytes()


def test_invalid_arguments_raise_before_launch():
    case = wl.build_case("tiny_fp32")
    dc = DevCase(case)
    out = torch.empty_like(dc.q)
    with pytest.raises(pa.PAError) as ei:
        pa.decode(out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens,
                  case.scale, 64, split_tokens=24)
    assert ei.value.status == pa.PA_ERR_INVALID_ARG
    with pytest.raises(pa.PAError) as ei:
        pa.decode(out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens,
                  case.scale, 64 * 16 + 1)
    assert ei.value.status == pa.PA_ERR_INVALID_ARG


def test_workspace_reuse_across_calls():
    """Arrival counters return to zero: repeated calls on one workspace stay correct."""
    _say("workspace reuse qwen2_1p5b_bf16 split 64/128")
    case = wl.build_case("qwen2_1p5b_bf16")
    dc = DevCase(case)
    want = _oracle_decode(case)
    need = max(pa.workspace_size(case.num_seqs, 1, 12, 2, 128, case.max_context_len,
                                 torch.bfloat16, s) for s in (64, 128))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    first = None
    for rep in range(3):
        for split in (64, 128):
            out = torch.full_like(dc.q, float("nan"))
            pa.decode(out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens,
                      case.scale, case.max_context_len, split_tokens=split, workspace=ws)
            torch.cuda.synchronize()
            assert max_abs_err(out, want) < TOL["bf16"], (rep, split)
            if split == 64:
                if first is None:
                    first = out.clone()
                assert torch.equal(out.view(torch.int16), first.view(torch.int16))


# ----------------------------------------------------------------------------
# pa_decode_append: cache write of the new token + decode in one launch
# ----------------------------------------------------------------------------
def test_decode_append_equals_write_then_decode_bitwise():
    """Full-size batch-64 layer: same output bits and same cache bytes as the two calls."""
    _say("decode_append batch64 layer 3")
    case = wl.build_case("batch64_28layer_bf16", layer=3)
    two = DevCase(case)
    one = DevCase(case)
    pa.reshape_and_cache(two.new_k, two.new_v, two.k_cache, two.v_cache, two.slot_mapping)
    ref = torch.empty_like(two.q)
    pa.decode(ref, two.q, two.k_cache, two.v_cache, two.block_tables, two.context_lens,
              case.scale, case.max_context_len)
    out = torch.empty_like(one.q)
    pa.decode_append(out, one.q, one.new_k, one.new_v, one.k_cache, one.v_cache,
                     one.slot_mapping, one.block_tables, one.context_lens, case.scale,
                     case.max_context_len)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    want_k, want_v = oracle.reshape_and_cache(case.new_k, case.new_v, case.k_cache,
                                              case.v_cache, case.slot_mapping)
    assert host_bits(one.k_cache).tobytes() == want_k.tobytes()
    assert host_bits(one.v_cache).tobytes() == want_v.tobytes()
    case.k_cache, case.v_cache = want_k, want_v
    assert max_abs_err(out, _oracle_decode(case)) < TOL["bf16"]


@pytest.mark.parametrize("planned", [False, True])
def test_decode_append_matrix_core_equals_write_then_decode_bitwise(planned):
    """Qwen2-shaped layer (G = 6, bf16: the matrix-core kernel): one launch gives the
    two calls' output bits and cache bytes, with and without a work plan."""
    _say("decode_append qwen2 shape, planned", planned)
    case = wl.build_case("qwen2_1p5b_bf16")
    two, one = DevCase(case), DevCase(case)
    plan = None
    if planned:
        plan = pa.make_plan(two.block_tables, two.context_lens, case.spec.q_heads,
                            case.spec.kv_heads, case.spec.head_dim, case.max_context_len,
                            torch.bfloat16)
    pa.reshape_and_cache(two.new_k, two.new_v, two.k_cache, two.v_cache, two.slot_mapping)
    ref = torch.empty_like(two.q)
    pa.decode(ref, two.q, two.k_cache, two.v_cache, two.block_tables, two.context_lens,
              case.scale, case.max_context_len, plan=plan)
    out = torch.empty_like(one.q)
    pa.decode_append(out, one.q, one.new_k, one.new_v, one.k_cache, one.v_cache,
                     one.slot_mapping, one.block_tables, one.context_lens, case.scale,
                     case.max_context_len, plan=plan)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    want_k, want_v = oracle.reshape_and_cache(case.new_k, case.new_v, case.k_cache,
                                              case.v_cache, case.slot_mapping)
    assert host_bits(one.k_cache).tobytes() == want_k.tobytes()
    assert host_bits(one.v_cache).tobytes() == want_v.tobytes()
    case.k_cache, case.v_cache = want_k, want_v
    assert max_abs_err(out, _oracle_decode(case)) < TOL["bf16"]


@pytest.mark.parametrize("tag", ["f32", "bf16"])
@pytest.mark.parametrize("G", [1, 2, 4, 6, 8])
@pytest.mark.parametrize("split", [0, 32])
def test_decode_append_edges(tag, G, split):
    _say("decode_append edges", tag, "G", G, "split", split)
    rng = np.random.default_rng(300 + G + split)
    lens = [1, 2, 15, 16, 17, 32, 33, 100, 513]
    case = _random_case(rng, lens, Hkv=2, G=G, D=128 if tag == "bf16" else 64, tag=tag)
    D = case.spec.head_dim
    lens_a = np.asarray(lens, np.int64)
    slots = wl.slots_for_positions(case.block_tables, np.arange(len(lens)), lens_a - 1)
    new = rng.standard_normal((len(lens), 2, D), dtype=np.float32)
    newv = rng.standard_normal((len(lens), 2, D), dtype=np.float32)
    nk, nv = wl.encode(new, tag), wl.encode(newv, tag)
    dc = DevCase(case)
    out = torch.empty_like(dc.q)
    pa.decode_append(out, dc.q, dev(nk), dev(nv), dc.k_cache, dc.v_cache, dev(slots),
                     dc.block_tables, dc.context_lens, case.scale, case.max_context_len,
                     split_tokens=split)
    torch.cuda.synchronize()
    want_k, want_v = oracle.reshape_and_cache(nk, nv, case.k_cache, case.v_cache, slots)
    assert host_bits(dc.k_cache).tobytes() == want_k.tobytes()
    assert host_bits(dc.v_cache).tobytes() == want_v.tobytes()
    case.k_cache, case.v_cache = want_k, want_v
    assert max_abs_err(out, _oracle_decode(case)) < TOL[tag]


def test_decode_append_negative_slot_writes_nothing():
    _say("decode_append negative slot")
    rng = np.random.default_rng(9)
    lens = [20, 40]
    case = _random_case(rng, lens, Hkv=2, G=2, D=128, tag="bf16")
    slots = wl.slots_for_positions(case.block_tables, np.arange(2), np.asarray(lens) - 1)
    slots[0] = -1
    nk = wl.encode(rng.standard_normal((2, 2, 128), dtype=np.float32), "bf16")
    nv = wl.encode(rng.standard_normal((2, 2, 128), dtype=np.float32), "bf16")
    dc = DevCase(case)
    out = torch.empty_like(dc.q)
    pa.decode_append(out, dc.q, dev(nk), dev(nv), dc.k_cache, dc.v_cache, dev(slots),
                     dc.block_tables, dc.context_lens, case.scale, case.max_context_len)
    torch.cuda.synchronize()
    want_k, _ = oracle.reshape_and_cache(nk, nv, case.k_cache, case.v_cache, slots)
    assert host_bits(dc.k_cache).tobytes() == want_k.tobytes()
    case.k_cache = want_k
    _, want_v = oracle.reshape_and_cache(nk, nv, case.k_cache, case.v_cache, slots)
    case.v_cache = want_v
    want = _oracle_decode(case)
    assert max_abs_err(out[1], want[1], TOL["bf16"]) < TOL["bf16"]


@pytest.mark.parametrize("tag,G", [("f32", 2), ("bf16", 6), ("int8", 6)])
def test_long_pieces_span_several_table_registers(tag, G):
    """A piece longer than 64 blocks reads its table entries from several lane registers."""
    _say("long pieces", tag, "G", G)
    rng = np.random.default_rng(77 + G)
    lens = [1, 1000, 1025, 2048, 2049, 4096, 4097, 5000]
    case = _random_case(rng, lens, Hkv=2, G=G, D=128, tag=tag)
    dc = DevCase(case)
    want = _oracle_decode(case)
    for split in (1040, 2048, 4096, 0):
        out = _decode(dc, split)
        assert max_abs_err(out, want) < TOL[tag], (split, max_abs_err(out, want))
