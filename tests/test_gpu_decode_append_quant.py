"""pa_decode_append_quant: the requantizing int8 cache write of one new token per
sequence and the decode over it, in one launch.

Against the two calls it fuses (pa_reshape_and_cache_quant, then pa_decode on the
written cache): the same cache codes, scales and output bits.  Against the oracle:
the cache and scales bit-exact (oracle/requant.py), the output within the int8
tolerance (oracle.decode over the oracle's written cache).
"""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_gqa_pa_amd import _lib as pa
from paged_kv_gqa_pa_amd import workloads as wl
from tests.gpu_util import TOL, DevCase, dev, host_bits, max_abs_err
from tests.test_gpu_decode import _random_case

pytestmark = pytest.mark.gpu

KDT = {"bf16": torch.bfloat16, "f32": torch.float32}


def _say(*a):
    print("[case]", *a, flush=True)


def _setup(rng, lens, Hkv, G, D, in_tag, poison=True):
    case = _random_case(rng, lens, Hkv=Hkv, G=G, D=D, tag="int8", poison=poison)
    N = len(lens)
    slots = wl.slots_for_positions(case.block_tables, np.arange(N), np.asarray(lens, np.int64) - 1)
    # N(0, 1) rows as in the configurations (a row beyond the block's maximum raises its
    # scale; the absolute int8 tolerance is set for outputs of that size)
    nk = wl.encode(rng.standard_normal((N, Hkv, D), dtype=np.float32), in_tag)
    nv = wl.encode(rng.standard_normal((N, Hkv, D), dtype=np.float32), in_tag)
    return case, slots, nk, nv


def _fused(case, slots, nk, nv, split=0, plan=False):
    dc = DevCase(case)
    out = torch.empty_like(dc.q)
    p = None
    if plan:
        p = pa.make_plan(dc.block_tables, dc.context_lens, case.spec.q_heads, case.spec.kv_heads,
                         case.spec.head_dim, case.max_context_len, torch.int8, split_tokens=split)
    pa.decode_append_quant(out, dc.q, dev(nk), dev(nv), dc.k_cache, dc.v_cache, dc.k_scale,
                           dc.v_scale, dev(slots), dc.block_tables, dc.context_lens, case.scale,
                           case.max_context_len, split_tokens=split, plan=p)
    torch.cuda.synchronize()
    return out, dc


def _two_calls(case, slots, nk, nv, split=0):
    dc = DevCase(case)
    pa.reshape_and_cache_quant(dev(nk), dev(nv), dc.k_cache, dc.v_cache, dc.k_scale, dc.v_scale,
                               dev(slots))
    out = torch.empty_like(dc.q)
    pa.decode(out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, case.scale,
              case.max_context_len, dc.k_scale, dc.v_scale, split_tokens=split)
    torch.cuda.synchronize()
    return out, dc


def _same(a, b):
    return host_bits(a).tobytes() == host_bits(b).tobytes()


LENS = [1, 2, 15, 16, 17, 31, 33, 100, 255, 513]


@pytest.mark.parametrize("in_tag", ["bf16", "f32"])
@pytest.mark.parametrize("G", [1, 2, 6, 8, 16])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("split", [0, 64])
def test_append_quant_equals_write_then_decode_bitwise(in_tag, G, D, split):
    _say("decode_append_quant", in_tag, "G", G, "D", D, "split", split)
    rng = np.random.default_rng(4000 + 7 * G + D + split + (1 if in_tag == "f32" else 0))
    case, slots, nk, nv = _setup(rng, LENS, 2, G, D, in_tag)
    got, dg = _fused(case, slots, nk, nv, split)
    want, dw = _two_calls(case, slots, nk, nv, split)
    assert _same(dg.k_cache, dw.k_cache) and _same(dg.v_cache, dw.v_cache)
    assert _same(dg.k_scale, dw.k_scale) and _same(dg.v_scale, dw.v_scale)
    assert _same(got, want)
    # the oracle: cache and scales exactly, the output within tolerance
    wk, wv, wks, wvs = oracle.reshape_and_cache_int8(nk, nv, in_tag, case.k_cache, case.v_cache,
                                                     case.k_scale, case.v_scale, slots)
    assert host_bits(dg.k_cache).tobytes() == wk.tobytes()
    assert host_bits(dg.v_cache).tobytes() == wv.tobytes()
    assert host_bits(dg.k_scale).tobytes() == wks.tobytes()
    assert host_bits(dg.v_scale).tobytes() == wvs.tobytes()
    ref = oracle.decode(case.q, wk, wv, case.block_tables, case.context_lens, case.scale, "bf16",
                        "int8", wks, wvs)
    assert max_abs_err(got, ref, TOL["int8"]) < TOL["int8"]


@pytest.mark.parametrize("planned", [False, True])
def test_append_quant_long_context_pieces(planned):
    """Long-context shape (12 / 2 heads, head_dim 128) over several pieces: the last
    piece requantizes; planned and unplanned give the same bits."""
    _say("decode_append_quant long contexts, planned", planned)
    rng = np.random.default_rng(4100)
    lens = [5000, 4097, 8192, 6001]
    case, slots, nk, nv = _setup(rng, lens, 2, 6, 128, "bf16")
    got, dg = _fused(case, slots, nk, nv, 0, plan=planned)
    want, dw = _two_calls(case, slots, nk, nv, 0)
    assert _same(got, want)
    assert _same(dg.k_cache, dw.k_cache) and _same(dg.k_scale, dw.k_scale)
    assert _same(dg.v_cache, dw.v_cache) and _same(dg.v_scale, dw.v_scale)


def test_append_quant_steps_in_a_row():
    """Three decode steps, each writing the next position (a block fills and the next
    one starts): fused and two-call caches and outputs stay identical."""
    _say("decode_append_quant three steps")
    rng = np.random.default_rng(4200)
    lens = np.array([14, 15, 16, 40, 47], np.int32)
    case = _random_case(rng, (lens + 3).tolist(), Hkv=2, G=6, D=128, tag="int8", poison=False)
    dg, dw = DevCase(case), DevCase(case)
    N = len(lens)
    for step in range(3):
        L = lens + step + 1
        slots = wl.slots_for_positions(case.block_tables, np.arange(N), L.astype(np.int64) - 1)
        nk = dev(wl.encode(rng.standard_normal((N, 2, 128), dtype=np.float32), "bf16"))
        nv = dev(wl.encode(rng.standard_normal((N, 2, 128), dtype=np.float32), "bf16"))
        q = dev(wl.encode(rng.standard_normal((N, 12, 128), dtype=np.float32), "bf16"))
        cl = dev(L.astype(np.int32))
        o1, o2 = torch.empty_like(q), torch.empty_like(q)
        pa.decode_append_quant(o1, q, nk, nv, dg.k_cache, dg.v_cache, dg.k_scale, dg.v_scale,
                               dev(slots), dg.block_tables, cl, case.scale, case.max_context_len)
        pa.reshape_and_cache_quant(nk, nv, dw.k_cache, dw.v_cache, dw.k_scale, dw.v_scale, dev(slots))
        pa.decode(o2, q, dw.k_cache, dw.v_cache, dw.block_tables, cl, case.scale,
                  case.max_context_len, dw.k_scale, dw.v_scale)
        torch.cuda.synchronize()
        assert _same(o1, o2), step
        assert _same(dg.k_cache, dw.k_cache) and _same(dg.k_scale, dw.k_scale), step
        assert _same(dg.v_cache, dw.v_cache) and _same(dg.v_scale, dw.v_scale), step


def test_append_quant_negative_slot_writes_nothing():
    _say("decode_append_quant negative slot")
    rng = np.random.default_rng(4300)
    case, slots, nk, nv = _setup(rng, [20, 40, 33], 2, 6, 128, "bf16")
    slots[1] = -1
    got, dg = _fused(case, slots, nk, nv)
    wk, wv, wks, wvs = oracle.reshape_and_cache_int8(nk, nv, "bf16", case.k_cache, case.v_cache,
                                                     case.k_scale, case.v_scale, slots)
    assert host_bits(dg.k_cache).tobytes() == wk.tobytes()
    assert host_bits(dg.v_scale).tobytes() == wvs.tobytes()
    # the rows with real slots are exact write-then-decode results
    ref = oracle.decode(case.q, wk, wv, case.block_tables, case.context_lens, case.scale, "bf16",
                        "int8", wks, wvs)
    assert max_abs_err(got[[0, 2]], ref[[0, 2]], TOL["int8"]) < TOL["int8"]


def test_append_quant_rejects_bad_arguments():
    rng = np.random.default_rng(4400)
    case, slots, nk, nv = _setup(rng, [20], 2, 6, 128, "bf16")
    dc = DevCase(case)
    out = torch.empty_like(dc.q)
    with pytest.raises(TypeError):
        pa.decode_append_quant(out, dc.q, dev(nk).to(torch.int8), dev(nv).to(torch.int8),
                               dc.k_cache, dc.v_cache, dc.k_scale, dc.v_scale, dev(slots),
                               dc.block_tables, dc.context_lens, case.scale, case.max_context_len)
    with pytest.raises(ValueError):
        pa.decode_append_quant(out, dc.q, dev(nk), dev(nv), dc.k_cache, dc.v_cache,
                               dc.k_scale.t().contiguous(), dc.v_scale, dev(slots),
                               dc.block_tables, dc.context_lens, case.scale, case.max_context_len)
    # the plain fused call still refuses an int8 cache
    with pytest.raises(pa.PAError) as ei:
        pa.decode_append(out, dc.q, dc.k_cache[:, :1, 0].transpose(0, 1).contiguous(),
                         dc.v_cache[:, :1, 0].transpose(0, 1).contiguous(), dc.k_cache,
                         dc.v_cache, dev(slots), dc.block_tables, dc.context_lens, case.scale,
                         case.max_context_len)
    assert ei.value.status == pa.PA_ERR_UNSUPPORTED
