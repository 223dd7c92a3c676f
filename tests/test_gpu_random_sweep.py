"""A seeded sweep over random shapes and entry points, each against the oracle.

Every case draws an entry point (decode, decode with a work plan, the fused
cache write + decode, the fused requantizing int8 write + decode, verify,
verify with a work plan, variable-length verify, chunked prefill), a cache type, head_dim, group size, KV-head count,
a batch whose lengths mix block edges with random ones, a piece length, and
a pool with poisoned spare blocks and partial-block tails; the GPU result is
compared with the oracle on the same inputs at the cache type's tolerance
(and the fused call's cache bytes exactly).  The draws reach combinations
that the per-feature tests do not enumerate.
"""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_gqa_pa_amd import _lib as pa
from paged_kv_gqa_pa_amd import workloads as wl
from tests.gpu_util import TOL, DevCase, dev, host_bits, max_abs_err
from tests.test_gpu_decode import _random_case
from tests.test_gpu_verify import _random_verify_case

pytestmark = pytest.mark.gpu

ENTRIES = ("decode", "decode_plan", "append", "append_quant", "verify", "verify_plan", "varlen",
           "prefill")
CASES = 210
WIDE = 70
KDT = {"f32": torch.float32, "bf16": torch.bfloat16, "int8": torch.int8}


def _say(*a):
    print("[case]", *a, flush=True)


def _lengths(rng, n, lo, hi):
    """n lengths in [lo, hi]: about half on or next to a block edge."""
    edges = [16 * k + d for k in range(hi // 16 + 1) for d in (-1, 0, 1)]
    edges = [e for e in edges if lo <= e <= hi] or [lo]
    return [int(rng.choice(edges)) if rng.random() < 0.5 else int(rng.integers(lo, hi + 1))
            for _ in range(n)]


def _draw(i):
    """Case i: cases CASES .. CASES + WIDE - 1 draw wider shapes (more KV heads and
    sequences, up to 16 query tokens, contexts past several pieces)."""
    wide = i >= CASES
    rng = np.random.default_rng((60_000 if wide else 50_000) + i)
    entry = ENTRIES[i % len(ENTRIES)]
    D = int(rng.choice([64, 128]))
    Hkv = int(rng.integers(1, 9 if wide else 4))
    if entry in ("decode", "decode_plan", "append", "append_quant"):
        G = int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8, 16]))
        T = 1
    else:
        G = int(rng.choice([1, 2, 3, 4, 6, 8, 16]))
        T = int(rng.integers(1, (17 if wide else 9) if entry != "prefill" else 41))
    kv = {"append": ["f32", "bf16", "bf16"], "append_quant": ["int8"],
          "decode": ["f32", "bf16", "int8"],
          "decode_plan": ["f32", "bf16", "int8"]}.get(entry, ["bf16", "int8"])
    kv = str(rng.choice(kv))
    N = int(rng.integers(1, 21 if wide else 10))
    lo = 1 if entry.startswith("append") else (T if entry == "prefill" else 0)
    hi = int(rng.choice([700, 2100, 4500] if wide else [64, 300, 1100]))
    lens = _lengths(rng, N, lo, hi)
    split = int(rng.choice([0, 16, 48, 128, 512] + ([1024, 4096] if wide else [])))
    return rng, entry, kv, D, Hkv, G, T, lens, split


@pytest.mark.parametrize("i", range(CASES + WIDE))
def test_random_sweep(i):
    rng, entry, kv, D, Hkv, G, T, lens, split = _draw(i)
    _say("sweep", i, entry, kv, "D", D, "Hkv", Hkv, "G", G, "T", T, "split", split, "lens", lens)
    Hq = Hkv * G
    tol = TOL[kv]
    if entry == "append_quant":
        # the requantizing int8 write + decode in one launch: the cache, scales and output
        # against the oracle's requantizing write and decode
        in_tag = str(rng.choice(["bf16", "f32"]))
        case = _random_case(rng, lens, Hkv=Hkv, G=G, D=D, tag="int8", poison=True)
        dc = DevCase(case)
        slots = wl.slots_for_positions(case.block_tables, np.arange(len(lens)),
                                       np.asarray(lens, np.int64) - 1)
        nk = wl.encode(rng.standard_normal((len(lens), Hkv, D), dtype=np.float32), in_tag)
        nv = wl.encode(rng.standard_normal((len(lens), Hkv, D), dtype=np.float32), in_tag)
        out = torch.empty_like(dc.q)
        pa.decode_append_quant(out, dc.q, dev(nk), dev(nv), dc.k_cache, dc.v_cache, dc.k_scale,
                               dc.v_scale, dev(slots), dc.block_tables, dc.context_lens,
                               case.scale, case.max_context_len, split_tokens=split)
        torch.cuda.synchronize()
        wk, wv, wks, wvs = oracle.reshape_and_cache_int8(nk, nv, in_tag, case.k_cache,
                                                         case.v_cache, case.k_scale,
                                                         case.v_scale, slots)
        assert host_bits(dc.k_cache).tobytes() == wk.tobytes()
        assert host_bits(dc.v_cache).tobytes() == wv.tobytes()
        assert host_bits(dc.k_scale).tobytes() == wks.tobytes()
        assert host_bits(dc.v_scale).tobytes() == wvs.tobytes()
        want = oracle.decode(case.q, wk, wv, case.block_tables, case.context_lens, case.scale,
                             "bf16", "int8", wks, wvs)
        assert max_abs_err(out, want, tol) < tol
        return
    if entry in ("decode", "decode_plan", "append"):
        case = _random_case(rng, lens, Hkv=Hkv, G=G, D=D, tag=kv, poison=True)
        dc = DevCase(case)
        out = torch.empty_like(dc.q)
        plan = None
        if entry == "decode_plan":
            plan = pa.make_plan(dc.block_tables, dc.context_lens, Hq, Hkv, D,
                                case.max_context_len, KDT[kv], split_tokens=split)
        if entry == "append":
            slots = wl.slots_for_positions(case.block_tables, np.arange(len(lens)),
                                           np.asarray(lens, np.int64) - 1)
            nk = wl.encode(rng.standard_normal((len(lens), Hkv, D), dtype=np.float32), kv)
            nv = wl.encode(rng.standard_normal((len(lens), Hkv, D), dtype=np.float32), kv)
            pa.decode_append(out, dc.q, dev(nk), dev(nv), dc.k_cache, dc.v_cache, dev(slots),
                             dc.block_tables, dc.context_lens, case.scale, case.max_context_len,
                             split_tokens=split)
            torch.cuda.synchronize()
            want_k, want_v = oracle.reshape_and_cache(nk, nv, case.k_cache, case.v_cache, slots)
            assert host_bits(dc.k_cache).tobytes() == want_k.tobytes()
            assert host_bits(dc.v_cache).tobytes() == want_v.tobytes()
            case.k_cache, case.v_cache = want_k, want_v
        else:
            pa.decode(out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens,
                      case.scale, case.max_context_len, dc.k_scale, dc.v_scale,
                      split_tokens=split, plan=plan)
            torch.cuda.synchronize()
        want = oracle.decode(case.q, case.k_cache, case.v_cache, case.block_tables,
                             case.context_lens, case.scale, case.spec.q_dtype, kv,
                             case.k_scale, case.v_scale)
        assert max_abs_err(out, want, tol) < tol
        return

    case = _random_verify_case(rng, lens, Hkv=Hkv, G=G, D=D, T=T, poison=True, kv=kv)
    dc = DevCase(case)
    if entry in ("verify", "verify_plan"):
        plan = None
        if entry == "verify_plan":
            plan = pa.make_plan(dc.block_tables, dc.context_lens, Hq, Hkv, D,
                                case.max_context_len, KDT[kv], num_query_tokens=T,
                                split_tokens=split)
        out = torch.empty_like(dc.q)
        pa.verify(out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, case.scale,
                  case.max_context_len, dc.k_scale, dc.v_scale, split_tokens=split, plan=plan)
        torch.cuda.synchronize()
        want = oracle.verify(case.q, case.k_cache, case.v_cache, case.block_tables,
                             case.context_lens, case.scale, "bf16", kv, case.k_scale, case.v_scale)
        assert max_abs_err(out, want, tol) < tol
        return

    # variable-length verify and prefill: T_b tokens per sequence, packed; sequence b's
    # tokens are its last T_b positions
    counts = rng.integers(0 if entry == "varlen" else 1, T + 1, size=len(lens))
    qs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    qp = np.concatenate([case.q[b, :int(c)] for b, c in enumerate(counts)], axis=0) \
        if qs[-1] else np.zeros((0, Hq, D), case.q.dtype)
    qp = np.ascontiguousarray(qp)
    lens_b = np.maximum(case.context_lens.astype(np.int64) - T + counts, 0).astype(np.int32)
    q = dev(qp)
    out = torch.empty_like(q)
    if entry == "varlen":
        pa.verify_varlen(out, q, dc.k_cache, dc.v_cache, dc.block_tables, dev(lens_b), dev(qs),
                         case.scale, int(case.max_context_len), T, dc.k_scale, dc.v_scale,
                         split_tokens=split)
    else:
        pa.prefill(out, q, dc.k_cache, dc.v_cache, dc.block_tables, dev(lens_b), dev(qs),
                   case.scale, T, dc.k_scale, dc.v_scale)
    torch.cuda.synchronize()
    want = oracle.verify_varlen(qp, case.k_cache, case.v_cache, case.block_tables, lens_b, qs,
                                case.scale, "bf16", kv, case.k_scale, case.v_scale)
    assert max_abs_err(out, want, tol) < tol
