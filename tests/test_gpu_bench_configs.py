"""The launch configurations bench.py times, at full size, against the oracle.

- Batch-64 step, one layer: a work plan made for the step's table and lengths,
  then pa_reshape_and_cache + pa_decode_planned, and pa_decode_append_planned
  (the fused step) on a fresh copy of the caches.  Both equal the unplanned
  calls bit for bit and meet the oracle on the whole output.
- Speculative verify (64 sequences, T = 5) started from a work plan: equal to the
  unplanned call bit for bit, and the oracle on the whole output.
- Chunked prefill as bench.py draws it (16 sequences, a 512-token chunk on
  U{0..1536} prior positions from default_rng(12), 16/8 heads, D = 128, a bf16
  cache of 8192 blocks), started from a prefill work plan: equal to the natural
  order bit for bit; the oracle on three sampled sequences (each sequence's
  rows depend on its own context only), the longest prior among them.
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


def test_batch64_planned_step_and_fused_step():
    _say("batch64_28layer_bf16 layer 5: planned write + decode, planned decode_append")
    case = wl.build_case("batch64_28layer_bf16", layer=5)
    spec = case.spec
    Hq, Hkv, D = spec.q_heads, spec.kv_heads, spec.head_dim
    dc = DevCase(case)
    k0, v0 = dc.k_cache.clone(), dc.v_cache.clone()
    plan = pa.make_plan(dc.block_tables, dc.context_lens, Hq, Hkv, D, spec.max_len,
                        torch.bfloat16)

    # write, then decode with and without the plan
    pa.reshape_and_cache(dc.new_k, dc.new_v, dc.k_cache, dc.v_cache, dc.slot_mapping)
    planned = torch.empty_like(dc.q)
    natural = torch.empty_like(dc.q)
    pa.decode(planned, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens,
              case.scale, spec.max_len, plan=plan)
    pa.decode(natural, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens,
              case.scale, spec.max_len)
    torch.cuda.synchronize()
    assert host_bits(planned).tobytes() == host_bits(natural).tobytes()
    k_written = host_bits(dc.k_cache).tobytes()
    v_written = host_bits(dc.v_cache).tobytes()

    want_k, want_v = oracle.reshape_and_cache(case.new_k, case.new_v, case.k_cache,
                                              case.v_cache, case.slot_mapping)
    want = oracle.decode(case.q, want_k, want_v, case.block_tables, case.context_lens,
                         case.scale, "bf16", "bf16")
    err = max_abs_err(planned, want)
    assert err < TOL["bf16"], err

    # the fused step on the original caches: same cache bytes, same output bits
    dc.k_cache.copy_(k0)
    dc.v_cache.copy_(v0)
    fused = torch.empty_like(dc.q)
    pa.decode_append(fused, dc.q, dc.new_k, dc.new_v, dc.k_cache, dc.v_cache, dc.slot_mapping,
                     dc.block_tables, dc.context_lens, case.scale, spec.max_len, plan=plan)
    torch.cuda.synchronize()
    assert host_bits(dc.k_cache).tobytes() == k_written
    assert host_bits(dc.v_cache).tobytes() == v_written
    assert host_bits(fused).tobytes() == host_bits(planned).tobytes()


def test_spec_verify_planned_full_size():
    _say("spec_verify_bf16 full size with a work plan")
    case = wl.build_case("spec_verify_bf16")
    spec = case.spec
    Hq, Hkv, D, T = spec.q_heads, spec.kv_heads, spec.head_dim, spec.num_query_tokens
    dc = DevCase(case)
    split = pa.default_split_tokens(Hq, Hkv, D, torch.bfloat16, num_query_tokens=T)
    plan = pa.make_plan(dc.block_tables, dc.context_lens, Hq, Hkv, D, spec.max_len,
                        torch.bfloat16, num_query_tokens=T, split_tokens=split)
    planned = torch.empty_like(dc.q)
    natural = torch.empty_like(dc.q)
    for out, p in ((planned, plan), (natural, None)):
        pa.verify(out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens,
                  case.scale, spec.max_len, split_tokens=split, plan=p)
    torch.cuda.synchronize()
    assert host_bits(planned).tobytes() == host_bits(natural).tobytes()
    want = oracle.verify(case.q, case.k_cache, case.v_cache, case.block_tables,
                         case.context_lens, case.scale, "bf16", "bf16")
    err = max_abs_err(planned, want)
    assert err < TOL["bf16"], err


def _bench_prefill_inputs():
    """The bench's chunked-prefill shapes, lengths and table (default_rng(12)); contents from
    a seeded numpy generator in stored (bf16 bit) form."""
    N, T, Hq, Hkv, D, NB = 16, 512, 16, 8, 128, 8192
    rng = np.random.default_rng(12)
    prior = rng.integers(0, 1537, size=N)
    lens = (prior + T).astype(np.int32)
    maxb = int(-(-lens.max() // 16))
    perm = rng.permutation(NB).astype(np.int32)
    table = np.full((N, maxb), -1, np.int32)
    pos = 0
    for b, L in enumerate(lens):
        nb = -(-int(L) // 16)
        table[b, :nb] = perm[pos:pos + nb]
        pos += nb
    gen = np.random.default_rng(13)
    kc = wl.f32_to_bf16_bits(gen.standard_normal((Hkv, NB, 16, D), dtype=np.float32))
    vc = wl.f32_to_bf16_bits(gen.standard_normal((Hkv, NB, 16, D), dtype=np.float32))
    q = wl.f32_to_bf16_bits(gen.standard_normal((N * T, Hq, D), dtype=np.float32))
    qs = np.arange(0, N * T + 1, T).astype(np.int32)
    return N, T, Hq, Hkv, D, prior, lens, table, kc, vc, q, qs


def test_chunked_prefill_bench_workload_planned():
    _say("chunked prefill, bench workload: 16 x 512 tokens on U{0..1536}, prefill plan")
    N, T, Hq, Hkv, D, prior, lens, table, kc, vc, q, qs = _bench_prefill_inputs()
    scale = 1.0 / float(np.sqrt(D))
    d_k, d_v, d_q = dev(kc), dev(vc), dev(q)
    d_bt, d_cl, d_qs = dev(table), dev(lens), dev(qs)
    plan = pa.make_prefill_plan(d_cl, d_qs, N * T, T, Hq, Hkv, table.shape[1])
    planned = torch.empty_like(d_q)
    natural = torch.empty_like(d_q)
    pa.prefill(planned, d_q, d_k, d_v, d_bt, d_cl, d_qs, scale, T, plan=plan)
    pa.prefill(natural, d_q, d_k, d_v, d_bt, d_cl, d_qs, scale, T)
    torch.cuda.synchronize()
    assert host_bits(planned).tobytes() == host_bits(natural).tobytes()
    got = planned.float().cpu().numpy()
    # three sequences: the longest prior, the shortest, and one drawn
    picks = sorted({int(np.argmax(prior)), int(np.argmin(prior)), 5})
    for b in picks:
        sel_q = q[qs[b]:qs[b + 1]]
        want = oracle.verify_varlen(sel_q, kc, vc, table[b:b + 1], lens[b:b + 1],
                                    np.array([0, T], np.int32), scale, "bf16", "bf16")
        err = float(np.abs(got[qs[b]:qs[b + 1]].astype(np.float64) - want).max())
        _say("  sequence", b, "prior", int(prior[b]), "max-abs err", err)
        assert err < TOL["bf16"], (b, err)
