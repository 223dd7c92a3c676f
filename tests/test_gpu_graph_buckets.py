"""Captured steps per batch-size bucket (paged_kv_gqa_pa_amd.graphs.StepGraphs).

A batch of n sequences replayed on the bucket above n (padding rows on a spare
block) must give, for its n rows, the bits of eager calls on the unpadded batch,
and leave every layer's caches equal to the eager ones outside the spare block.
Two steps in a row per bucket (the second with every context one token longer)
check that replays follow new inputs; one eager result per step is also checked
against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_gqa_pa_amd import _lib as pa
from paged_kv_gqa_pa_amd import workloads as wl
from paged_kv_gqa_pa_amd.graphs import StepGraphs
from tests.gpu_util import TOL, dev, host_bits, max_abs_err

pytestmark = pytest.mark.gpu

LAYERS, HQ, HKV, D, NB, MAXB = 3, 16, 8, 128, 1024, 40


def _say(*a):
    print("[case]", *a, flush=True)


def _caches(seed, hkv=HKV):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    kc = [torch.randn((hkv, NB, 16, D), generator=g, device="cuda").bfloat16() for _ in range(LAYERS)]
    vc = [torch.randn((hkv, NB, 16, D), generator=g, device="cuda").bfloat16() for _ in range(LAYERS)]
    return kc, vc


def _batch(rng, n, T, spare):
    """n sequences: lengths (new tokens included), tables over blocks 0 .. NB-2 (the spare
    block NB-1 is never assigned), and the slots of the T new tokens (the last T positions)."""
    lens = rng.integers(T, 400, size=n).astype(np.int32)
    perm = rng.permutation(NB - 1).astype(np.int32)
    table = wl.assign_blocks(lens + 1, perm, MAXB)        # room for the next step's token
    slots = np.array([table[b, p // 16] * 16 + p % 16
                      for b in range(n) for p in range(int(lens[b]) - T, int(lens[b]))], np.int64)
    assert spare not in table
    return lens, table, slots


def _eager(kc, vc, q, kn, vn, table, lens, slots, T, fused, scale):
    outs = []
    bt, cl, sm = dev(table), dev(lens), dev(slots)
    for l in range(LAYERS):
        o = torch.empty_like(q[l])
        if fused:
            pa.decode_append(o, q[l], kn[l], vn[l], kc[l], vc[l], sm, bt, cl, scale, MAXB * 16)
        else:
            pa.reshape_and_cache(kn[l], vn[l], kc[l], vc[l], sm)
            if T == 1:
                pa.decode(o, q[l], kc[l], vc[l], bt, cl, scale, MAXB * 16)
            else:
                pa.verify(o, q[l], kc[l], vc[l], bt, cl, scale, MAXB * 16)
        outs.append(o)
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("T,fused,hq,hkv", [(1, False, HQ, HKV), (1, True, HQ, HKV),
                                            (1, True, 12, 2),     # fused on the matrix cores
                                            (5, False, HQ, HKV),
                                            (5, False, 12, 2)])   # Qwen2 heads: 30 rows per group
def test_bucketed_steps_match_eager(T, fused, hq, hkv):
    _say("bucketed step graphs T", T, "fused", fused, "heads", hq, hkv)
    spare = NB - 1
    scale = 1.0 / float(np.sqrt(D))
    kc, vc = _caches(7, hkv)
    kc_e = [k.clone() for k in kc]
    vc_e = [v.clone() for v in vc]
    graphs = StepGraphs(kc, vc, hq, MAXB, spare, scale, buckets=(1, 4, 16, 64),
                        num_query_tokens=T, fused=fused)
    rng = np.random.default_rng(40 + T + int(fused) + hq)
    for n in (1, 3, 16, 37):
        lens, table, slots = _batch(rng, n, T, spare)
        for step in range(2):
            if step == 1:   # the next step: one more token per sequence
                lens = lens + 1
                slots = np.array([table[b, p // 16] * 16 + p % 16
                                  for b in range(n) for p in range(int(lens[b]) - T, int(lens[b]))],
                                 np.int64)
            _say("  batch", n, "bucket", graphs.bucket_for(n), "step", step)
            qshape = (n, hq, D) if T == 1 else (n, T, hq, D)
            q = [torch.randn(qshape, device="cuda").bfloat16() for _ in range(LAYERS)]
            kn = [torch.randn((n * T, hkv, D), device="cuda").bfloat16() for _ in range(LAYERS)]
            vn = [torch.randn((n * T, hkv, D), device="cuda").bfloat16() for _ in range(LAYERS)]
            want = _eager(kc_e, vc_e, q, kn, vn, table, lens, slots, T, fused, scale)
            got = graphs.step(q, kn, vn, dev(table), dev(lens), dev(slots))
            torch.cuda.synchronize()
            for l in range(LAYERS):
                assert host_bits(got[l]).tobytes() == host_bits(want[l]).tobytes(), (n, step, l)
                for a, e in ((kc[l], kc_e[l]), (vc[l], vc_e[l])):
                    assert torch.equal(a[:, :spare].view(torch.int16), e[:, :spare].view(torch.int16))
            if step == 0 and n == 3:
                # the eager reference itself against the oracle (layer 0)
                k_host = host_bits(kc_e[0])
                v_host = host_bits(vc_e[0])
                qh = host_bits(q[0])
                if T == 1:
                    ref = oracle.decode(qh, k_host, v_host, table, lens, scale, "bf16", "bf16")
                else:
                    ref = oracle.verify(qh, k_host, v_host, table, lens, scale, "bf16", "bf16")
                assert max_abs_err(want[0], ref) < TOL["bf16"]


@pytest.mark.parametrize("T,fused", [(1, False), (1, True), (5, False)])
def test_bucketed_steps_int8_match_eager(T, fused):
    """int8 caches: the requantizing write (fused with the decode, or before it), bf16
    queries and new rows; real rows and the caches and scales outside the spare block
    bit-identical to eager calls on the unpadded batch."""
    _say("bucketed step graphs, int8 cache, T", T, "fused", fused)
    hq, hkv = 12, 2
    spare = NB - 1
    scale = 1.0 / float(np.sqrt(D))
    rng0 = np.random.default_rng(70 + T + int(fused))
    kc, vc, ks, vs = [], [], [], []
    for _ in range(LAYERS):
        kcode, kscale = wl.quantize_int8_blocks(rng0.standard_normal((hkv, NB, 16, D), dtype=np.float32))
        vcode, vscale = wl.quantize_int8_blocks(rng0.standard_normal((hkv, NB, 16, D), dtype=np.float32))
        kc.append(dev(kcode))
        ks.append(dev(kscale))
        vc.append(dev(vcode))
        vs.append(dev(vscale))
    kc_e, vc_e = [k.clone() for k in kc], [v.clone() for v in vc]
    ks_e, vs_e = [k.clone() for k in ks], [v.clone() for v in vs]
    graphs = StepGraphs(kc, vc, hq, MAXB, spare, scale, buckets=(1, 4, 16, 64),
                        num_query_tokens=T, fused=fused, k_scales=ks, v_scales=vs)
    rng = np.random.default_rng(80 + T + int(fused))
    for n in (1, 3, 16, 37):
        lens, table, slots = _batch(rng, n, T, spare)
        _say("  batch", n, "bucket", graphs.bucket_for(n))
        qshape = (n, hq, D) if T == 1 else (n, T, hq, D)
        q = [torch.randn(qshape, device="cuda").bfloat16() for _ in range(LAYERS)]
        kn = [torch.randn((n * T, hkv, D), device="cuda").bfloat16() for _ in range(LAYERS)]
        vn = [torch.randn((n * T, hkv, D), device="cuda").bfloat16() for _ in range(LAYERS)]
        bt, cl, sm = dev(table), dev(lens), dev(slots)
        want = []
        for l in range(LAYERS):
            o = torch.empty_like(q[l])
            if fused:
                pa.decode_append_quant(o, q[l], kn[l], vn[l], kc_e[l], vc_e[l], ks_e[l], vs_e[l],
                                       sm, bt, cl, scale, MAXB * 16)
            else:
                pa.reshape_and_cache_quant(kn[l], vn[l], kc_e[l], vc_e[l], ks_e[l], vs_e[l], sm)
                fn = pa.decode if T == 1 else pa.verify
                fn(o, q[l], kc_e[l], vc_e[l], bt, cl, scale, MAXB * 16, ks_e[l], vs_e[l])
            want.append(o)
        got = graphs.step(q, kn, vn, bt, cl, sm)
        torch.cuda.synchronize()
        for l in range(LAYERS):
            assert host_bits(got[l]).tobytes() == host_bits(want[l]).tobytes(), (n, l)
            for a, e in ((kc[l], kc_e[l]), (vc[l], vc_e[l])):
                assert torch.equal(a[:, :spare], e[:, :spare])
            for a, e in ((ks[l], ks_e[l]), (vs[l], vs_e[l])):
                assert torch.equal(a[:, :spare], e[:, :spare])


def test_bucket_limits():
    _say("bucket limits")
    kc, vc = _caches(9)
    graphs = StepGraphs(kc[:1], vc[:1], HQ, MAXB, NB - 1, 0.1, buckets=(2, 8), use_plan=False)
    assert graphs.bucket_for(1) == 2 and graphs.bucket_for(2) == 2 and graphs.bucket_for(3) == 8
    with pytest.raises(ValueError):
        graphs.bucket_for(9)
    with pytest.raises(ValueError):
        StepGraphs(kc[:1], vc[:1], HQ, MAXB, NB, 0.1)            # spare block outside the cache
    with pytest.raises(ValueError):
        StepGraphs(kc[:1], vc[:1], HQ, MAXB, NB - 1, 0.1, num_query_tokens=2, fused=True)
    # inputs that would broadcast into the static buffers are refused
    n = 3
    q = [torch.zeros((1, HQ, D), device="cuda").bfloat16()]
    kv = [torch.zeros((n, HKV, D), device="cuda").bfloat16()]
    bt = torch.zeros((n, 4), dtype=torch.int32, device="cuda")
    cl = torch.ones(n, dtype=torch.int32, device="cuda")
    sm = torch.zeros(n, dtype=torch.int64, device="cuda")
    with pytest.raises(ValueError):
        graphs.step(q, kv, kv, bt, cl, sm)
