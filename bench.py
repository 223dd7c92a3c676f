"""Benchmark: batch-64 paged GQA decode step over 28 layer caches on one MI355X.

One step = for each of 28 layers: the new K/V token of every sequence written
into that layer's cache, then decode attention of one query token per sequence
over the context that includes it (64 sequences, 16 query / 8 KV heads,
head_dim 128, bf16, block size 16, context = 256-token prompt + U{1..256}
generated tokens, a shuffled pool of 16384 blocks per layer, one shared block
table).  The timed step runs each layer as one pa_decode_append launch (the
write and the decode in one kernel); the same step as pa_reshape_and_cache +
pa_decode (two launches per layer) is timed beside it.  Each step first makes one work plan
(pa_plan: the step's (sequence, piece) units ordered longest first, shared by
the 28 layers); ``--no-plan`` starts the work in the natural order instead.
The step is captured once in a HIP graph and replayed (the pages' change 4:
graphs per batch bucket); ``--eager`` launches every kernel from Python
instead.

Printed: one JSON line with tokens/s for the whole step (``value``), the decode
kernel's achieved HBM bandwidth on algorithmic bytes against the 8 TB/s peak
(``roofline``), the CPU oracle timed on a bounded sample (``cpu_baseline``),
and (``other_workloads``) the per-call time, bandwidth and roofline fraction
of the other seeded workloads: the Qwen2-1.5B-shaped decode, the speculative
verify and the long-context int8 decode.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

WORKLOAD = "batch64_28layer_bf16"
METRIC = "paged GQA decode attention: achieved HBM GB/s (% of peak) + tokens/s at batch 64"
HBM_PEAK_GBPS = 8000.0
ROTATION_BYTES = 1 << 30
# The five seeded workloads by their configuration keys.
CONFIG_KEYS = {"tiny_fp32": "C1", "qwen2_1p5b_bf16": "C2", "batch64_28layer_bf16": "C3",
               "spec_verify_bf16": "C4", "long_ctx_int8": "C5"}


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--split", type=int, default=0, help="split_tokens (0 = library default)")
    p.add_argument("--eager", action="store_true", help="launch from Python instead of a graph")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-buckets", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="target CPU time of the oracle baseline sample (batch-64 workload)")
    p.add_argument("--cpu-seconds-other", type=float, default=3.0,
                   help="target CPU time per leg of the oracle baselines of the other workloads")
    p.add_argument("--decode-reps", type=int, default=20,
                   help="graph replays of the 28 decode launches for the per-kernel timing")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run one 256 MiB device-to-device copy (known bytes) so hardware "
                        "byte counters can be scaled")
    p.add_argument("--no-plan", action="store_true",
                   help="start the attention work in the natural order instead of a work plan")
    p.add_argument("--natural", action="store_true",
                   help="also time the 28 decode launches in the natural order (same kernel "
                        "symbol as the planned launches: leave off for profiled runs)")
    p.add_argument("--no-other-workloads", action="store_true",
                   help="skip the per-call timings of the other workloads")
    p.add_argument("--traffic-file", default=os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                         "profiles", "pa_decode_batch64_traffic.json"))
    return p.parse_args()


def algorithmic_bytes(lens, q_heads, kv_heads, head_dim, elem=2):
    """Bytes pa_decode must move for one layer: K and V of exactly L_b positions per
    (sequence, KV head), q in, out, the used block-table entries and the lengths."""
    lens = np.asarray(lens, np.int64)
    kv = int(lens.sum()) * kv_heads * head_dim * elem * 2
    qo = len(lens) * q_heads * head_dim * elem * 2
    tables = int(((lens + 15) // 16).sum()) * 4 + len(lens) * 4
    return kv + qo + tables


def attention_bytes(lens, T, q_heads, kv_heads, head_dim, kv_elem, q_elem=2):
    """Algorithmic bytes of one pa_decode / pa_verify call: K and V of exactly L_b
    positions per (sequence, KV head), q in and out, the used table entries, the
    lengths, and for an int8 cache the two fp32 scales of each used block."""
    lens = np.asarray(lens, np.int64)
    blocks = int(((lens + 15) // 16).sum())
    kv = int(lens.sum()) * kv_heads * head_dim * kv_elem * 2
    qo = len(lens) * T * q_heads * head_dim * q_elem * 2
    scales = blocks * kv_heads * 8 if kv_elem == 1 else 0
    return kv + qo + blocks * 4 + len(lens) * 4 + scales


def bucket_timing(torch, pa, kc, vc, qs, nks, nvs, bt, cl, sm, table, scale, reps, sizes=(1, 8, 64),
                  fused=True):
    """The batch-64 step (28 x write + decode: one pa_decode_append launch per layer, or
    with fused=False pa_reshape_and_cache + pa_decode; a pa_plan first in the buckets
    whose units outnumber the CUs, StepGraphs' default) captured per batch-size bucket by
    StepGraphs, for batches of the first n sequences; µs per step from graph replays
    (inputs copied in once; each replay rewrites the same new-token slots)."""
    from paged_kv_gqa_pa_amd.graphs import StepGraphs
    NB = kc[0].shape[1]
    used = np.zeros(NB, bool)
    used[table[table >= 0]] = True
    spare = int(np.flatnonzero(~used)[-1])
    sg = StepGraphs(kc, vc, qs[0].shape[1], table.shape[1], spare, scale, buckets=sizes,
                    fused=fused)
    out = {}
    for n in sizes:
        sg.step([q[:n] for q in qs], [k[:n] for k in nks], [v[:n] for v in nvs], bt[:n], cl[:n],
                sm[:n])
        for _ in range(3):
            sg.replay(n)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            sg.replay(n)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        out[str(n)] = {"us_per_step": round(us, 1), "tokens_per_s": round(n / (us * 1e-6), 1)}
        print(f"[bench] step graph{'' if fused else ' (write, then decode)'}, batch {n}: "
              f"{us:.1f} us/step, {n / (us * 1e-6):.0f} tokens/s", flush=True)
    del sg
    return out


def other_workloads(torch, pa, wl, dev, reps=10, use_plan=True):
    """Per-call timings of the other seeded workloads.  Each call reads its own
    replica of the caches (enough replicas to pass 1 GB per round, far beyond the
    256 MB last-level cache), launched from one HIP graph; events on the launch
    stream.  Cache contents are random (the timing does not depend on them); the
    lengths and block tables are the seeded ones."""
    out = {}
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32, "int8": torch.int8}
    for name in ("tiny_fp32", "qwen2_1p5b_bf16", "spec_verify_bf16", "spec_verify_varlen_bf16",
                 "long_ctx_int8"):
        varlen = name == "spec_verify_varlen_bf16"
        spec = wl.CONFIGS["spec_verify_bf16" if varlen else name]
        lens, table = wl.structure(spec)
        counts = None
        if varlen:
            # the speculative workload with 1..5 new tokens per sequence (seeded): the
            # prior context is kept, so each length becomes prior + T_b
            counts = np.random.default_rng(spec.seed + 100).integers(1, 6, size=spec.num_seqs)
            lens = (lens - spec.num_query_tokens + counts).astype(np.int32)
        N, T, Hq, Hkv, D, NB = (spec.num_seqs, spec.num_query_tokens, spec.q_heads,
                                spec.kv_heads, spec.head_dim, spec.num_blocks)
        kdt = tdt[spec.kv_dtype]
        elem = {torch.bfloat16: 2, torch.float32: 4, torch.int8: 1}[kdt]
        q_elem = 4 if spec.q_dtype == "f32" else 2
        # Bytes one call touches (its K/V rows, q, out, table entries, lengths, scales);
        # replicas enough that one rotation touches at least 1 GiB of distinct memory, four
        # times the 256 MB last-level cache.  The tiny workload (58 KB, launch-bound)
        # runs on one copy: its time is reported with no roofline claim.
        touched = (attention_bytes(lens, 1, Hq, Hkv, D, elem, q_elem) +
                   (int(counts.sum()) if varlen else N * T) * Hq * D * q_elem * 2 -
                   N * Hq * D * q_elem * 2)
        R = 1 if name == "tiny_fp32" else int(np.ceil(ROTATION_BYTES / touched))

        def mk():
            if kdt == torch.int8:
                return torch.randint(-127, 128, (Hkv, NB, 16, D), device=dev, dtype=torch.int8)
            return torch.randn((Hkv, NB, 16, D), device=dev, dtype=kdt)
        kc = [mk() for _ in range(R)]
        vc = [mk() for _ in range(R)]
        ks = vs = None
        if kdt == torch.int8:
            ks = torch.rand((Hkv, NB), device=dev) * 0.02 + 0.01
            vs = torch.rand((Hkv, NB), device=dev) * 0.02 + 0.01
        bt = torch.from_numpy(table).to(dev)
        cl = torch.from_numpy(lens).to(dev)
        if varlen:
            total = int(counts.sum())
            q = torch.randn((total, Hq, D), device=dev, dtype=torch.bfloat16)
            qs = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).to(dev)
        else:
            total = N * T
            q = torch.randn((N, T, Hq, D) if T > 1 else (N, Hq, D), device=dev,
                            dtype=torch.float32 if spec.q_dtype == "f32" else torch.bfloat16)
        o = torch.empty_like(q)
        split = pa.default_split_tokens(Hq, Hkv, D, kdt, num_query_tokens=T)
        wsb = pa.workspace_size(N, T, Hq, Hkv, D, spec.max_len, kdt, split)
        ws = torch.zeros(max(256, wsb), dtype=torch.uint8, device=dev)
        fn = pa.verify if T > 1 else pa.decode
        # One work plan for the call's tables and lengths (made once, as once per step),
        # where it pays: lengths that vary on a bandwidth-bound launch.  The Qwen2-shaped
        # decode is latency-bound (64 workgroups; the plan row's read delays the query
        # load by ~0.2 us) and the long-context lengths are all equal.
        plan = None
        if use_plan and name == "spec_verify_bf16":
            plan = pa.make_plan(bt, cl, Hq, Hkv, D, spec.max_len, kdt, num_query_tokens=T,
                                split_tokens=split)

        # At least 16 calls per graph, so that the replay's own launch cost is spread
        # over many calls; consecutive calls still read different replicas.
        cycles = -(-16 // R)

        def calls():
            for r in [r for _ in range(cycles) for r in range(R)]:
                if varlen:
                    pa.verify_varlen(o, q, kc[r], vc[r], bt, cl, qs, 1.0 / float(np.sqrt(D)),
                                     spec.max_len, T, split_tokens=split, workspace=ws)
                else:
                    fn(o, q, kc[r], vc[r], bt, cl, 1.0 / float(np.sqrt(D)), spec.max_len, ks, vs,
                       split_tokens=split, workspace=ws, plan=plan)
        calls()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            calls()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * R * cycles)
        alg = touched
        gbps = alg / (us * 1e-6) / 1e9
        out[name] = {"config": CONFIG_KEYS.get(name, CONFIG_KEYS["spec_verify_bf16"] + " (1..5 tokens)"),
                     "us_per_call": round(us, 2), "algorithmic_bytes": alg,
                     "hbm_gbps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "query_tokens_per_s": round(total / (us * 1e-6), 1),
                     "rotation": {"replicas": R, "bytes_touched_per_call": alg,
                                  "bytes_per_rotation": R * alg, "calls_per_graph": R * cycles},
                     "split_tokens": split, "work_plan": plan is not None,
                     "kernel": "rows_pass1" if (T > 1 or elem == 1 or Hq // Hkv >= 4) else "decode_pass1",
                     "shape": f"N={N} T={'1..5 per sequence, ' + str(total) + ' rows' if varlen else T} "
                              f"Hq={Hq} Hkv={Hkv} D={D} kv={spec.kv_dtype}"}
        if name == "tiny_fp32":
            out[name]["note"] = "launch-bound (58 KB per call): time reported, no roofline claim"
            del out[name]["frac"]
        print(f"[bench] {name}: {us:.2f} us/call, {gbps:.0f} GB/s ({100 * gbps / HBM_PEAK_GBPS:.1f}%), "
              f"{R} replicas x {alg / 1e6:.1f} MB per rotation", flush=True)
        if name != "tiny_fp32":
            out[name]["read_pattern"] = read_pattern_timing(torch, kc, vc, bt, cl, spec.max_len,
                                                            split, R, cycles, reps, us)
        if name == "long_ctx_int8":
            out[name]["append_step"] = int8_append_timing(torch, pa, dev, kc, vc, ks, vs, q, o, bt,
                                                          cl, lens, table, spec, split, ws, R,
                                                          cycles, reps)
        del kc, vc, g
        torch.cuda.empty_cache()
    out["int8_requant_write"] = requant_write_timing(torch, pa, dev, reps)
    out["chunked_prefill_bf16"] = prefill_timing(torch, pa, dev, reps)
    return out


def int8_append_timing(torch, pa, dev, kc, vc, ks, vs, q, o, bt, cl, lens, table, spec, split,
                       ws, R, cycles, reps):
    """A decode step over the long-context int8 caches with its cache write: one new
    bf16 token per sequence written with requantization of its block and attended
    over, as one pa_decode_append_quant launch and as pa_reshape_and_cache_quant +
    pa_decode, over the same replicas (events on the launch stream)."""
    N, Hkv, D = spec.num_seqs, spec.kv_heads, spec.head_dim
    g_ = torch.Generator(device=dev)
    g_.manual_seed(spec.seed + 200)
    nk = torch.randn((N, Hkv, D), device=dev, dtype=torch.bfloat16, generator=g_)
    nv = torch.randn((N, Hkv, D), device=dev, dtype=torch.bfloat16, generator=g_)
    from paged_kv_gqa_pa_amd import workloads as wl
    sm = torch.from_numpy(wl.slots_for_positions(table, np.arange(N),
                                                 lens.astype(np.int64) - 1)).to(dev)
    scale = 1.0 / float(np.sqrt(D))
    order = [r for _ in range(cycles) for r in range(R)]

    def fused():
        for r in order:
            pa.decode_append_quant(o, q, nk, nv, kc[r], vc[r], ks, vs, sm, bt, cl, scale,
                                   spec.max_len, split_tokens=split, workspace=ws)

    def two_calls():
        for r in order:
            pa.reshape_and_cache_quant(nk, nv, kc[r], vc[r], ks, vs, sm)
            pa.decode(o, q, kc[r], vc[r], bt, cl, scale, spec.max_len, ks, vs,
                      split_tokens=split, workspace=ws)
    res = {"entry_points": "pa_decode_append_quant vs pa_reshape_and_cache_quant + pa_decode",
           "new_rows": "bf16"}
    for key, fn in (("fused_us_per_call", fused), ("write_then_decode_us_per_call", two_calls)):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        res[key] = round(e0.elapsed_time(e1) * 1e3 / (reps * len(order)), 2)
        del g
    print(f"[bench]   with the requantizing write of the new tokens: "
          f"{res['fused_us_per_call']:.2f} us in one launch, "
          f"{res['write_then_decode_us_per_call']:.2f} us as write + decode", flush=True)
    return res


def read_pattern_timing(torch, kc, vc, bt, cl, max_len, split, R, cycles, reps, us_call):
    """The call's own K/V tile reads without arithmetic (libpa_probe's tile_read: the same
    units, pieces and tiles in the natural order, nothing computed or written) over the
    same replicas, with four and with eight waves per workgroup: the read pattern's own
    time, against which the attention call (pass 1 and, with pieces, the merge) is set."""
    from paged_kv_gqa_pa_amd import _probe as probe
    sink = torch.zeros(1, dtype=torch.int32, device=bt.device)
    res = {}
    for waves in (4, 8):
        def reads():
            for r in [r for _ in range(cycles) for r in range(R)]:
                probe.tile_read(kc[r], vc[r], bt, cl, max_len, split, sink, waves=waves)
        reads()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            reads()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        res[f"{waves}_waves_us"] = round(e0.elapsed_time(e1) * 1e3 / (reps * R * cycles), 2)
        del g
    best = min(res.values())
    res["call_over_best_pattern_us"] = round(us_call - best, 2)
    print(f"[bench]   its tile reads alone: {res['4_waves_us']:.2f} us (4 waves), "
          f"{res['8_waves_us']:.2f} us (8 waves)", flush=True)
    return res


def prefill_timing(torch, pa, dev, reps=10, calls=8):
    """Chunked prefill (pa_prefill, started from a prefill work plan; the natural order
    is timed beside it): 16 sequences, each a 512-token chunk on top of a seeded prior
    context U{0..1536}, 16 query / 8 KV heads, head_dim 128, bf16 cache of 8192 blocks.  Reported against the bf16 matrix-core peak (the causal products are the
    work: 4 * head_dim flops per (query row, visible position)) and as HBM bytes (K/V of
    each sequence once, q, out, tables)."""
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
    g_ = torch.Generator(device=dev)
    g_.manual_seed(13)
    kc = torch.randn((Hkv, NB, 16, D), device=dev, dtype=torch.bfloat16, generator=g_)
    vc = torch.randn((Hkv, NB, 16, D), device=dev, dtype=torch.bfloat16, generator=g_)
    q = torch.randn((N * T, Hq, D), device=dev, dtype=torch.bfloat16, generator=g_)
    o = torch.empty_like(q)
    bt = torch.from_numpy(table).to(dev)
    cl = torch.from_numpy(lens).to(dev)
    qs = torch.from_numpy(np.arange(0, N * T + 1, T).astype(np.int32)).to(dev)

    # one prefill work plan (tiles longest first), made once for the call's offsets and lengths
    plan = pa.make_prefill_plan(cl, qs, N * T, T, Hq, Hkv, maxb)

    def timed(use_plan):
        def run():
            for _ in range(calls):
                pa.prefill(o, q, kc, vc, bt, cl, qs, 1.0 / float(np.sqrt(D)), T,
                           plan=plan if use_plan else None)
        run()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * calls)
    us_natural = timed(False)
    us = timed(True)
    visible = int(sum(int(p) * T + T * (T + 1) // 2 for p in prior))   # per head
    flops = 4 * D * Hq * visible
    alg = (int(lens.sum()) * Hkv * D * 2 * 2 + 2 * N * T * Hq * D * 2 +
           int(((lens + 15) // 16).sum()) * 4 + N * 8)
    tflops = flops / (us * 1e-6) / 1e12
    res = {"shape": f"N={N} chunk={T} prior=U{{0..1536}} Hq={Hq} Hkv={Hkv} D={D} kv=bf16",
           "us_per_call": round(us, 2), "flops": flops, "tflops": round(tflops, 1),
           "mfma_frac": round(tflops / 2500.0, 4), "algorithmic_bytes": alg,
           "hbm_gbps": round(alg / (us * 1e-6) / 1e9, 1), "query_tokens_per_s": round(N * T / (us * 1e-6), 1),
           "kernel": "prefill_rows", "work_plan": True,
           "natural_order_us_per_call": round(us_natural, 2)}
    print(f"[bench] chunked prefill: {us:.2f} us/call, {tflops:.1f} TFLOP/s "
          f"({100 * tflops / 2500.0:.1f}% of bf16 matrix peak; natural order {us_natural:.2f} us)",
          flush=True)
    del kc, vc
    torch.cuda.empty_cache()
    return res


def requant_write_timing(torch, pa, dev, reps=10, calls=20):
    """Decode-step cache write into an int8 cache that requantizes each target
    block (64 tokens, 8 KV heads, head_dim 128, bf16 rows; every token in its
    own block of a 8192-block cache), beside the plain bf16 row copy at the same
    shape.  Both launched from a HIP graph of `calls` writes; events on the
    launch stream."""
    T, H, D, NB = 64, 8, 128, 8192
    g_ = torch.Generator(device=dev)
    g_.manual_seed(11)
    kc = torch.randint(-127, 128, (H, NB, 16, D), dtype=torch.int8, device=dev, generator=g_)
    vc = torch.randint(-127, 128, (H, NB, 16, D), dtype=torch.int8, device=dev, generator=g_)
    ks = torch.rand((H, NB), device=dev, generator=g_) * 0.02 + 0.01
    vs = torch.rand((H, NB), device=dev, generator=g_) * 0.02 + 0.01
    key = torch.randn((T, H, D), device=dev, dtype=torch.bfloat16, generator=g_)
    val = torch.randn((T, H, D), device=dev, dtype=torch.bfloat16, generator=g_)
    blocks = torch.randperm(NB, device=dev, generator=g_)[:T]
    slots = (blocks * 16 + torch.randint(0, 16, (T,), device=dev, generator=g_)).to(torch.int64)
    kb = torch.zeros((H, NB, 16, D), dtype=torch.bfloat16, device=dev)
    vb = torch.zeros_like(kb)
    res = {"shape": f"T={T} Hkv={H} D={D} num_blocks={NB} rows=bf16"}
    for name, fn in (("requant_us_per_call", lambda: pa.reshape_and_cache_quant(key, val, kc, vc, ks, vs, slots)),
                     ("bf16_copy_us_per_call", lambda: pa.reshape_and_cache(key, val, kb, vb, slots))):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(calls):
                fn()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        res[name] = round(e0.elapsed_time(e1) * 1e3 / (reps * calls), 2)
    # bytes: read and write the block's codes, read the new rows and scales (K and V)
    res["algorithmic_bytes"] = T * H * 2 * (2 * 16 * D + 2 * D + 2 * 4) + 8 * T
    print(f"[bench] int8 requant write: {res['requant_us_per_call']} us/call "
          f"(bf16 copy {res['bf16_copy_us_per_call']} us)", flush=True)
    del kc, vc, kb, vb
    torch.cuda.empty_cache()
    return res


def cache_write_bytes(num_tokens, kv_heads, head_dim, elem=2):
    return num_tokens * kv_heads * head_dim * elem * 2 * 2 + num_tokens * 8


_CPU_CASE = None


def _oracle_one_seq(b):
    """Worker: the oracle's decode of sequence b of the sampled layer (all its heads)."""
    import oracle
    c = _CPU_CASE
    return oracle.decode(c.q[b:b + 1], c.k_cache, c.v_cache, c.block_tables[b:b + 1],
                         c.context_lens[b:b + 1], c.scale, "bf16", "bf16")


def _pool_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:  # pragma: no cover
        pass


def cpu_baseline(target_s: float):
    """The fp64 oracle on a bounded sample of the same workload: layer 0's decode
    repeated for about target_s seconds, (i) on one core with one BLAS thread,
    (ii) on every host core through a process pool over sequences (one BLAS
    thread per worker, at most 16 workers).  Runs before anything touches the
    GPU, so the pool's forked workers hold no device state."""
    global _CPU_CASE
    import multiprocessing as mp
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    import oracle
    from paged_kv_gqa_pa_amd import workloads as wl
    case = wl.build_case(WORKLOAD, layer=0)
    spec = case.spec
    alg = algorithmic_bytes(case.context_lens, spec.q_heads, spec.kv_heads, spec.head_dim)
    ctx = threadpool_limits(1) if threadpool_limits else None
    try:
        n_layers = 0
        t0 = time.perf_counter()
        while True:
            oracle.decode(case.q, case.k_cache, case.v_cache, case.block_tables,
                          case.context_lens, case.scale, "bf16", "bf16")
            n_layers += 1
            el = time.perf_counter() - t0
            if el >= target_s:
                break
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    per_layer = el / n_layers
    tok_s = spec.num_seqs / (per_layer * spec.layers)
    gbps = alg / per_layer / 1e9
    res = {"value": round(tok_s, 2), "unit": "tokens/s", "cores": 1, "kind": "oracle",
           "sample": f"{n_layers} decode passes of layer 0 (64 seqs, 16q/8kv heads, D=128) in "
                     f"{el:.1f} s; tokens/s = 64 / (28 x time per layer); cache write not timed; "
                     f"{gbps:.3f} GB/s on the same algorithmic bytes",
           "cpu_model": _cpu_model(), "host_cpus": os.cpu_count()}
    workers = max(1, min(16, os.cpu_count() or 1))
    _CPU_CASE = case
    try:
        with mp.get_context("fork").Pool(workers, initializer=_pool_init) as pool:
            pool.map(_oracle_one_seq, range(min(workers, spec.num_seqs)))   # start-up
            n_all = 0
            t0 = time.perf_counter()
            while True:
                pool.map(_oracle_one_seq, range(spec.num_seqs), chunksize=2)
                n_all += 1
                el_all = time.perf_counter() - t0
                if el_all >= target_s:
                    break
        per_all = el_all / n_all
        res["all_cores"] = {
            "value": round(spec.num_seqs / (per_all * spec.layers), 2), "unit": "tokens/s",
            "cores": workers, "kind": "oracle",
            "sample": f"{n_all} decode passes of layer 0 over a {workers}-process pool "
                      f"(one sequence per task) in {el_all:.1f} s; {alg / per_all / 1e9:.3f} GB/s"}
    finally:
        _CPU_CASE = None
    return res


# The oracle per (sequence, KV head) unit of the other configurations: the cases are
# built before the pool forks, so the workers see them.
_CPU_CASES = {}


def _oracle_unit(name, b, g):
    """The oracle's result for sequence b, KV head g (its G query heads) of a config."""
    import oracle
    c = _CPU_CASES[name]
    spec = c.spec
    G = spec.q_heads // spec.kv_heads
    hs = slice(g * G, (g + 1) * G)
    ks = None if c.k_scale is None else c.k_scale[g:g + 1]
    vs = None if c.v_scale is None else c.v_scale[g:g + 1]
    if spec.num_query_tokens > 1:
        return oracle.verify(c.q[b:b + 1, :, hs], c.k_cache[g:g + 1], c.v_cache[g:g + 1],
                             c.block_tables[b:b + 1], c.context_lens[b:b + 1], c.scale,
                             spec.q_dtype, spec.kv_dtype, ks, vs)
    return oracle.decode(c.q[b:b + 1, hs], c.k_cache[g:g + 1], c.v_cache[g:g + 1],
                         c.block_tables[b:b + 1], c.context_lens[b:b + 1], c.scale,
                         spec.q_dtype, spec.kv_dtype, ks, vs)


def _oracle_unit_task(args):
    return _oracle_unit(*args).shape


def oracle_config_baselines(target_s, workers):
    """The fp64 oracle timed on every other configuration (C1, C2, C4, C5) over its
    (sequence, KV head) units: (i) one core, one BLAS thread, units in order until
    about target_s seconds have passed (a whole call or a bounded part of one);
    (ii) a process pool of `workers` processes over the units, whole calls repeated
    for about target_s seconds.  Query tokens per second and GB/s on the same
    algorithmic bytes the GPU figures use."""
    import multiprocessing as mp
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    from paged_kv_gqa_pa_amd import workloads as wl
    names = ("tiny_fp32", "qwen2_1p5b_bf16", "spec_verify_bf16", "long_ctx_int8")
    for n in names:
        _CPU_CASES[n] = wl.build_case(n)
    out = {}
    try:
        for n in names:
            c = _CPU_CASES[n]
            spec = c.spec
            units = [(n, b, g) for b in range(spec.num_seqs) for g in range(spec.kv_heads)]
            tokens = spec.num_seqs * spec.num_query_tokens
            kv_elem = {"f32": 4, "bf16": 2, "int8": 1}[spec.kv_dtype]
            alg = attention_bytes(c.context_lens, spec.num_query_tokens, spec.q_heads,
                                  spec.kv_heads, spec.head_dim, kv_elem,
                                  4 if spec.q_dtype == "f32" else 2)
            ctx = threadpool_limits(1) if threadpool_limits else None
            try:
                done, t0 = 0, time.perf_counter()
                while True:
                    _oracle_unit(*units[done % len(units)])
                    done += 1
                    el = time.perf_counter() - t0
                    if el >= target_s:
                        break
            finally:
                if ctx is not None:
                    ctx.__exit__(None, None, None)
            per_call = el / done * len(units)
            out[CONFIG_KEYS[n]] = {
                "workload": n, "unit": "query tokens/s", "kind": "oracle",
                "algorithmic_bytes": alg,
                "one_core": {"value": round(tokens / per_call, 3), "cores": 1,
                             "gbps": round(alg / per_call / 1e9, 4),
                             "sample": f"{done} (sequence, KV head) units (a call has "
                                       f"{len(units)}) in {el:.1f} s on one core"}}
        with mp.get_context("fork").Pool(workers, initializer=_pool_init) as pool:
            pool.map(_oracle_unit_task, [("tiny_fp32", 0, 0)] * workers)   # start-up
            for n in names:
                spec = _CPU_CASES[n].spec
                units = [(n, b, g) for b in range(spec.num_seqs) for g in range(spec.kv_heads)]
                r = out[CONFIG_KEYS[n]]
                calls, t0 = 0, time.perf_counter()
                while True:
                    pool.map(_oracle_unit_task, units, chunksize=max(1, len(units) // (4 * workers)))
                    calls += 1
                    el = time.perf_counter() - t0
                    if el >= target_s:
                        break
                per_call = el / calls
                tokens = spec.num_seqs * spec.num_query_tokens
                r["all_cores"] = {"value": round(tokens / per_call, 3), "cores": workers,
                                  "gbps": round(r["algorithmic_bytes"] / per_call / 1e9, 4),
                                  "sample": f"{calls} whole calls over a {workers}-process pool "
                                            f"in {el:.1f} s"}
    finally:
        _CPU_CASES.clear()
    return out


def _cpu_model():
    """The host CPU as lscpu names it (model name, family / model / stepping, sockets and
    cores), else /proc/cpuinfo's model name."""
    import subprocess
    info = {}
    try:
        res = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10)
        for line in res.stdout.splitlines():
            if ":" in line:
                k, v = line.split(":", 1)
                info[k.strip()] = v.strip()
    except (OSError, subprocess.SubprocessError):
        pass
    name = info.get("Model name")
    if not name:
        try:
            with open("/proc/cpuinfo") as f:
                for line in f:
                    if line.startswith("model name"):
                        name = line.split(":", 1)[1].strip()
                        break
        except OSError:
            pass
    parts = [name or "unknown"]
    if info.get("CPU family"):
        parts.append(f"family {info['CPU family']} model {info.get('Model', '?')} "
                     f"stepping {info.get('Stepping', '?')}")
    if info.get("Socket(s)"):
        parts.append(f"{info['Socket(s)']} socket(s) x {info.get('Core(s) per socket', '?')} cores x "
                     f"{info.get('Thread(s) per core', '?')} threads")
    return "; ".join(parts)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the decode path is measured on a single MI355X "
              "(multi-GPU sharding is a design note, not a measured path).", file=sys.stderr)
        sys.exit(2)

    cpu = None
    if not args.no_cpu_baseline:
        # before the GPU is touched: the all-cores legs fork worker processes
        print("[bench] cpu baseline ...", flush=True)
        cpu = cpu_baseline(args.cpu_seconds)
        print(f"[bench] cpu baseline: {cpu['value']} tokens/s on 1 core, "
              f"{cpu['all_cores']['value']} on {cpu['all_cores']['cores']}", flush=True)
        cpu["other_configs"] = oracle_config_baselines(args.cpu_seconds_other,
                                                       cpu["all_cores"]["cores"])
        for k, r in cpu["other_configs"].items():
            print(f"[bench] cpu baseline {k} {r['workload']}: {r['one_core']['value']} query "
                  f"tokens/s on 1 core, {r['all_cores']['value']} on {r['all_cores']['cores']}",
                  flush=True)

    import torch
    from paged_kv_gqa_pa_amd import _lib as pa
    from paged_kv_gqa_pa_amd import _probe as probe
    from paged_kv_gqa_pa_amd import workloads as wl

    pa.lib()  # fail loudly if the HIP library is missing
    probe.lib()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    spec = wl.CONFIGS[WORKLOAD]
    N, Hq, Hkv, D, NB, Lyr = spec.num_seqs, spec.q_heads, spec.kv_heads, spec.head_dim, spec.num_blocks, spec.layers
    lens, table = wl.structure(spec)
    slots = wl.slots_for_positions(table, np.arange(N), lens.astype(np.int64) - 1)
    print(f"[bench] {WORKLOAD}: N={N} Hq={Hq} Hkv={Hkv} D={D} layers={Lyr} "
          f"L in [{lens.min()},{lens.max()}] mean {lens.mean():.1f}", flush=True)

    gen = torch.Generator(device=dev)
    gen.manual_seed(spec.seed)
    bt = torch.from_numpy(table).to(dev)
    cl = torch.from_numpy(lens).to(dev)
    sm = torch.from_numpy(slots).to(dev)
    kc, vc, qs, nks, nvs, outs = [], [], [], [], [], []
    for _ in range(Lyr):
        kc.append(torch.randn((Hkv, NB, 16, D), generator=gen, device=dev, dtype=torch.bfloat16))
        vc.append(torch.randn((Hkv, NB, 16, D), generator=gen, device=dev, dtype=torch.bfloat16))
        qs.append(torch.randn((N, Hq, D), generator=gen, device=dev, dtype=torch.bfloat16))
        nks.append(torch.randn((N, Hkv, D), generator=gen, device=dev, dtype=torch.bfloat16))
        nvs.append(torch.randn((N, Hkv, D), generator=gen, device=dev, dtype=torch.bfloat16))
        outs.append(torch.empty((N, Hq, D), device=dev, dtype=torch.bfloat16))
    max_len = spec.max_len
    ws_bytes = pa.workspace_size(N, 1, Hq, Hkv, D, max_len, torch.bfloat16, args.split)
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    # One work plan per step (the step's tables and lengths serve all 28 layers).
    plan = None
    if not args.no_plan:
        plan = torch.empty(pa.plan_size(N, 1, Hq, Hkv, D, max_len, torch.bfloat16, args.split),
                           dtype=torch.uint8, device=dev)

    def make_plan():
        if plan is not None:
            pa.make_plan(bt, cl, Hq, Hkv, D, max_len, torch.bfloat16, split_tokens=args.split,
                         plan=plan)
    scale = 1.0 / float(np.sqrt(D))
    torch.cuda.synchronize()
    print(f"[bench] caches ready: {2 * Lyr * kc[0].numel() * 2 / 2**30:.1f} GiB, "
          f"workspace {ws_bytes} B", flush=True)

    def step():
        make_plan()
        for l in range(Lyr):
            pa.reshape_and_cache(nks[l], nvs[l], kc[l], vc[l], sm)
            pa.decode(outs[l], qs[l], kc[l], vc[l], bt, cl, scale, max_len,
                      split_tokens=args.split, workspace=ws, plan=plan)

    def step_fused():
        make_plan()
        for l in range(Lyr):
            pa.decode_append(outs[l], qs[l], nks[l], nvs[l], kc[l], vc[l], sm, bt, cl, scale,
                             max_len, split_tokens=args.split, workspace=ws, plan=plan)

    def decode_only(use_plan=True):
        for l in range(Lyr):
            pa.decode(outs[l], qs[l], kc[l], vc[l], bt, cl, scale, max_len,
                      split_tokens=args.split, workspace=ws, plan=plan if use_plan else None)

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for _ in range(max(1, args.warmup)):
            step()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()

    run_natural = None
    if args.eager:
        run_step = step
        run_fused = step_fused
        run_decode = decode_only
        if args.natural and plan is not None:
            run_natural = lambda: decode_only(False)
    else:
        g_step = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_step):
            step()
        g_fused = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_fused):
            step_fused()
        g_dec = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_dec):
            decode_only()
        run_step = g_step.replay
        run_fused = g_fused.replay
        run_decode = g_dec.replay
        if args.natural and plan is not None:
            g_nat = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_nat):
                decode_only(False)
            run_natural = g_nat.replay
        for _ in range(max(1, args.warmup)):
            run_step()
        torch.cuda.synchronize()
    print("[bench] warm", flush=True)
    if args.calibrate_copy:
        src = torch.ones(256 << 18, dtype=torch.float32, device=dev)   # 256 MiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print("[bench] calibration copy: 256 MiB read + 256 MiB written", flush=True)
        del src, dst

    # Whole step: W untimed steps, then K steps back to back between two events,
    # synchronised on both sides: the mean.  A second pass of K steps with an
    # event after every step gives the per-step median, min and max (each of
    # those events costs the stream a few µs between steps, so these run a
    # little above the mean).
    def timed_steps(run):
        for _ in range(max(1, args.warmup)):
            run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            run()
        e1.record()
        torch.cuda.synchronize()
        mean = e0.elapsed_time(e1) / args.steps
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        ev[0].record()
        for i in range(args.steps):
            run()
            ev[i + 1].record()
        torch.cuda.synchronize()
        return mean, sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))

    # The step: per layer, pa_decode_append writes the new token's K and V into
    # the layer's cache and attends over the context that includes it (one launch).
    ms_step, per_step = timed_steps(run_fused)
    tok_s = N / (ms_step / 1e3)
    print(f"[bench] step (write + decode in one launch per layer) {ms_step * 1e3:.1f} us", flush=True)
    # The same step as two launches per layer: pa_reshape_and_cache, then pa_decode.
    ms_split, per_split = timed_steps(run_step)
    print(f"[bench] step (pa_reshape_and_cache + pa_decode per layer) {ms_split * 1e3:.1f} us",
          flush=True)

    # Decode kernel alone: back-to-back launches over the 28 layers (distinct caches,
    # 2.8 GB per pass, far beyond the 256 MB last-level cache), events on the launch stream.
    torch.cuda.synchronize()
    # the mean from the passes back to back between two events; the per-pass
    # spread from a second run with an event after every pass
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    d0.record()
    for _ in range(args.decode_reps):
        run_decode()
    d1.record()
    torch.cuda.synchronize()
    us_decode = d0.elapsed_time(d1) * 1e3 / (args.decode_reps * Lyr)
    dv = [torch.cuda.Event(enable_timing=True) for _ in range(args.decode_reps + 1)]
    dv[0].record()
    for i in range(args.decode_reps):
        run_decode()
        dv[i + 1].record()
    torch.cuda.synchronize()
    per_pass = sorted(dv[i].elapsed_time(dv[i + 1]) * 1e3 / Lyr for i in range(args.decode_reps))
    bytes_launch = algorithmic_bytes(lens, Hq, Hkv, D)
    gbps = bytes_launch / (us_decode * 1e-6) / 1e9
    print(f"[bench] decode {us_decode:.2f} us/launch, {gbps:.0f} GB/s"
          f"{' (work plan)' if plan is not None else ''}", flush=True)
    natural = None
    if run_natural is not None:
        torch.cuda.synchronize()
        n0, n1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n0.record()
        for _ in range(args.decode_reps):
            run_natural()
        n1.record()
        torch.cuda.synchronize()
        us_nat = n0.elapsed_time(n1) * 1e3 / (args.decode_reps * Lyr)
        natural = {"us_per_launch": round(us_nat, 3),
                   "gbps": round(bytes_launch / (us_nat * 1e-6) / 1e9, 1)}
        print(f"[bench] decode, natural order {us_nat:.2f} us/launch", flush=True)

    # Reference reads: a plain streaming read of four layer caches (4 x 512 MiB,
    # each launch far beyond the last-level cache), and the decode's own tile
    # reads without arithmetic over the 28 layers.
    kv_bytes = 2 * int(lens.sum()) * Hkv * D * 2
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    reads = kc[:4]
    for r in reads:
        probe.stream_read(r, sink)
    torch.cuda.synchronize()
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    for _ in range(3):
        for r in reads:
            probe.stream_read(r, sink)
    s1.record()
    torch.cuda.synchronize()
    stream_gbps = 3 * sum(r.numel() * 2 for r in reads) / (s0.elapsed_time(s1) * 1e-3) / 1e9
    split_used = args.split or pa.default_split_tokens(Hq, Hkv, D, torch.bfloat16)
    tile = {}
    for waves in (4, 8):
        def tiles():
            for l in range(Lyr):
                probe.tile_read(kc[l], vc[l], bt, cl, max_len, split_used, sink, waves=waves)
        tiles()
        torch.cuda.synchronize()
        gt = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gt):
            tiles()
        gt.replay()
        torch.cuda.synchronize()
        t0_, t1_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0_.record()
        for _ in range(args.decode_reps):
            gt.replay()
        t1_.record()
        torch.cuda.synchronize()
        us_t = t0_.elapsed_time(t1_) * 1e3 / (args.decode_reps * Lyr)
        tile[waves] = {"us_per_launch": round(us_t, 3), "gbps": round(kv_bytes / (us_t * 1e-6) / 1e9, 1)}
        del gt
    best_tile = max(t["gbps"] for t in tile.values())
    print(f"[bench] streaming read {stream_gbps:.0f} GB/s; decode-pattern tile read "
          f"{tile[4]['gbps']:.0f} GB/s (4 waves), {tile[8]['gbps']:.0f} GB/s (8 waves)", flush=True)

    # Captured steps per batch-size bucket (paged_kv_gqa_pa_amd.graphs): the first n
    # sequences of the workload as a batch of n, each on its own bucket.
    buckets = None
    if not args.no_buckets:
        buckets = bucket_timing(torch, pa, kc, vc, qs, nks, nvs, bt, cl, sm, table, scale,
                                args.decode_reps, fused=True)
        buckets["write_then_decode"] = bucket_timing(torch, pa, kc, vc, qs, nks, nvs, bt, cl, sm,
                                                     table, scale, args.decode_reps, fused=False)

    traffic = None
    if os.path.exists(args.traffic_file):
        try:
            with open(args.traffic_file) as f:
                tr = json.load(f)
            if tr.get("kernel_source_hash") == _kernel_hash():
                traffic = tr.get("bytes_per_launch")
        except (OSError, ValueError):
            traffic = None

    res = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "step_ms_with_events": {"median": round(per_step[len(per_step) // 2], 4),
                                "min": round(per_step[0], 4), "max": round(per_step[-1], 4)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "num_seqs": N, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": D, "block_size": 16, "layers": Lyr, "num_blocks_per_layer": NB,
                   "context": "256 + U{1..256} (new token included)",
                   "step": ("" if plan is None else "pa_plan + ") +
                           "28 x pa_decode_append (per layer: the new token's K/V written into "
                           "the cache and attention over the context that includes it, one launch)",
                   "launch": "eager" if args.eager else "hipgraph",
                   "split_tokens": args.split or pa.default_split_tokens(Hq, Hkv, D, torch.bfloat16)},
        "write_then_decode_step": {
            "ms_per_step": round(ms_split, 4), "tokens_per_s": round(N / (ms_split / 1e3), 1),
            "step_ms_with_events": {"median": round(per_split[len(per_split) // 2], 4),
                                    "min": round(per_split[0], 4), "max": round(per_split[-1], 4)},
            "entry_points": "28 x (pa_reshape_and_cache + pa_decode)" +
                            ("" if plan is None else ", after one pa_plan per step")},
        "hbm_gbps": round(gbps, 1),
        "pct_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "kernel": "decode_pass1",
                     "work_plan": plan is not None,
                     "natural_order": natural,
                     "us_per_launch": round(us_decode, 3), "algorithmic_bytes_per_launch": bytes_launch,
                     "us_per_launch_over_passes": {"median": round(per_pass[len(per_pass) // 2], 3),
                                                   "min": round(per_pass[0], 3),
                                                   "max": round(per_pass[-1], 3)}},
        "achievable": {"stream_read_gbps": round(stream_gbps, 1),
                       "decode_frac_of_stream_read": round(gbps / stream_gbps, 4),
                       "tile_read": {f"{w}_waves": t for w, t in tile.items()},
                       "decode_frac_of_tile_read": round(gbps / best_tile, 4),
                       "note": "stream read: 4 x 512 MiB layer caches, 16-byte non-temporal loads; "
                               "tile read: the decode's K/V reads (exact rows, same grid order and "
                               "pieces) with no arithmetic, over the same 28 layers"},
    }
    if buckets is not None:
        res["step_graph_buckets"] = buckets
    if not args.no_other_workloads:
        res["other_workloads"] = other_workloads(torch, pa, wl, dev, use_plan=not args.no_plan)
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


# The sources the batch-64 decode kernel (decode_pass1) is built from: stored
# hardware byte counts stay valid while these are unchanged.
DECODE_KERNEL_SOURCES = ("pa_decode.hip", "pa_device.h", "pa_kernels.h")


def _kernel_hash():
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "paged_kv_gqa_pa_amd", "csrc")
    for n in DECODE_KERNEL_SOURCES:
        with open(os.path.join(csrc, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
