"""Graph capture: every call is capturable and replays give the eager bits.

The calls enqueue kernels only (no allocation, synchronisation or host reads),
so a HIP graph of them replays the same work.  Each replay is checked against
the eager result, with eager work and synchronisations in between.
"""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_gqa_pa_amd import _lib as pa
from paged_kv_gqa_pa_amd import workloads as wl
from tests.gpu_util import TOL, DevCase, host_bits, max_abs_err

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


@pytest.mark.parametrize("name,split", [("qwen2_1p5b_bf16", 128), ("long_ctx_int8", 1024),
                                        ("spec_verify_bf16", 256)])
def test_graph_replays_match_eager(name, split):
    """Pass 1 plus the merge pass (several pieces), captured once, replayed three times."""
    _say("graph replay", name, "split", split)
    case = wl.build_case(name)
    dc = DevCase(case)
    spec = case.spec
    T = spec.num_query_tokens
    fn = pa.verify if T > 1 else pa.decode
    kdt = {"bf16": torch.bfloat16, "int8": torch.int8, "f32": torch.float32}[spec.kv_dtype]
    need = pa.workspace_size(spec.num_seqs, T, spec.q_heads, spec.kv_heads, spec.head_dim,
                             case.max_context_len, kdt, split)
    assert need > 0, "the case must exercise the merge pass"
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")

    def call(out):
        fn(out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, case.scale,
           case.max_context_len, dc.k_scale, dc.v_scale, split_tokens=split, workspace=ws)

    eager = torch.empty_like(dc.q)
    call(eager)
    torch.cuda.synchronize()
    want = (oracle.verify if T > 1 else oracle.decode)(
        case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens, case.scale,
        spec.q_dtype, spec.kv_dtype, case.k_scale, case.v_scale)
    assert max_abs_err(eager, want) < TOL[spec.kv_dtype]

    out = torch.empty_like(dc.q)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        call(out)   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out)
    ref = host_bits(eager).tobytes()
    for rep in range(3):
        out.fill_(float("nan"))
        scratch = torch.empty_like(dc.q)
        call(scratch)               # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert host_bits(out).tobytes() == ref, f"replay {rep} differs from the eager call"


def test_graph_step_cache_write_and_decode():
    """pa_decode_append captured in a graph: replays write the same cache row and output."""
    _say("graph replay decode_append")
    case = wl.build_case("batch64_28layer_bf16", layer=1)
    dc = DevCase(case)
    k0, v0 = dc.k_cache.clone(), dc.v_cache.clone()

    def call(out):
        pa.decode_append(out, dc.q, dc.new_k, dc.new_v, dc.k_cache, dc.v_cache, dc.slot_mapping,
                         dc.block_tables, dc.context_lens, case.scale, case.max_context_len)

    eager = torch.empty_like(dc.q)
    call(eager)
    torch.cuda.synchronize()
    k_after = host_bits(dc.k_cache).tobytes()
    dc.k_cache.copy_(k0)
    dc.v_cache.copy_(v0)
    out = torch.empty_like(dc.q)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        call(out)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out)
    for rep in range(3):
        dc.k_cache.copy_(k0)
        dc.v_cache.copy_(v0)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert host_bits(out).tobytes() == host_bits(eager).tobytes(), rep
        assert host_bits(dc.k_cache).tobytes() == k_after, rep
