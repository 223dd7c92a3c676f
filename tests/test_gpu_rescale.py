"""Running maxima that keep rising, on every attention kernel against the oracle.

Every key of a KV head points along one direction that all of its query heads share,
with a length that grows with the position, so a row's scores climb along the context:
about 4 (log2 units) per 32 positions, which makes the kernels raise their reference
maximum and rescale every second stage or so, each time because of the lanes that hold
the newest keys.  Decode on the vector-ALU kernel (two query heads per KV head) and on
the matrix-core kernel (six), with and without pieces; verify; chunked prefill.
"""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_gqa_pa_amd import _lib as pa
from paged_kv_gqa_pa_amd import workloads as wl
from tests.gpu_util import TOL, DevCase, dev, max_abs_err
from tests.test_gpu_decode import _random_case
from tests.test_gpu_prefill import _pack, _prefill, _want
from tests.test_gpu_verify import _random_verify_case

pytestmark = pytest.mark.gpu

RATE = 0.25   # key length per position (head_dim 128, scale 1/sqrt(128), |q| = 4)


def _say(*a):
    print("[case]", *a, flush=True)


def _grow(rng, case, q_shape):
    """Keys along a unit direction per KV head, of length RATE * position, and every
    query of that head's group along the same direction with length 4 (bf16 bits)."""
    Hkv, D = case.spec.kv_heads, case.spec.head_dim
    G = case.spec.q_heads // Hkv
    u = rng.standard_normal((Hkv, D)).astype(np.float32)
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    k = case.k_cache
    for b, L in enumerate(case.context_lens):
        for pos in range(int(L)):
            phys = case.block_tables[b, pos // 16]
            k[:, phys, pos % 16] = wl.f32_to_bf16_bits(RATE * pos * u)
    qdir = np.repeat(4.0 * u, G, axis=0)                      # [Hq, D]
    q = np.broadcast_to(qdir, q_shape).astype(np.float32)
    case.q[...] = wl.f32_to_bf16_bits(np.ascontiguousarray(q))


@pytest.mark.parametrize("G", [2, 6])
@pytest.mark.parametrize("split", [0, 64])
def test_decode_rising_maximum(G, split):
    _say("decode rising maximum G", G, "split", split)
    rng = np.random.default_rng(5100 + G + split)
    case = _random_case(rng, [700, 333, 5, 1029, 64], Hkv=2, G=G, D=128, tag="bf16", poison=True)
    _grow(rng, case, case.q.shape)
    dc = DevCase(case)
    out = torch.empty_like(dc.q)
    pa.decode(out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, case.scale,
              case.max_context_len, split_tokens=split)
    torch.cuda.synchronize()
    want = oracle.decode(case.q, case.k_cache, case.v_cache, case.block_tables,
                         case.context_lens, case.scale, "bf16", "bf16")
    assert max_abs_err(out, want, TOL["bf16"]) < TOL["bf16"]


@pytest.mark.parametrize("split", [0, 128])
def test_verify_rising_maximum(split):
    _say("verify rising maximum split", split)
    rng = np.random.default_rng(5200 + split)
    case = _random_verify_case(rng, [700, 40, 517], Hkv=2, G=2, D=128, T=5, poison=True)
    _grow(rng, case, case.q.shape)
    dc = DevCase(case)
    out = torch.empty_like(dc.q)
    pa.verify(out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, case.scale,
              case.max_context_len, split_tokens=split)
    torch.cuda.synchronize()
    want = oracle.verify(case.q, case.k_cache, case.v_cache, case.block_tables,
                         case.context_lens, case.scale, "bf16", "bf16")
    assert max_abs_err(out, want, TOL["bf16"]) < TOL["bf16"]


@pytest.mark.parametrize("G", [2, 6])
def test_prefill_rising_maximum(G):
    _say("prefill rising maximum G", G)
    rng = np.random.default_rng(5300 + G)
    T = 70
    lens = [700, 90, 333]
    case = _random_verify_case(rng, lens, Hkv=2, G=G, D=128, T=T, poison=True)
    _grow(rng, case, case.q.shape)
    dc = DevCase(case)
    qp, qs, lens = _pack(case, [70, 33, 70], lens)
    err = max_abs_err(_prefill(case, dc, qp, qs, lens, T), _want(case, qp, qs, lens))
    assert err < TOL["bf16"], err
