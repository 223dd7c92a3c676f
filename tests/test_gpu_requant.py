"""GPU parity of pa_reshape_and_cache_quant (requantizing int8 cache write).

The codes and scales are integers / floats decided by fp32 arithmetic taken
in the same precision on both sides, so the comparison is bit-exact on the
whole cache (untouched blocks included).
"""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_gqa_pa_amd import _lib as pa
from paged_kv_gqa_pa_amd import workloads as wl
from tests.gpu_util import dev, host_bits

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _cache(rng, Hkv, nb, D, empty_blocks=()):
    """Quantised cache of normal draws; listed blocks hold nothing (codes 0, scale 1)."""
    x = rng.standard_normal((Hkv, nb, 16, D), dtype=np.float32)
    x[:, list(empty_blocks)] = 0.0
    # some blocks partially filled: trailing rows never written
    x[:, 1, 9:] = 0.0
    return wl.quantize_int8_blocks(x)


def _run(rng, tag, D, Hkv, nb, slots, mag=1.0, empty_blocks=(0,)):
    kc, ks = _cache(rng, Hkv, nb, D, empty_blocks)
    vc, vs = _cache(rng, Hkv, nb, D, empty_blocks)
    T = len(slots)
    key = wl.encode(mag * rng.standard_normal((T, Hkv, D), dtype=np.float32), tag)
    val = wl.encode(mag * rng.standard_normal((T, Hkv, D), dtype=np.float32), tag)
    slots = np.asarray(slots, np.int64)
    dk, dv, dks, dvs = dev(kc), dev(vc), dev(ks), dev(vs)
    pa.reshape_and_cache_quant(dev(key), dev(val), dk, dv, dks, dvs, dev(slots))
    torch.cuda.synchronize()
    wk, wv, wks, wvs = oracle.reshape_and_cache_int8(key, val, tag, kc, vc, ks, vs, slots)
    assert host_bits(dks).tobytes() == wks.tobytes()
    assert host_bits(dvs).tobytes() == wvs.tobytes()
    assert host_bits(dk).tobytes() == wk.tobytes()
    assert host_bits(dv).tobytes() == wv.tobytes()


@pytest.mark.parametrize("tag,D", [("bf16", 128), ("f32", 64), ("f32", 128), ("bf16", 64)])
def test_requant_write_small(tag, D):
    """Padding slots, an empty block, a partial block, two tokens in one block."""
    _say("requant write", tag, D)
    rng = np.random.default_rng(23)
    Hkv, nb = 3, 9
    slots = [3, -1, 16 * nb - 1, 40, -7, 0, 77, 5, 3]   # 3 twice, block 0 four times
    _run(rng, tag, D, Hkv, nb, slots)


def test_requant_write_growing_block():
    """A new row larger than the block's maximum raises the scale for every row."""
    _say("requant write, rows that raise the block maximum")
    rng = np.random.default_rng(5)
    _run(rng, "bf16", 128, 2, 4, [20, 21, 22, 37], mag=40.0)


@pytest.mark.parametrize("T", [300, 700])
def test_requant_write_many_tokens_same_blocks(T):
    """Hundreds of tokens over a few blocks: ownership and order across many chunks of slots."""
    _say("requant write,", T, "tokens over 5 blocks")
    rng = np.random.default_rng(99)
    nb = 12
    slots = rng.integers(16 * 3, 16 * 8, size=T)
    slots[rng.random(T) < 0.1] = -1
    _run(rng, "f32", 64, 2, nb, slots)


def test_requant_write_decode_batch():
    """Decode-step write at the served shape: 64 sequences, 8 KV heads, head_dim 128."""
    _say("requant write, batch 64 x 8 KV heads, bf16 rows")
    rng = np.random.default_rng(64)
    nb = 256
    blocks = rng.permutation(nb)[:64]
    slots = blocks * 16 + rng.integers(0, 16, size=64)
    slots[[5, 40]] = -1
    _run(rng, "bf16", 128, 8, nb, slots, empty_blocks=(blocks[0], blocks[1]))


def test_requant_write_then_decode_matches_oracle():
    """Decode over a cache written by the requantizing write agrees with the oracle."""
    _say("requant write then int8 decode")
    rng = np.random.default_rng(8)
    Hkv, G, D, nb = 2, 6, 128, 16
    kc, ks = _cache(rng, Hkv, nb, D, (0,))
    vc, vs = _cache(rng, Hkv, nb, D, (0,))
    tables = np.array([[3, 7, 1], [0, 11, 4]], np.int32)
    lens = np.array([40, 33], np.int32)
    slots = np.array([tables[0, 39 // 16] * 16 + 39 % 16, tables[1, 32 // 16] * 16 + 32 % 16],
                     np.int64)
    key = wl.encode(rng.standard_normal((2, Hkv, D), dtype=np.float32), "bf16")
    val = wl.encode(rng.standard_normal((2, Hkv, D), dtype=np.float32), "bf16")
    q = wl.encode(rng.standard_normal((2, Hkv * G, D), dtype=np.float32), "bf16")
    dk, dv, dks, dvs = dev(kc), dev(vc), dev(ks), dev(vs)
    pa.reshape_and_cache_quant(dev(key), dev(val), dk, dv, dks, dvs, dev(slots))
    dq = dev(q)
    out = torch.empty_like(dq)
    scale = 1.0 / np.sqrt(D)
    pa.decode(out, dq, dk, dv, dev(tables), dev(lens), scale, 48, dks, dvs)
    torch.cuda.synchronize()
    wk, wv, wks, wvs = oracle.reshape_and_cache_int8(key, val, "bf16", kc, vc, ks, vs, slots)
    want = oracle.decode(q, wk, wv, tables, lens, scale, "bf16", "int8", wks, wvs)
    got = out.float().cpu().numpy().astype(np.float64)
    assert float(np.abs(got - want).max()) < 2e-2


def test_requant_write_rejects_bad_arguments():
    kc = torch.zeros(2, 4, 16, 96, dtype=torch.int8, device="cuda")
    sc = torch.ones(2, 4, dtype=torch.float32, device="cuda")
    key = torch.zeros(1, 2, 96, dtype=torch.bfloat16, device="cuda")
    slots = torch.zeros(1, dtype=torch.int64, device="cuda")
    with pytest.raises(pa.PAError) as ei:
        pa.reshape_and_cache_quant(key, key, kc, kc.clone(), sc, sc.clone(), slots)
    assert ei.value.status == pa.PA_ERR_UNSUPPORTED
