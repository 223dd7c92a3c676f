"""Pins of the requantizing int8 cache-write oracle to things other than itself.

Each ``pin_*`` takes an oracle module exposing ``requantize_block`` and
``reshape_and_cache_int8`` and raises AssertionError on a disagreement with
what the pages and the arithmetic fix ("A Rust inference server for Qwen2 on
Apple Silicon", "Day 4 measurements -- int8 KV", "Partial blocks"):

* a write into an empty block equals the workload's own block quantiser
  (``workloads.quantize_int8_blocks``, written separately) applied to a block
  holding only that row;
* a row that does not raise the block maximum leaves every other code as it
  was (values on the grid come back exactly at an unchanged scale);
* after any write the block dequantizes to within half a scale step of the
  float block it stands for (the page's error estimate, scale / 2);
* index order: two tokens in one call equal two calls, and a slot written
  twice keeps the later row;
* K and V carry separate scales; negative slots and other blocks are left
  bit for bit.
"""
from __future__ import annotations

import numpy as np

from paged_kv_gqa_pa_amd import workloads as wl


def _bf16(x):
    return wl.f32_to_bf16_bits(np.asarray(x, np.float32))


def _widen_bf16(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _block_case(rng, D=8, nb=4, H=2, filled=10):
    """int8 caches whose blocks hold `filled` quantized rows and zero rows after them."""
    x = rng.standard_normal((H, nb, 16, D)).astype(np.float32)
    x[:, :, filled:, :] = 0.0
    codes, scales = wl.quantize_int8_blocks(x)
    return x, codes, scales


def pin_fresh_block_matches_workload_quantiser(o):
    rng = np.random.default_rng(11)
    D = 8
    row = _bf16(rng.standard_normal(D) * 3.0)
    for off in (0, 7, 15):
        codes, scale = o.requantize_block(np.zeros((16, D), np.int8), np.float32(0.37), off,
                                          _widen_bf16(row))
        dense = np.zeros((1, 1, 16, D), np.float32)
        dense[0, 0, off] = _widen_bf16(row)
        want_c, want_s = wl.quantize_int8_blocks(dense)
        assert codes.tobytes() == want_c[0, 0].tobytes(), "fresh block codes"
        assert np.float32(scale) == want_s[0, 0], "fresh block scale"
    # an all-zero row into an empty block: scale 1, codes 0
    codes, scale = o.requantize_block(np.zeros((16, D), np.int8), np.float32(0.5), 3,
                                      np.zeros(D, np.float32))
    assert not codes.any() and np.float32(scale) == np.float32(1.0), "all-zero block"


def pin_grid_values_survive(o):
    rng = np.random.default_rng(12)
    x, codes, scales = _block_case(rng, H=1, nb=1)
    c0, s0 = codes[0, 0], scales[0, 0]
    small = np.full(8, 0.25, np.float32) * np.float32(s0)   # far below the block maximum
    c1, s1 = o.requantize_block(c0, s0, 12, small)
    assert abs(float(s1) - float(s0)) <= float(np.spacing(np.float32(s0))), "scale unchanged"
    keep = [r for r in range(16) if r != 12]
    assert c1[keep].tobytes() == c0[keep].tobytes(), "codes on the grid must come back exactly"


def pin_error_bound(o):
    rng = np.random.default_rng(13)
    for trial in range(20):
        x, codes, scales = _block_case(rng, H=1, nb=1, filled=int(rng.integers(0, 16)))
        off = int(rng.integers(0, 16))
        row = (rng.standard_normal(8) * float(rng.choice([0.1, 1.0, 30.0]))).astype(np.float32)
        c1, s1 = o.requantize_block(codes[0, 0], scales[0, 0], off, row)
        target = codes[0, 0].astype(np.float64) * float(scales[0, 0])
        target[off] = row
        deq = c1.astype(np.float64) * float(s1)
        # half a step of the new scale (the target holds the old rows as they were
        # stored, so their earlier rounding is not part of this bound)
        bound = 0.5 * float(s1) * (1 + 1e-6)
        assert np.abs(deq[off] - target[off]).max() <= bound, "new row within scale / 2"
        assert np.abs(deq - target).max() <= 0.5 * float(s1) * (1 + 1e-5) + 1e-30, "block within scale / 2"
        assert float(s1) * 127 >= np.abs(target).max() * (1 - 1e-6), "scale covers the block maximum"


def pin_index_order_and_separate_scales(o):
    rng = np.random.default_rng(14)
    H, nb, D = 2, 4, 8
    _, kc, ks = _block_case(rng, D=D, nb=nb, H=H)
    _, vc, vs = _block_case(rng, D=D, nb=nb, H=H)
    key = _bf16(rng.standard_normal((3, H, D)) * np.array([1.0, 5.0, 0.5])[:, None, None])
    val = _bf16(rng.standard_normal((3, H, D)))
    slots = np.array([16 * 2 + 11, 16 * 2 + 4, -1], np.int64)   # two tokens into block 2
    one = o.reshape_and_cache_int8(key, val, "bf16", kc, vc, ks, vs, slots)
    a = o.reshape_and_cache_int8(key[:1], val[:1], "bf16", kc, vc, ks, vs, slots[:1])
    two = o.reshape_and_cache_int8(key[1:2], val[1:2], "bf16", *a, slots[1:2])
    for x, y in zip(one, two):
        assert np.asarray(x).tobytes() == np.asarray(y).tobytes(), "one call == consecutive calls"
    # a slot written twice keeps the later row
    twice = np.array([16 * 1 + 3, 16 * 1 + 3], np.int64)
    r = o.reshape_and_cache_int8(key[:2], val[:2], "bf16", kc, vc, ks, vs, twice)
    b = o.reshape_and_cache_int8(key[:1], val[:1], "bf16", kc, vc, ks, vs, twice[:1])
    b = o.reshape_and_cache_int8(key[1:2], val[1:2], "bf16", *b, twice[1:2])
    assert all(np.asarray(x).tobytes() == np.asarray(y).tobytes() for x, y in zip(r, b))
    deq = r[0][:, 1, 3].astype(np.float64) * r[2][:, 1][:, None]
    assert np.abs(deq - _widen_bf16(key[1])).max() <= 0.5 * float(r[2][:, 1].max()) * 1.00001, \
        "later row wins"
    # separate K and V scales; untouched blocks, scales and padding rows
    nk, nv, nks, nvs = one
    assert not np.allclose(nks[:, 2], nvs[:, 2]), "K and V scales are separate"
    for blk in (0, 1, 3):
        assert nk[:, blk].tobytes() == kc[:, blk].tobytes() and nv[:, blk].tobytes() == vc[:, blk].tobytes()
        assert nks[:, blk].tobytes() == ks[:, blk].tobytes() and nvs[:, blk].tobytes() == vs[:, blk].tobytes()
    assert ks.tobytes() != nks.tobytes(), "inputs are not modified in place"


PINS = [pin_fresh_block_matches_workload_quantiser, pin_grid_values_survive, pin_error_bound,
        pin_index_order_and_separate_scales]
