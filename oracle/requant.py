"""Plain CPU oracle for the requantizing int8 cache write.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports or calls this
module: only the tests do.  It shares no code with the HIP library.

What it computes ("A Rust inference server for Qwen2 on Apple Silicon",
"Day 4 measurements -- int8 KV", "Partial blocks" and the cost list before
it): an int8 block holds 16 positions of one KV head with one float scale.
A write of a new token into block p at offset o requantizes the whole block:

    X = codes[p] * scale[p]           dequantize the 16 slots
    X[o, :] = new row                 overwrite the incoming row
    scale' = max|X| / 127             recompute the scale (1 when the block is all 0)
    codes[p] = clip(rint(X / scale'), -127, 127)

Unwritten slots hold code 0, so they never raise the maximum; a value already
on the grid comes back unchanged when the scale does not change.  Tokens are
applied in index order, so several tokens aimed at one block in one call
equal the same tokens written by consecutive calls.  Negative slots are
skipped (padding rows); no other block or scale changes.

Precision: the codes are integers decided by floating point, so the oracle
takes every step in float32 -- the precision of the stored scales and of the
workload's quantiser -- with correctly rounded multiply and divide and rint
rounding half to even.  Readings where the pages are silent: the scale of an
all-zero block is 1.0 (the workload's convention); the new row arrives as
bf16 or fp32 and is widened exactly to float32; the K and V caches are
requantized independently, each with its own scale.
"""
from __future__ import annotations

import numpy as np

__all__ = ["requantize_block", "reshape_and_cache_int8"]

_F127 = np.float32(127.0)


def _row_f32(row, tag: str) -> np.ndarray:
    if tag == "f32":
        return np.asarray(row, dtype=np.float32)
    if tag == "bf16":
        hi = np.asarray(row, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return hi.view(np.float32)
    raise ValueError(f"unknown input tag {tag!r}")


def requantize_block(codes: np.ndarray, scale: np.float32, offset: int, row_f32: np.ndarray):
    """One write: codes [16, D] int8 and its scale, the new row at `offset` -> (codes', scale')."""
    x = np.asarray(codes, dtype=np.int8).astype(np.float32) * np.float32(scale)
    x[offset, :] = row_f32
    amax = np.float32(np.abs(x).max())
    new_scale = np.float32(amax / _F127) if amax > 0 else np.float32(1.0)
    q = np.rint(x / new_scale)
    return np.clip(q, -127, 127).astype(np.int8), new_scale


def reshape_and_cache_int8(key, value, in_tag, k_codes, v_codes, k_scale, v_scale, slot_mapping):
    """Expected int8 caches and scales after writing each token in index order.

    key/value: [num_tokens, H_kv, D] stored as ``in_tag`` ("bf16" bit patterns
    or "f32"); caches [H_kv, num_blocks, 16, D] int8; scales [H_kv, num_blocks]
    float32.  Returns new arrays; the inputs are left untouched.
    """
    kc, vc = np.array(k_codes, copy=True), np.array(v_codes, copy=True)
    ks = np.array(k_scale, dtype=np.float32, copy=True)
    vs = np.array(v_scale, dtype=np.float32, copy=True)
    bs = kc.shape[2]
    for i, slot in enumerate(np.asarray(slot_mapping, np.int64)):
        if slot < 0:
            continue
        blk, off = int(slot) // bs, int(slot) % bs
        for g in range(kc.shape[0]):
            kc[g, blk], ks[g, blk] = requantize_block(kc[g, blk], ks[g, blk], off,
                                                      _row_f32(key[i, g], in_tag))
            vc[g, blk], vs[g, blk] = requantize_block(vc[g, blk], vs[g, blk], off,
                                                      _row_f32(value[i, g], in_tag))
    return kc, vc, ks, vs
