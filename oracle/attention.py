"""Plain fp64 CPU oracle for paged grouped-query decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports or calls this
module: only the tests, the smoke check and the CPU-baseline leg of the
benchmark do.  It shares no code with the HIP library.

What it computes, and where the pages define it:

* Dense softmax attention over a sequence's cached context, one query row at
  a time: scores = scale * K q, subtract the maximum, exponentiate, normalise,
  weight V.  This is the per-row formula of the NumPy model in "Anatomy of a
  Decode-Step Stall: Where p99 Inter-Token Latency Really Comes From",
  section "Full Source" (engine.py, ``Model._layer``), and the "dense
  reference" that "From 183 ms to 19 ms per decode step" checks its paged
  kernels against (sections "Where it started" and "Limits").
* The context is gathered from the paged, head-major cache through the block
  table ("From 183 ms to 19 ms per decode step", "Four changes, one profile at
  a time", changes 2 and 3): position j of sequence b lives in physical block
  ``block_tables[b, j // block_size]`` at offset ``j % block_size``.  Only
  positions ``j < context_lens[b]`` exist; nothing past them is read (a zero
  key is not neutral -- "A Rust inference server for Qwen2 on Apple Silicon",
  "Day 3 measurements", "Known gaps").
* Grouped-query attention: query head h reads KV head ``h // G`` with
  ``G = q_heads // kv_heads`` (consecutive groups, the repeat-interleave
  expansion the Qwen2 page calls ``repeat_kv``; "From 183 ms to 19 ms",
  change 1, serves each group from one K/V read).
* Verify (several new tokens per sequence): query token t of T sees cached
  positions ``j <= L - T + t`` -- the causal convention of the prefill code in
  "Anatomy of a Decode-Step Stall" (engine.py, ``forward_prefill``: an upper
  triangular mask sliced at the chunk's start), applied to the k+1 tokens of a
  verify step ("From 183 ms to 19 ms", "Then speculative decoding got
  slower").
* Variable-length verify: sequence b contributes its own number of new
  tokens T_b (at most k+1; the pages pad every sequence to k+1 -- "From 183
  ms to 19 ms", "Then speculative decoding got slower"), its query rows packed
  one sequence after another; each sequence is then the verify above with its
  own T_b.
* int8 caches are read as ``code * scale`` with one float scale per
  (kv_head, block) -- the stored values, widened exactly to fp64.
* The cache write places token i's K/V for every KV head at flat slot
  ``slot_mapping[i] = phys_block * block_size + offset``; negative slots are
  skipped; nothing else changes.

Readings where the pages are silent: an empty context (L = 0) yields a zero
output row; bf16 is widened by placing its 16 bits in the top half of a
float32.
"""
from __future__ import annotations

import numpy as np

__all__ = ["widen", "gather_context", "attend", "decode", "verify", "verify_varlen",
           "reshape_and_cache"]


def widen(stored: np.ndarray, tag: str) -> np.ndarray:
    """Stored values -> float64, exactly.  ``tag`` is "f32", "bf16" or "int8"."""
    if tag == "f32":
        return np.asarray(stored, dtype=np.float32).astype(np.float64)
    if tag == "bf16":
        hi = np.asarray(stored, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return hi.view(np.float32).astype(np.float64)
    if tag == "int8":
        return np.asarray(stored, dtype=np.int8).astype(np.float64)
    raise ValueError(f"unknown dtype tag {tag!r}")


def gather_context(cache, table_row, length, kv_head, tag, block_scale=None):
    """K (or V) rows of positions 0..length-1 of one sequence, as fp64 [length, D]."""
    bs = cache.shape[2]
    j = np.arange(length)
    phys = np.asarray(table_row)[j // bs].astype(np.int64)
    rows = widen(cache[kv_head, phys, j % bs, :], tag)
    if tag == "int8":
        rows = rows * np.asarray(block_scale, np.float64)[kv_head, phys][:, None]
    return rows


def attend(q_rows, keys, values, scale, visible=None):
    """Dense softmax attention of query rows [R, D] over keys/values [L, D].

    ``visible`` (bool [R, L]) limits which keys each row sees (default: all).
    Which keys count is decided by visibility alone, never by the values: a
    NaN or infinite score, or a non-finite V row, at a visible position
    propagates into the row's output as the dense formula gives it.  A row
    that sees no key returns zeros.
    """
    q_rows = np.asarray(q_rows, np.float64)
    R, L = q_rows.shape[0], keys.shape[0]
    out = np.zeros((R, values.shape[1]), np.float64)
    if L == 0:
        return out
    seen_all = np.ones((R, L), bool) if visible is None else np.asarray(visible, bool)
    with np.errstate(invalid="ignore"):
        s = (q_rows @ keys.T) * float(scale)
        for r in range(R):
            seen = seen_all[r]
            if not seen.any():
                continue
            row = s[r, seen]
            e = np.exp(row - row.max())
            out[r] = (e / e.sum()) @ values[seen]
    return out


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, q_tag, kv_tag,
           k_scale=None, v_scale=None):
    """One query token per sequence.  q: [N, H_q, D] stored; returns fp64 [N, H_q, D]."""
    q64 = widen(q, q_tag)
    N, Hq, D = q64.shape
    Hkv = k_cache.shape[0]
    G = Hq // Hkv
    out = np.zeros((N, Hq, D), np.float64)
    for b in range(N):
        L = int(context_lens[b])
        for g in range(Hkv):
            K = gather_context(k_cache, block_tables[b], L, g, kv_tag, k_scale)
            V = gather_context(v_cache, block_tables[b], L, g, kv_tag, v_scale)
            out[b, g * G:(g + 1) * G] = attend(q64[b, g * G:(g + 1) * G], K, V, scale)
    return out


def verify(q, k_cache, v_cache, block_tables, context_lens, scale, q_tag, kv_tag,
           k_scale=None, v_scale=None):
    """T query tokens per sequence, causal among themselves.

    q: [N, T, H_q, D] stored; context_lens include the T new tokens.  Token t
    sees positions 0 .. L - T + t.  Returns fp64 [N, T, H_q, D].
    """
    q64 = widen(q, q_tag)
    N, T, Hq, D = q64.shape
    Hkv = k_cache.shape[0]
    G = Hq // Hkv
    out = np.zeros((N, T, Hq, D), np.float64)
    for b in range(N):
        L = int(context_lens[b])
        last_seen = L - T + np.arange(T)                       # per query token
        for g in range(Hkv):
            K = gather_context(k_cache, block_tables[b], L, g, kv_tag, k_scale)
            V = gather_context(v_cache, block_tables[b], L, g, kv_tag, v_scale)
            rows = q64[b, :, g * G:(g + 1) * G].reshape(T * G, D)     # row = t * G + i
            vis = np.arange(L)[None, :] <= np.repeat(last_seen, G)[:, None]
            o = attend(rows, K, V, scale, vis)
            out[b, :, g * G:(g + 1) * G] = o.reshape(T, G, D)
    return out


def verify_varlen(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, q_tag,
                  kv_tag, k_scale=None, v_scale=None):
    """Per-sequence query counts over packed query rows.

    q: [total, H_q, D] stored; sequence b's query tokens are rows
    query_start[b] .. query_start[b+1]-1 (T_b of them, possibly none), and it
    is the verify of one sequence with T = T_b: its token t sees positions
    0 .. L_b - T_b + t.  Returns fp64 [total, H_q, D].
    """
    qs = np.asarray(query_start, np.int64)
    q = np.asarray(q)
    out = np.zeros(q.shape, np.float64)
    for b in range(len(qs) - 1):
        lo, hi = int(qs[b]), int(qs[b + 1])
        if hi <= lo:
            continue
        out[lo:hi] = verify(q[None, lo:hi], k_cache, v_cache, block_tables[b:b + 1],
                            context_lens[b:b + 1], scale, q_tag, kv_tag, k_scale, v_scale)[0]
    return out


def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping):
    """Expected caches after writing each new token's K/V into its slot.

    key/value: [num_tokens, H_kv, D] in the cache's stored form.  Returns new
    arrays; the inputs are left untouched.
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    bs = kc.shape[2]
    for i, slot in enumerate(np.asarray(slot_mapping, np.int64)):
        if slot < 0:
            continue
        blk, off = int(slot) // bs, int(slot) % bs
        kc[:, blk, off, :] = key[i]
        vc[:, blk, off, :] = value[i]
    return kc, vc
