"""Seeded synthetic inputs for paged grouped-query decode attention.

This module draws random contents and lays them out the way a paged KV cache
holds them; it computes no attention.  It is the one piece shared by the CPU
oracle tests and the GPU path: both receive the same stored arrays from here.

Layout (all numpy, row-major):

* KV cache: head-major ``[kv_heads, num_blocks, block_size, head_dim]`` -- the
  layout of "From 183 ms to 19 ms per decode step", section "Four changes, one
  profile at a time", change 2 (head-major KV cache).
* ``block_tables[num_seqs, max_blocks_per_seq]`` int32: logical block i of
  sequence b lives in physical block ``block_tables[b, i]``; entries past
  ``ceil(L_b / block_size)`` are -1 and are never read.
* ``context_lens[num_seqs]`` int32: L_b, the number of cached positions the
  query attends to, *including* the token being decoded (the decode step
  writes the new K/V first and then attends over ``[:position + 1]``, as the
  model loop of "Anatomy of a Decode-Step Stall", section "Full Source",
  engine.py, does).
* ``slot_mapping[num_tokens]`` int64: flat slot ``phys_block * block_size +
  offset`` of each new token (one index over the cache slots of one head).

Stored forms ("dtype tags"):

* ``"f32"``  -- numpy float32.
* ``"bf16"`` -- numpy uint16 holding bfloat16 bit patterns, produced from
  float32 draws by round-to-nearest-even.
* ``"int8"`` -- numpy int8 codes in [-127, 127] plus one float32 scale per
  (kv_head, block) (``scale = absmax / 127`` over that block's draws).

Draw recipe (fixed, so every consumer sees identical inputs):

* ``rng = default_rng(seed)`` draws, in order, the context lengths and the
  physical-block permutation.  Sequences take consecutive runs of the
  permutation, sequence 0 first.
* Layer ``l``'s contents come from ``default_rng((seed, l + 1))``, in order:
  q, K of the allocated blocks (ascending physical id), V likewise, then the
  new tokens' K and V.  Values are standard normal float32, then encoded.
* Unallocated blocks are zero, or poison (NaN; for int8 code 127 with scale
  1e30) when ``poison=True``; with poison the slots at positions >= L_b of a
  sequence's last block are poisoned as well (NaN; for int8 code 127, the
  block keeping the scale of its drawn contents).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = [
    "CONFIGS",
    "PagedCase",
    "build_case",
    "f32_to_bf16_bits",
    "quantize_int8_blocks",
    "encode",
    "assign_blocks",
    "slots_for_positions",
    "poison_float",
    "poison_int8",
]

BLOCK_SIZE = 16


# ----------------------------------------------------------------------------
# encodings
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.

    NaN stays NaN (quiet bit forced); infinities and overflow to infinity
    follow IEEE rounding.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = (bits + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    nan = np.isnan(x)
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = ((bits[nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return out


def quantize_int8_blocks(x: np.ndarray):
    """Symmetric int8 codes with one scale per leading (kv_head, block) pair.

    ``x``: float32 ``[kv_heads, nb, block_size, head_dim]``.  Returns
    ``(codes int8 same shape, scales float32 [kv_heads, nb])`` with
    ``scale = absmax / 127`` (1.0 where absmax is 0) and
    ``code = clip(rint(x / scale), -127, 127)`` computed in float32.
    """
    x = np.asarray(x, dtype=np.float32)
    absmax = np.abs(x).max(axis=(2, 3))
    scales = (absmax / np.float32(127.0)).astype(np.float32)
    scales[scales == 0] = np.float32(1.0)
    codes = np.rint(x / scales[:, :, None, None])
    codes = np.clip(codes, -127, 127).astype(np.int8)
    return codes, scales


def encode(x: np.ndarray, tag: str) -> np.ndarray:
    """Encode float32 draws into the stored form for ``"f32"`` / ``"bf16"``."""
    if tag == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if tag == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(f"encode: unsupported tag {tag!r}")


# ----------------------------------------------------------------------------
# block tables and slots
# ----------------------------------------------------------------------------
def assign_blocks(context_lens, perm, max_blocks_per_seq, block_size=BLOCK_SIZE):
    """Block table from consecutive runs of a physical-block permutation.

    Sequence b needs ``ceil(L_b / block_size)`` blocks; it takes the next run
    of ``perm``.  Unused entries are -1.
    """
    n = len(context_lens)
    table = np.full((n, max_blocks_per_seq), -1, dtype=np.int32)
    off = 0
    for b, L in enumerate(context_lens):
        nb = -(-int(L) // block_size)
        if nb > max_blocks_per_seq:
            raise ValueError("context longer than the block table allows")
        if off + nb > len(perm):
            raise ValueError("block pool exhausted")
        table[b, :nb] = perm[off:off + nb]
        off += nb
    return table


def slots_for_positions(block_tables, seq_ids, positions, block_size=BLOCK_SIZE):
    """Flat cache slot of (sequence, position) pairs: phys * block_size + offset."""
    seq_ids = np.asarray(seq_ids, dtype=np.int64)
    positions = np.asarray(positions, dtype=np.int64)
    phys = block_tables[seq_ids, positions // block_size].astype(np.int64)
    if (phys < 0).any():
        raise ValueError("position outside the allocated blocks")
    return phys * block_size + positions % block_size


def poison_float(cache, tag, block_tables, context_lens, block_size=BLOCK_SIZE):
    """Poison an fp32 or bf16 cache in place with NaN: every block no table row
    uses, and the slots at positions >= L_b of a sequence's last block.  Returns
    (spare blocks, poisoned tails)."""
    fill = encode(np.full(1, np.nan, np.float32), tag)[0]
    used = np.unique(block_tables[block_tables >= 0])
    spare = np.setdiff1d(np.arange(cache.shape[1]), used)
    cache[:, spare] = fill
    tails = 0
    for b, L in enumerate(np.asarray(context_lens)):
        if int(L) % block_size:
            phys = block_tables[b, (int(L) - 1) // block_size]
            cache[:, phys, int(L) % block_size:, :] = fill
            tails += 1
    return len(spare), tails


def poison_int8(codes, scales, block_tables, context_lens, block_size=BLOCK_SIZE):
    """Poison an int8 cache in place: blocks no table row uses get code 127 and
    scale 1e30; slots at positions >= L_b of a sequence's last block get code 127
    (the block keeps its scale).  Returns (spare blocks, poisoned tails)."""
    used = np.unique(block_tables[block_tables >= 0])
    spare = np.setdiff1d(np.arange(codes.shape[1]), used)
    codes[:, spare] = 127
    scales[:, spare] = np.float32(1e30)
    tails = 0
    for b, L in enumerate(np.asarray(context_lens)):
        if int(L) % block_size:
            phys = block_tables[b, (int(L) - 1) // block_size]
            codes[:, phys, int(L) % block_size:, :] = 127
            tails += 1
    return len(spare), tails


# ----------------------------------------------------------------------------
# configurations (the five workloads)
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Spec:
    name: str
    seed: int
    num_seqs: int
    q_heads: int
    kv_heads: int
    head_dim: int
    num_blocks: int
    q_dtype: str
    kv_dtype: str
    max_len: int                 # largest context length the draw can produce
    num_query_tokens: int = 1    # T: 1 = decode, k+1 = speculative verify
    layers: int = 1
    lens: Optional[tuple] = None  # fixed lengths, else drawn
    len_lo: int = 1               # drawn part: uniform integer in [len_lo, len_hi]
    len_hi: int = 1
    len_base: int = 0             # L_b = len_base + draw (+ num_query_tokens for verify)
    block_size: int = BLOCK_SIZE

    @property
    def max_blocks_per_seq(self) -> int:
        return -(-self.max_len // self.block_size)


CONFIGS = {
    # 4 sequences, lengths {1,17,33,64}, 2 q heads / 1 kv head, D=64, 16 blocks.
    "tiny_fp32": Spec("tiny_fp32", seed=0, num_seqs=4, q_heads=2, kv_heads=1, head_dim=64,
                      num_blocks=16, q_dtype="f32", kv_dtype="f32", max_len=64,
                      lens=(1, 17, 33, 64)),
    # Qwen2-1.5B-shaped layer: 12 q / 2 kv heads, D=128, batch 32, L ~ U{1..512}.
    "qwen2_1p5b_bf16": Spec("qwen2_1p5b_bf16", seed=1, num_seqs=32, q_heads=12, kv_heads=2,
                            head_dim=128, num_blocks=2048, q_dtype="bf16", kv_dtype="bf16",
                            max_len=512, len_lo=1, len_hi=512),
    # Batch-64 decode step over 28 layer caches: 16 q / 8 kv heads, D=128,
    # L = 256-token prompt + U{1..256} generated tokens (new token included).
    "batch64_28layer_bf16": Spec("batch64_28layer_bf16", seed=2, num_seqs=64, q_heads=16,
                                 kv_heads=8, head_dim=128, num_blocks=16384, q_dtype="bf16",
                                 kv_dtype="bf16", max_len=512, layers=28, len_base=256,
                                 len_lo=1, len_hi=256),
    # Speculative verify: 64 seqs, prior context U{256..1024} + k+1 = 5 new tokens.
    "spec_verify_bf16": Spec("spec_verify_bf16", seed=3, num_seqs=64, q_heads=16, kv_heads=8,
                             head_dim=128, num_blocks=8192, q_dtype="bf16", kv_dtype="bf16",
                             max_len=1024 + 5, num_query_tokens=5, len_lo=256, len_hi=1024),
    # Long-context int8 KV: batch 8, 32768 positions, 12 q / 2 kv heads, D=128.
    "long_ctx_int8": Spec("long_ctx_int8", seed=4, num_seqs=8, q_heads=12, kv_heads=2,
                          head_dim=128, num_blocks=16384, q_dtype="bf16", kv_dtype="int8",
                          max_len=32768, lens=(32768,) * 8),
}


@dataclasses.dataclass
class PagedCase:
    """One drawn workload instance (one layer) in stored form."""
    spec: Spec
    layer: int
    context_lens: np.ndarray      # int32 [N]
    block_tables: np.ndarray      # int32 [N, max_blocks_per_seq]
    q: np.ndarray                 # [N, H_q, D] (decode) or [N, T, H_q, D] (verify), stored form
    k_cache: np.ndarray           # [H_kv, num_blocks, bs, D], stored form
    v_cache: np.ndarray
    k_scale: Optional[np.ndarray]  # float32 [H_kv, num_blocks] for int8, else None
    v_scale: Optional[np.ndarray]
    new_k: np.ndarray             # [N*T, H_kv, D] stored form (tokens at L_b-T .. L_b-1)
    new_v: np.ndarray
    slot_mapping: np.ndarray      # int64 [N*T]
    scale: float

    @property
    def num_seqs(self):
        return self.spec.num_seqs

    @property
    def max_context_len(self) -> int:
        return self.spec.max_len


def draw_lengths(spec: Spec, rng) -> np.ndarray:
    if spec.lens is not None:
        lens = np.asarray(spec.lens, dtype=np.int64)
    else:
        lens = spec.len_base + rng.integers(spec.len_lo, spec.len_hi + 1, size=spec.num_seqs)
        if spec.num_query_tokens > 1:
            lens = lens + spec.num_query_tokens
    if lens.max() > spec.max_len:
        raise AssertionError("length draw exceeds the configured maximum")
    return lens.astype(np.int32)


def structure(spec: Spec, seed: Optional[int] = None):
    """Context lengths and block table of a configuration (layer independent)."""
    rng = np.random.default_rng(spec.seed if seed is None else seed)
    lens = draw_lengths(spec, rng)
    perm = rng.permutation(spec.num_blocks).astype(np.int32)
    table = assign_blocks(lens, perm, spec.max_blocks_per_seq, spec.block_size)
    return lens, table


def build_case(spec, layer: int = 0, poison: bool = False, seed: Optional[int] = None,
               structure_override=None) -> PagedCase:
    """Draw one layer of a configuration (see the module docstring for the recipe)."""
    if isinstance(spec, str):
        spec = CONFIGS[spec]
    seed = spec.seed if seed is None else seed
    if structure_override is not None:
        lens, table = structure_override
    else:
        lens, table = structure(spec, seed)
    N, Hq, Hkv, D, bs = spec.num_seqs, spec.q_heads, spec.kv_heads, spec.head_dim, spec.block_size
    T = spec.num_query_tokens
    used = np.unique(table[table >= 0])
    rng = np.random.default_rng((seed, layer + 1))

    q32 = rng.standard_normal((N, T, Hq, D) if T > 1 else (N, Hq, D), dtype=np.float32)
    k32 = rng.standard_normal((Hkv, len(used), bs, D), dtype=np.float32)
    v32 = rng.standard_normal((Hkv, len(used), bs, D), dtype=np.float32)
    nk32 = rng.standard_normal((N * T, Hkv, D), dtype=np.float32)
    nv32 = rng.standard_normal((N * T, Hkv, D), dtype=np.float32)

    k_scale = v_scale = None
    shape = (Hkv, spec.num_blocks, bs, D)
    if spec.kv_dtype == "int8":
        kc, ks = quantize_int8_blocks(k32)
        vc, vs = quantize_int8_blocks(v32)
        k_cache = np.zeros(shape, np.int8)
        v_cache = np.zeros(shape, np.int8)
        k_scale = np.ones((Hkv, spec.num_blocks), np.float32)
        v_scale = np.ones((Hkv, spec.num_blocks), np.float32)
        k_cache[:, used] = kc
        v_cache[:, used] = vc
        k_scale[:, used] = ks
        v_scale[:, used] = vs
        if poison:
            poison_int8(k_cache, k_scale, table, lens, bs)
            poison_int8(v_cache, v_scale, table, lens, bs)
        # New tokens are handed over in bf16; an int8 cache write is a separate step.
        new_k = f32_to_bf16_bits(nk32)
        new_v = f32_to_bf16_bits(nv32)
    else:
        st = np.float32 if spec.kv_dtype == "f32" else np.uint16
        k_cache = np.zeros(shape, st)
        v_cache = np.zeros(shape, st)
        k_cache[:, used] = encode(k32, spec.kv_dtype)
        v_cache[:, used] = encode(v32, spec.kv_dtype)
        if poison:
            poison_float(k_cache, spec.kv_dtype, table, lens, bs)
            poison_float(v_cache, spec.kv_dtype, table, lens, bs)
        new_k = encode(nk32, spec.kv_dtype)
        new_v = encode(nv32, spec.kv_dtype)

    q = encode(q32, spec.q_dtype)
    seq_ids = np.repeat(np.arange(N), T)
    positions = (np.repeat(lens.astype(np.int64), T) - T + np.tile(np.arange(T), N))
    keep = positions >= 0
    slot = np.full(N * T, -1, np.int64)
    slot[keep] = slots_for_positions(table, seq_ids[keep], positions[keep], bs)
    return PagedCase(spec=spec, layer=layer, context_lens=lens, block_tables=table, q=q,
                     k_cache=k_cache, v_cache=v_cache, k_scale=k_scale, v_scale=v_scale,
                     new_k=new_k, new_v=new_v, slot_mapping=slot,
                     scale=1.0 / math.sqrt(D))
