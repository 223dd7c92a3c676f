"""The oracle against its pins, and proof that the pins catch plausible mistakes.

Each mutation below plants one mistake in a copy of the oracle's source (on
the CPU, never in the product) and checks that at least one pin fails.
"""
import importlib.util
import os
import types

import pytest

import oracle.attention as real_oracle
from tests import oracle_pins

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "attention.py")


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(real_oracle)


MUTATIONS = {
    # block index / offset swapped in the block-table walk
    "walk_offset_as_block": ("phys = np.asarray(table_row)[j // bs]", "phys = np.asarray(table_row)[j % bs]"),
    # wrong GQA mapping: query head group read from the next KV head
    "gqa_wrong_kv_head": ("K = gather_context(k_cache, block_tables[b], L, g, kv_tag, k_scale)\n            V = gather_context(v_cache, block_tables[b], L, g, kv_tag, v_scale)\n            out[b, g * G",
                          "K = gather_context(k_cache, block_tables[b], L, (g + 1) % Hkv, kv_tag, k_scale)\n            V = gather_context(v_cache, block_tables[b], L, (g + 1) % Hkv, kv_tag, v_scale)\n            out[b, g * G"),
    # dropped softmax scale
    "dropped_scale": ("s = (q_rows @ keys.T) * float(scale)", "s = (q_rows @ keys.T)"),
    # the scale's sign dropped
    "scale_magnitude_only": ("s = (q_rows @ keys.T) * float(scale)", "s = (q_rows @ keys.T) * abs(float(scale))"),
    # transposed operand: scores against V instead of K
    "scores_against_v": ("s = (q_rows @ keys.T) * float(scale)", "s = (q_rows @ values.T) * float(scale)"),
    # wrong normaliser
    "normalise_by_max": ("out[r] = (e / e.sum()) @ values[seen]", "out[r] = (e / e.max()) @ values[seen]"),
    # causal off-by-one in verify
    "verify_mask_off_by_one": ("vis = np.arange(L)[None, :] <= np.repeat(last_seen, G)[:, None]",
                               "vis = np.arange(L)[None, :] < np.repeat(last_seen, G)[:, None]"),
    # verify rows interleaved the wrong way (head-major instead of token-major)
    "verify_row_order": ("rows = q64[b, :, g * G:(g + 1) * G].reshape(T * G, D)",
                         "rows = q64[b, :, g * G:(g + 1) * G].transpose(1, 0, 2).reshape(T * G, D)"),
    # int8 scale taken per block of the wrong head
    "int8_scale_wrong_head": ("[kv_head, phys][:, None]", "[0, phys][:, None]"),
    # int8 scale ignored
    "int8_scale_dropped": ("rows = rows * np.asarray(block_scale, np.float64)[kv_head, phys][:, None]", "rows = rows"),
    # bf16 widened from the wrong half
    "bf16_low_half": ("<< np.uint32(16)", "<< np.uint32(8)"),
    # cache write offset from the wrong end
    "cache_write_offset": ("blk, off = int(slot) // bs, int(slot) % bs", "blk, off = int(slot) // bs, bs - 1 - int(slot) % bs"),
    # context length off by one
    "varlen_drop_last_token": ("out[lo:hi] = verify(q[None, lo:hi]", "out[lo:hi - 1] = verify(q[None, lo:hi - 1]"),
    "varlen_first_seq_length": ("context_lens[b:b + 1], scale, q_tag", "context_lens[0:1], scale, q_tag"),
    # keys chosen by the finiteness of their score instead of by visibility
    "mask_by_finite_score": ("seen = seen_all[r]", "seen = seen_all[r] & np.isfinite(s[r])"),
    # visibility ignored (every row sees the whole context)
    "visibility_ignored": ("seen_all = np.ones((R, L), bool) if visible is None else np.asarray(visible, bool)",
                           "seen_all = np.ones((R, L), bool)"),
    "context_short_by_one": ("L = int(context_lens[b])\n        for g in range(Hkv):", "L = max(int(context_lens[b]) - 1, 0)\n        for g in range(Hkv):"),
}


def _mutant(name):
    old, new = MUTATIONS[name]
    src = open(ORACLE_SRC).read()
    assert src.count(old) >= 1, f"mutation {name}: pattern not found"
    src = src.replace(old, new)
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src, f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    mod = _mutant(name)
    failed = []
    for pin in oracle_pins.PINS:
        try:
            pin(mod)
        except (AssertionError, IndexError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"mutation {name} passed every pin"
