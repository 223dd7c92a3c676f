"""The requantizing int8 cache-write oracle against its pins, and mutations the pins catch.

Each mutation plants one plausible mistake in a copy of the oracle's source
(on the CPU) and checks that at least one pin fails.
"""
import os
import types

import pytest

import oracle.requant as real
from tests import oracle_pins_requant as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "requant.py")


@pytest.mark.parametrize("pin", pins.PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(real)


MUTATIONS = {
    "floor_instead_of_rint": ("q = np.rint(x / new_scale)", "q = np.floor(x / new_scale)"),
    "scale_not_recomputed": ("new_scale = np.float32(amax / _F127) if amax > 0 else np.float32(1.0)",
                             "new_scale = np.float32(scale)"),
    "codes_not_dequantized": ("x = np.asarray(codes, dtype=np.int8).astype(np.float32) * np.float32(scale)",
                              "x = np.asarray(codes, dtype=np.int8).astype(np.float32)"),
    "row_not_written": ("x[offset, :] = row_f32", "x[offset, :] = x[offset, :]"),
    "scale_from_new_row_only": ("amax = np.float32(np.abs(x).max())", "amax = np.float32(np.abs(row_f32).max())"),
    "scale_over_128": ("_F127 = np.float32(127.0)", "_F127 = np.float32(128.0)"),
    "v_uses_k_scale": ("vc[g, blk], vs[g, blk] = requantize_block(vc[g, blk], vs[g, blk], off,",
                       "vc[g, blk], vs[g, blk] = requantize_block(vc[g, blk], ks[g, blk], off,"),
    "reverse_token_order": ("for i, slot in enumerate(np.asarray(slot_mapping, np.int64)):",
                            "for i, slot in reversed(list(enumerate(np.asarray(slot_mapping, np.int64)))):"),
    "offset_from_end": ("blk, off = int(slot) // bs, int(slot) % bs", "blk, off = int(slot) // bs, bs - 1 - int(slot) % bs"),
    "zero_block_scale_zero": ("if amax > 0 else np.float32(1.0)", "if amax > 0 else np.float32(0.0)"),
}


def _mutant(name):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation {name}: pattern not found"
    mod = types.ModuleType(f"requant_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    mod = _mutant(name)
    failed = []
    for pin in pins.PINS:
        try:
            with __import__("numpy").errstate(all="ignore"):
                pin(mod)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"no pin catches mutation {name}"
