"""ctypes binding of libpa_probe.so (bandwidth reference kernels, include/pa_probe.h).

Measurement only: the benchmark uses these to report the attention kernels'
bandwidth against what a plain read achieves on the same device.
"""
from __future__ import annotations

import ctypes
import os

import torch

from ._lib import _ptr, _stream

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa_probe.so")
EXPORTED = ["pa_probe_last_error", "pa_probe_stream_read", "pa_probe_tile_read"]

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run python -m paged_kv_gqa_pa_amd.build")
        l = ctypes.CDLL(LIB_PATH)
        vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        l.pa_probe_last_error.restype = ctypes.c_char_p
        l.pa_probe_last_error.argtypes = []
        l.pa_probe_stream_read.restype = i
        l.pa_probe_stream_read.argtypes = [vp, sz, i, vp, vp]
        l.pa_probe_tile_read.restype = i
        l.pa_probe_tile_read.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp, vp]
        _lib = l
    return _lib


def _check(status):
    if status != 0:
        raise RuntimeError(f"libpa_probe status {status}: {lib().pa_probe_last_error().decode()}")


def stream_read(buf: torch.Tensor, sink: torch.Tensor, grid: int = 0, stream=None):
    """Read every byte of the contiguous GPU tensor `buf` once."""
    _check(lib().pa_probe_stream_read(_ptr(buf), buf.numel() * buf.element_size(), grid,
                                      _ptr(sink), _stream(stream)))


def tile_read(k_cache, v_cache, block_tables, context_lens, max_context_len, split_tokens,
              sink, waves=4, stream=None):
    """The decode's K/V reads over a [kv_heads, num_blocks, 16, D] cache, without arithmetic."""
    H, NB, BS, D = k_cache.shape
    _check(lib().pa_probe_tile_read(_ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                    _ptr(context_lens), block_tables.shape[0], H,
                                    block_tables.shape[1], NB, D * k_cache.element_size(),
                                    split_tokens, max_context_len, waves, _ptr(sink),
                                    _stream(stream)))
