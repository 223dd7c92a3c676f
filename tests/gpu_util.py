"""Moving seeded workloads onto the GPU and results back (no attention arithmetic)."""
from __future__ import annotations

import numpy as np
import torch

from paged_kv_gqa_pa_amd import workloads as wl
from tests import parity_log

TOL = {"f32": 1e-4, "bf16": 2e-2, "int8": 2e-2}


def dev(a: np.ndarray) -> torch.Tensor:
    """numpy stored form -> GPU tensor (uint16 bit patterns become bfloat16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def host_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bytes of a GPU tensor as a numpy array (bf16 -> uint16 bit patterns)."""
    if t.dtype == torch.bfloat16:
        return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy()


class DevCase:
    """GPU copies of a PagedCase's arrays."""

    def __init__(self, case):
        self.case = case
        self.q = dev(case.q)
        self.k_cache = dev(case.k_cache)
        self.v_cache = dev(case.v_cache)
        self.block_tables = dev(case.block_tables)
        self.context_lens = dev(case.context_lens)
        opt = lambda a: None if a is None else dev(a)
        self.k_scale = opt(case.k_scale)
        self.v_scale = opt(case.v_scale)
        self.new_k = opt(case.new_k)
        self.new_v = opt(case.new_v)
        self.slot_mapping = opt(case.slot_mapping)


def max_abs_err(gpu, want: np.ndarray, tol: float = None) -> float:
    """Largest |gpu - oracle| over all elements (gpu: a tensor or a host array); the
    output must be finite.  Recorded per test with the tolerance it is held to
    (``tol``, when the caller names it) and printed."""
    got = host_f64(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    assert got.shape == want.shape
    assert np.isfinite(got).all(), "non-finite output"
    err = float(np.abs(got - want).max()) if got.size else 0.0
    excess = None
    if isinstance(gpu, torch.Tensor) and gpu.dtype == torch.bfloat16 and got.size:
        # the kernel's own error: beyond what rounding the oracle to bf16 costs
        # (every bf16 result carries that output rounding)
        bits = wl.f32_to_bf16_bits(want.astype(np.float32)).astype(np.uint32) << np.uint32(16)
        rounded = bits.view(np.float32).astype(np.float64)
        excess = float((np.abs(got - want) - np.abs(rounded - want)).max())
    parity_log.record(err, tol, excess)
    return err
