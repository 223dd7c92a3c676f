"""ctypes binding of libpa (argument marshalling only).

Every function takes torch tensors on the GPU, checks their dtype, shape and
contiguity, passes raw device pointers and the current HIP stream to the C
ABI (``include/pa.h``), and raises ``PAError`` on a non-OK status.  All
arithmetic runs in the HIP kernels; there is no fallback.

torch is imported before the library is loaded so that libpa binds to the HIP
runtime torch already loaded (both carry the soname libamdhip64.so.7), which
makes torch's streams and device pointers valid inside libpa.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# PA_LIB_VARIANT=debug selects the build with device-side precondition checks.
LIB_PATH = os.path.join(_HERE, "libpa_debug.so" if os.environ.get("PA_LIB_VARIANT") == "debug"
                        else "libpa.so")

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP = 0, -1, -2, -3, -4
PA_F32, PA_BF16, PA_INT8 = 0, 1, 2

EXPORTED = ["pa_version", "pa_last_error", "pa_device_check_status", "pa_reshape_and_cache", "pa_reshape_and_cache_quant",
            "pa_default_split_tokens",
            "pa_workspace_size", "pa_decode", "pa_decode_noalloc", "pa_decode_append", "pa_verify", "pa_verify_varlen",
            "pa_prefill", "pa_plan_size", "pa_plan", "pa_decode_planned",
            "pa_decode_append_planned", "pa_verify_planned", "pa_prefill_plan_size",
            "pa_prefill_plan", "pa_prefill_planned", "pa_decode_append_quant",
            "pa_decode_append_quant_planned"]

_DTYPE = {torch.float32: PA_F32, torch.bfloat16: PA_BF16, torch.int8: PA_INT8}


class PAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libpa status {status}: {message}")
        self.status = status


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run python -m paged_kv_gqa_pa_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.pa_version.restype = i
    lib.pa_version.argtypes = []
    lib.pa_last_error.restype = ctypes.c_char_p
    lib.pa_last_error.argtypes = []
    lib.pa_device_check_status.restype = i
    lib.pa_device_check_status.argtypes = [ctypes.POINTER(ctypes.c_uint), i]
    lib.pa_reshape_and_cache.restype = i
    lib.pa_reshape_and_cache.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, vp]
    lib.pa_reshape_and_cache_quant.restype = i
    lib.pa_reshape_and_cache_quant.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp]
    lib.pa_default_split_tokens.restype = i
    lib.pa_default_split_tokens.argtypes = [i, i, i, i, i]
    lib.pa_workspace_size.restype = sz
    lib.pa_workspace_size.argtypes = [i, i, i, i, i, i, i, i]
    lib.pa_decode.restype = i
    lib.pa_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp,           # pointers
                              i, i, i, i, i, i, i, i,                   # sizes
                              f, i, i, i, vp, sz, vp]
    lib.pa_decode_noalloc.restype = i
    lib.pa_decode_noalloc.argtypes = lib.pa_decode.argtypes[:-3] + [vp]
    lib.pa_decode_append.restype = i
    lib.pa_decode_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                     i, i, i, i, i, i, i, i,
                                     f, i, i, i, vp, sz, vp]
    lib.pa_decode_append_quant.restype = i
    lib.pa_decode_append_quant.argtypes = [vp, vp, vp, vp, i, vp, vp, vp, vp, vp, vp, vp,
                                           i, i, i, i, i, i, i, i,
                                           f, i, vp, sz, vp]
    lib.pa_decode_append_quant_planned.restype = i
    lib.pa_decode_append_quant_planned.argtypes = (lib.pa_decode_append_quant.argtypes[:-1] +
                                                   [vp, sz, vp])
    lib.pa_verify_varlen.restype = i
    lib.pa_verify_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                     i, i, i, i, i, i, i, i, i, i,
                                     f, i, i, i, vp, sz, vp]
    lib.pa_prefill.restype = i
    lib.pa_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp,
                               i, i, i, i, i, i, i, i, i, i,
                               f, i, i, vp]
    lib.pa_verify.restype = i
    lib.pa_verify.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp,
                              i, i, i, i, i, i, i, i, i,
                              f, i, i, i, vp, sz, vp]
    lib.pa_plan_size.restype = sz
    lib.pa_plan_size.argtypes = [i, i, i, i, i, i, i, i]
    lib.pa_plan.restype = i
    lib.pa_plan.argtypes = [vp, vp, i, i, i, i, i, i, i, i, i, vp, sz, vp]
    lib.pa_decode_planned.restype = i
    lib.pa_decode_planned.argtypes = lib.pa_decode.argtypes[:-1] + [vp, sz, vp]
    lib.pa_decode_append_planned.restype = i
    lib.pa_decode_append_planned.argtypes = lib.pa_decode_append.argtypes[:-1] + [vp, sz, vp]
    lib.pa_verify_planned.restype = i
    lib.pa_verify_planned.argtypes = lib.pa_verify.argtypes[:-1] + [vp, sz, vp]
    lib.pa_prefill_plan_size.restype = sz
    lib.pa_prefill_plan_size.argtypes = [i, i, i, i]
    lib.pa_prefill_plan.restype = i
    lib.pa_prefill_plan.argtypes = [vp, vp, i, i, i, i, i, i, vp, sz, vp]
    lib.pa_prefill_planned.restype = i
    lib.pa_prefill_planned.argtypes = lib.pa_prefill.argtypes[:-1] + [vp, sz, vp]
    _lib = lib
    return lib


def lib():
    """The loaded ctypes library (raises ImportError if it is not built)."""
    return _load()


def _check(status: int):
    if status != PA_OK:
        raise PAError(status, _load().pa_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {t.dim()}")


def _int8_scales(kvd, k_scale, v_scale, kv_heads, num_blocks):
    """The per-(KV head, block) scales of an int8 cache, checked against the cache's
    shape (the kernels index them as [kv_heads, num_blocks]); None for other caches."""
    if kvd != PA_INT8:
        return None, None
    for nm, s in (("k_scale", k_scale), ("v_scale", v_scale)):
        if s is None:
            raise ValueError(f"{nm} is required for an int8 cache")
        _need(s, nm, dtype=torch.float32, ndim=2)
        if tuple(s.shape) != (kv_heads, num_blocks):
            raise ValueError(f"{nm} must be [kv_heads, num_blocks] = {(kv_heads, num_blocks)}, "
                             f"got {tuple(s.shape)}")
    return k_scale, v_scale


def version() -> int:
    return _load().pa_version()


PA_CHECK_TABLE_ENTRY, PA_CHECK_CONTEXT_TABLE, PA_CHECK_CONTEXT_MAX = 1, 2, 4
PA_CHECK_SLOT, PA_CHECK_QUERY_START = 8, 16


def device_check_status(clear: bool = True) -> int:
    """The debug library's status word (PA_CHECK_* bits of the preconditions violated
    since the last clear); synchronises the device.  Raises PAError(PA_ERR_UNSUPPORTED)
    with the release library, which checks nothing."""
    flags = ctypes.c_uint(0)
    _check(_load().pa_device_check_status(ctypes.byref(flags), int(bool(clear))))
    return flags.value


def default_split_tokens(q_heads: int, kv_heads: int, head_dim: int, kv_dtype: torch.dtype,
                         num_query_tokens: int = 1) -> int:
    return _load().pa_default_split_tokens(num_query_tokens, q_heads, kv_heads, head_dim,
                                           _DTYPE[kv_dtype])


def workspace_size(num_seqs: int, num_query_tokens: int, q_heads: int, kv_heads: int,
                   head_dim: int, max_context_len: int, kv_dtype: torch.dtype,
                   split_tokens: int = 0) -> int:
    """Bytes of workspace decode/verify need (0 when one piece covers the context)."""
    return _load().pa_workspace_size(num_seqs, num_query_tokens, q_heads, kv_heads, head_dim,
                                     max_context_len, _DTYPE[kv_dtype], split_tokens)


def plan_size(num_seqs: int, num_query_tokens: int, q_heads: int, kv_heads: int, head_dim: int,
              max_context_len: int, kv_dtype: torch.dtype, split_tokens: int = 0) -> int:
    """Bytes of a work plan for these sizes (0 with pa_last_error set when none is possible)."""
    return _load().pa_plan_size(num_seqs, num_query_tokens, q_heads, kv_heads, head_dim,
                                max_context_len, _DTYPE[kv_dtype], split_tokens)


def make_plan(block_tables, context_lens, q_heads, kv_heads, head_dim, max_context_len,
              kv_dtype: torch.dtype, num_query_tokens=1, split_tokens=0, plan=None, stream=None):
    """Work plan (longest units first) for the attention calls of one step; returns the plan
    buffer (a uint8 tensor, allocated when `plan` is None)."""
    _need(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _need(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    N = block_tables.shape[0]
    if context_lens.shape[0] != N:
        raise ValueError("block_tables and context_lens disagree")
    kvd = _DTYPE[kv_dtype]
    need = _load().pa_plan_size(N, int(num_query_tokens), q_heads, kv_heads, head_dim,
                                int(max_context_len), kvd, int(split_tokens))
    if need == 0:
        raise PAError(PA_ERR_UNSUPPORTED, _load().pa_last_error().decode())
    if plan is None:
        plan = torch.empty(need, dtype=torch.uint8, device=block_tables.device)
    _need(plan, "plan")
    _check(_load().pa_plan(_ptr(block_tables), _ptr(context_lens), N, int(num_query_tokens),
                           q_heads, kv_heads, head_dim, block_tables.shape[1],
                           int(max_context_len), kvd, int(split_tokens), _ptr(plan),
                           plan.numel() * plan.element_size(), _stream(stream)))
    return plan


def _plan_args(plan):
    if plan is None:
        return None, 0
    _need(plan, "plan")
    return _ptr(plan), plan.numel() * plan.element_size()


def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, stream=None):
    """Write key/value [num_tokens, kv_heads, head_dim] into the caches at slot_mapping."""
    _need(key, "key", ndim=3)
    _need(value, "value", dtype=key.dtype, ndim=3)
    _need(k_cache, "k_cache", dtype=key.dtype, ndim=4)
    _need(v_cache, "v_cache", dtype=key.dtype, ndim=4)
    _need(slot_mapping, "slot_mapping", dtype=torch.int64, ndim=1)
    H, NB, BS, D = k_cache.shape
    if v_cache.shape != k_cache.shape or key.shape != value.shape:
        raise ValueError("cache or key/value shapes differ")
    T = key.shape[0]
    if key.shape[1:] != (H, D) or slot_mapping.shape[0] != T:
        raise ValueError("key [num_tokens, kv_heads, head_dim] does not match the cache")
    _check(_load().pa_reshape_and_cache(_ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache),
                                        _ptr(slot_mapping), T, H, D, NB, BS, _DTYPE[key.dtype],
                                        _stream(stream)))


def reshape_and_cache_quant(key, value, k_cache, v_cache, k_scale, v_scale, slot_mapping,
                            stream=None):
    """Write bf16/fp32 key/value rows into int8 caches, requantizing each target block.

    k_cache/v_cache [kv_heads, num_blocks, 16, head_dim] int8 and k_scale/v_scale
    [kv_heads, num_blocks] float32 are updated in place.
    """
    _need(key, "key", ndim=3)
    _need(value, "value", dtype=key.dtype, ndim=3)
    _need(k_cache, "k_cache", dtype=torch.int8, ndim=4)
    _need(v_cache, "v_cache", dtype=torch.int8, ndim=4)
    _need(k_scale, "k_scale", dtype=torch.float32, ndim=2)
    _need(v_scale, "v_scale", dtype=torch.float32, ndim=2)
    _need(slot_mapping, "slot_mapping", dtype=torch.int64, ndim=1)
    if key.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("key/value must be bfloat16 or float32")
    H, NB, BS, D = k_cache.shape
    if v_cache.shape != k_cache.shape or key.shape != value.shape:
        raise ValueError("cache or key/value shapes differ")
    if k_scale.shape != (H, NB) or v_scale.shape != (H, NB):
        raise ValueError("scales must be [kv_heads, num_blocks]")
    T = key.shape[0]
    if key.shape[1:] != (H, D) or slot_mapping.shape[0] != T:
        raise ValueError("key [num_tokens, kv_heads, head_dim] does not match the cache")
    _check(_load().pa_reshape_and_cache_quant(
        _ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
        _ptr(slot_mapping), T, H, D, NB, BS, _DTYPE[key.dtype], _stream(stream)))


def _attention(fn_verify: bool, out, q, k_cache, v_cache, block_tables, context_lens, scale,
               max_context_len, k_scale, v_scale, split_tokens, workspace, stream, plan=None):
    _need(q, "q")
    _need(out, "out", dtype=q.dtype)
    if out.shape != q.shape:
        raise ValueError("out must have the shape of q")
    _need(k_cache, "k_cache", ndim=4)
    _need(v_cache, "v_cache", dtype=k_cache.dtype, ndim=4)
    _need(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _need(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    Hkv, NB, BS, D = k_cache.shape
    if fn_verify:
        if q.dim() != 4:
            raise ValueError("verify q must be [num_seqs, num_query_tokens, q_heads, head_dim]")
        N, T, Hq, Dq = q.shape
    else:
        if q.dim() != 3:
            raise ValueError("decode q must be [num_seqs, q_heads, head_dim]")
        N, Hq, Dq = q.shape
        T = 1
    if Dq != D or block_tables.shape[0] != N or context_lens.shape[0] != N:
        raise ValueError("q, block_tables and context_lens disagree with the cache")
    kvd = _DTYPE[k_cache.dtype]
    k_scale, v_scale = _int8_scales(kvd, k_scale, v_scale, Hkv, NB)
    need = _load().pa_workspace_size(N, T, Hq, Hkv, D, int(max_context_len), kvd, int(split_tokens))
    if need and workspace is None:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _need(workspace, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lib_ = _load()
    pp = _plan_args(plan)
    if fn_verify:
        args = [_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                _ptr(block_tables), _ptr(context_lens), N, T, Hq, Hkv, D, BS, NB,
                block_tables.shape[1], int(max_context_len), float(scale), _DTYPE[q.dtype], kvd,
                int(split_tokens), _ptr(workspace), ws_bytes]
        fn = lib_.pa_verify if plan is None else lib_.pa_verify_planned
    else:
        args = [_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                _ptr(block_tables), _ptr(context_lens), N, Hq, Hkv, D, BS, NB,
                block_tables.shape[1], int(max_context_len), float(scale), _DTYPE[q.dtype], kvd,
                int(split_tokens), _ptr(workspace), ws_bytes]
        fn = lib_.pa_decode if plan is None else lib_.pa_decode_planned
    if plan is not None:
        args += list(pp)
    _check(fn(*args, _stream(stream)))
    return out


def decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
                   k_scale=None, v_scale=None, split_tokens=0, stream=None):
    """pa_decode_noalloc: decode with the split-K partials in the library's fixed device
    array (no workspace; nothing allocated)."""
    _need(q, "q", ndim=3)
    _need(out, "out", dtype=q.dtype, ndim=3)
    if out.shape != q.shape:
        raise ValueError("out must have the shape of q")
    _need(k_cache, "k_cache", ndim=4)
    _need(v_cache, "v_cache", dtype=k_cache.dtype, ndim=4)
    _need(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _need(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    Hkv, NB, BS, D = k_cache.shape
    N, Hq, Dq = q.shape
    if Dq != D or block_tables.shape[0] != N or context_lens.shape[0] != N:
        raise ValueError("q, block_tables and context_lens disagree with the cache")
    kvd = _DTYPE[k_cache.dtype]
    k_scale, v_scale = _int8_scales(kvd, k_scale, v_scale, Hkv, NB)
    _check(_load().pa_decode_noalloc(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
        _ptr(block_tables), _ptr(context_lens), N, Hq, Hkv, D, BS, NB, block_tables.shape[1],
        int(max_context_len), float(scale), _DTYPE[q.dtype], kvd, int(split_tokens),
        _stream(stream)))
    return out


def decode(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
           k_scale=None, v_scale=None, split_tokens=0, workspace=None, stream=None, plan=None):
    """Paged GQA decode: q/out [num_seqs, q_heads, head_dim].  With `plan` (make_plan) the
    work starts in the plan's order (pa_decode_planned; same bits)."""
    return _attention(False, out, q, k_cache, v_cache, block_tables, context_lens, scale,
                      max_context_len, k_scale, v_scale, split_tokens, workspace, stream, plan)


def verify(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
           k_scale=None, v_scale=None, split_tokens=0, workspace=None, stream=None, plan=None):
    """Multi-token causal verify: q/out [num_seqs, num_query_tokens, q_heads, head_dim].
    With `plan` (make_plan with num_query_tokens = T): pa_verify_planned."""
    return _attention(True, out, q, k_cache, v_cache, block_tables, context_lens, scale,
                      max_context_len, k_scale, v_scale, split_tokens, workspace, stream, plan)


def verify_varlen(out, q, k_cache, v_cache, block_tables, context_lens, query_start, scale,
                  max_context_len, max_query_tokens, k_scale=None, v_scale=None, split_tokens=0,
                  workspace=None, stream=None):
    """Verify with per-sequence query counts: q/out [total_query_tokens, q_heads, head_dim],
    sequence b's tokens at rows query_start[b] .. query_start[b+1]-1 (int32 [num_seqs+1])."""
    _need(q, "q", ndim=3)
    _need(out, "out", dtype=q.dtype, ndim=3)
    if out.shape != q.shape:
        raise ValueError("out must have the shape of q")
    _need(k_cache, "k_cache", ndim=4)
    _need(v_cache, "v_cache", dtype=k_cache.dtype, ndim=4)
    _need(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _need(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    _need(query_start, "query_start", dtype=torch.int32, ndim=1)
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    Hkv, NB, BS, D = k_cache.shape
    total, Hq, Dq = q.shape
    N = block_tables.shape[0]
    if Dq != D or context_lens.shape[0] != N or query_start.shape[0] != N + 1:
        raise ValueError("q, block_tables, context_lens and query_start disagree")
    kvd = _DTYPE[k_cache.dtype]
    k_scale, v_scale = _int8_scales(kvd, k_scale, v_scale, Hkv, NB)
    T = int(max_query_tokens)
    need = _load().pa_workspace_size(N, T, Hq, Hkv, D, int(max_context_len), kvd, int(split_tokens))
    if need and workspace is None:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _need(workspace, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_load().pa_verify_varlen(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
        _ptr(block_tables), _ptr(context_lens), _ptr(query_start), N, total, T, Hq, Hkv, D, BS,
        NB, block_tables.shape[1], int(max_context_len), float(scale), _DTYPE[q.dtype], kvd,
        int(split_tokens), _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def prefill_plan_size(num_seqs: int, max_query_tokens: int, q_heads: int, kv_heads: int) -> int:
    return _load().pa_prefill_plan_size(num_seqs, max_query_tokens, q_heads, kv_heads)


def make_prefill_plan(context_lens, query_start, total_query_tokens, max_query_tokens, q_heads,
                      kv_heads, max_blocks_per_seq, plan=None, stream=None):
    """Prefill work plan (row tiles longest first) for pa_prefill calls with these offsets and
    lengths; returns the plan buffer (a uint8 tensor, allocated when `plan` is None)."""
    _need(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    _need(query_start, "query_start", dtype=torch.int32, ndim=1)
    N = context_lens.shape[0]
    if query_start.shape[0] != N + 1:
        raise ValueError("query_start must have num_seqs + 1 entries")
    need = _load().pa_prefill_plan_size(N, int(max_query_tokens), q_heads, kv_heads)
    if need == 0:
        raise PAError(PA_ERR_UNSUPPORTED, _load().pa_last_error().decode())
    if plan is None:
        plan = torch.empty(need, dtype=torch.uint8, device=context_lens.device)
    _need(plan, "plan")
    _check(_load().pa_prefill_plan(_ptr(context_lens), _ptr(query_start), N,
                                   int(total_query_tokens), int(max_query_tokens), q_heads,
                                   kv_heads, int(max_blocks_per_seq), _ptr(plan),
                                   plan.numel() * plan.element_size(), _stream(stream)))
    return plan


def prefill(out, q, k_cache, v_cache, block_tables, context_lens, query_start, scale,
            max_query_tokens, k_scale=None, v_scale=None, max_context_len=None, stream=None,
            plan=None):
    """Chunked prefill: q/out [total_query_tokens, q_heads, head_dim] packed by sequence,
    query_start int32 [num_seqs+1]; sequence b's tokens are its last positions.  With `plan`
    (make_prefill_plan): pa_prefill_planned, same bits."""
    _need(q, "q", ndim=3)
    _need(out, "out", dtype=q.dtype, ndim=3)
    if out.shape != q.shape:
        raise ValueError("out must have the shape of q")
    _need(k_cache, "k_cache", ndim=4)
    _need(v_cache, "v_cache", dtype=k_cache.dtype, ndim=4)
    _need(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _need(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    _need(query_start, "query_start", dtype=torch.int32, ndim=1)
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    Hkv, NB, BS, D = k_cache.shape
    total, Hq, Dq = q.shape
    N = block_tables.shape[0]
    if Dq != D or context_lens.shape[0] != N or query_start.shape[0] != N + 1:
        raise ValueError("q, block_tables, context_lens and query_start disagree")
    kvd = _DTYPE[k_cache.dtype]
    k_scale, v_scale = _int8_scales(kvd, k_scale, v_scale, Hkv, NB)
    mcl = block_tables.shape[1] * BS if max_context_len is None else int(max_context_len)
    args = [_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
            _ptr(block_tables), _ptr(context_lens), _ptr(query_start), N, total,
            int(max_query_tokens), Hq, Hkv, D, BS, NB, block_tables.shape[1], mcl, float(scale),
            _DTYPE[q.dtype], kvd]
    if plan is None:
        _check(_load().pa_prefill(*args, _stream(stream)))
    else:
        _check(_load().pa_prefill_planned(*args, *_plan_args(plan), _stream(stream)))
    return out


def decode_append(out, q, key, value, k_cache, v_cache, slot_mapping, block_tables, context_lens,
                  scale, max_context_len, split_tokens=0, workspace=None, stream=None, plan=None):
    """Cache write of one new token per sequence plus decode, in one launch.

    key/value [num_seqs, kv_heads, head_dim]; slot_mapping int64 [num_seqs].
    """
    _need(q, "q", ndim=3)
    _need(out, "out", dtype=q.dtype, ndim=3)
    _need(k_cache, "k_cache", ndim=4)
    _need(v_cache, "v_cache", dtype=k_cache.dtype, ndim=4)
    _need(key, "key", dtype=k_cache.dtype, ndim=3)
    _need(value, "value", dtype=k_cache.dtype, ndim=3)
    _need(slot_mapping, "slot_mapping", dtype=torch.int64, ndim=1)
    _need(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _need(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    Hkv, NB, BS, D = k_cache.shape
    N, Hq, Dq = q.shape
    if (out.shape != q.shape or Dq != D or key.shape != (N, Hkv, D) or value.shape != key.shape
            or slot_mapping.shape[0] != N or block_tables.shape[0] != N
            or context_lens.shape[0] != N or v_cache.shape != k_cache.shape):
        raise ValueError("decode_append: inconsistent shapes")
    kvd = _DTYPE[k_cache.dtype]
    need = _load().pa_workspace_size(N, 1, Hq, Hkv, D, int(max_context_len), kvd, int(split_tokens))
    if need and workspace is None:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = [_ptr(out), _ptr(q), _ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache),
            _ptr(slot_mapping), _ptr(block_tables), _ptr(context_lens), N, Hq, Hkv, D, BS, NB,
            block_tables.shape[1], int(max_context_len), float(scale), _DTYPE[q.dtype], kvd,
            int(split_tokens), _ptr(workspace), ws_bytes]
    if plan is None:
        _check(_load().pa_decode_append(*args, _stream(stream)))
    else:
        _check(_load().pa_decode_append_planned(*args, *_plan_args(plan), _stream(stream)))
    return out


def decode_append_quant(out, q, key, value, k_cache, v_cache, k_scale, v_scale, slot_mapping,
                        block_tables, context_lens, scale, max_context_len, split_tokens=0,
                        workspace=None, stream=None, plan=None):
    """Requantizing cache write of one new token per sequence into an int8 cache plus the
    decode over it, in one launch (pa_decode_append_quant): the same cache bytes, scales and
    output as reshape_and_cache_quant followed by decode.

    key/value [num_seqs, kv_heads, head_dim] bfloat16 or float32; k_cache/v_cache int8 and
    k_scale/v_scale float32 [kv_heads, num_blocks] are updated in place; q/out bfloat16.
    """
    _need(q, "q", dtype=torch.bfloat16, ndim=3)
    _need(out, "out", dtype=torch.bfloat16, ndim=3)
    _need(k_cache, "k_cache", dtype=torch.int8, ndim=4)
    _need(v_cache, "v_cache", dtype=torch.int8, ndim=4)
    _need(k_scale, "k_scale", dtype=torch.float32, ndim=2)
    _need(v_scale, "v_scale", dtype=torch.float32, ndim=2)
    _need(key, "key", ndim=3)
    _need(value, "value", dtype=key.dtype, ndim=3)
    _need(slot_mapping, "slot_mapping", dtype=torch.int64, ndim=1)
    _need(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _need(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    if key.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("key/value must be bfloat16 or float32")
    Hkv, NB, BS, D = k_cache.shape
    N, Hq, Dq = q.shape
    if (out.shape != q.shape or Dq != D or key.shape != (N, Hkv, D) or value.shape != key.shape
            or slot_mapping.shape[0] != N or block_tables.shape[0] != N
            or context_lens.shape[0] != N or v_cache.shape != k_cache.shape):
        raise ValueError("decode_append_quant: inconsistent shapes")
    if k_scale.shape != (Hkv, NB) or v_scale.shape != (Hkv, NB):
        raise ValueError("scales must be [kv_heads, num_blocks]")
    need = _load().pa_workspace_size(N, 1, Hq, Hkv, D, int(max_context_len), PA_INT8,
                                     int(split_tokens))
    if need and workspace is None:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = [_ptr(out), _ptr(q), _ptr(key), _ptr(value), _DTYPE[key.dtype], _ptr(k_cache),
            _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(slot_mapping), _ptr(block_tables),
            _ptr(context_lens), N, Hq, Hkv, D, BS, NB, block_tables.shape[1], int(max_context_len),
            float(scale), int(split_tokens), _ptr(workspace), ws_bytes]
    if plan is None:
        _check(_load().pa_decode_append_quant(*args, _stream(stream)))
    else:
        _check(_load().pa_decode_append_quant_planned(*args, *_plan_args(plan), _stream(stream)))
    return out
