"""int8 caches with the poison convention actually in place.

A pool larger than the blocks in use, every unused block at code 127 with scale
1e30, and the slots past each sequence's context in its partial last block at
code 127 (lengths that are not multiples of 16).  Decode, verify, variable-length
verify and prefill over such a pool must match the oracle, which reads only the
visible positions; the tests first check that the poison is really there.
"""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_gqa_pa_amd import _lib as pa
from paged_kv_gqa_pa_amd import workloads as wl
from tests.gpu_util import TOL, DevCase, dev, max_abs_err

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _case(G, T, seed):
    """8 sequences, contexts U{1000..4000} (+T), 2 KV heads, D = 128, a pool of 4096
    blocks of which ~1250 are used; poisoned."""
    spec = wl.Spec("int8_poison", seed=seed, num_seqs=8, q_heads=2 * G, kv_heads=2, head_dim=128,
                   num_blocks=4096, q_dtype="bf16", kv_dtype="int8", max_len=4000 + T,
                   num_query_tokens=T, len_lo=1000, len_hi=4000)
    case = wl.build_case(spec, poison=True)
    used = np.unique(case.block_tables[case.block_tables >= 0])
    assert len(used) < spec.num_blocks // 2
    assert (case.k_scale == np.float32(1e30)).sum() == 2 * (spec.num_blocks - len(used))
    tails = [(b, int(L)) for b, L in enumerate(case.context_lens) if L % 16]
    assert len(tails) >= 4, "lengths must leave partial last blocks"
    for b, L in tails:
        phys = case.block_tables[b, (L - 1) // 16]
        assert (case.k_cache[:, phys, L % 16:] == 127).all()
        assert (case.v_cache[:, phys, L % 16:] == 127).all()
    return case


@pytest.mark.parametrize("G", [2, 6])
@pytest.mark.parametrize("split", [0, 256])
def test_int8_poison_decode(G, split):
    _say("int8 poison decode G", G, "split", split)
    case = _case(G, 1, 40 + G)
    dc = DevCase(case)
    out = torch.empty_like(dc.q)
    pa.decode(out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, case.scale,
              case.max_context_len, dc.k_scale, dc.v_scale, split_tokens=split)
    torch.cuda.synchronize()
    want = oracle.decode(case.q, case.k_cache, case.v_cache, case.block_tables,
                         case.context_lens, case.scale, "bf16", "int8", case.k_scale,
                         case.v_scale)
    err = max_abs_err(out, want, TOL["int8"])
    assert err < TOL["int8"], err


@pytest.mark.parametrize("G,T", [(2, 5), (3, 5), (6, 5), (8, 5)])
def test_int8_poison_verify(G, T):
    _say("int8 poison verify G", G, "T", T)
    case = _case(G, T, 50 + G)
    dc = DevCase(case)
    for split in (0, 512):
        out = torch.empty_like(dc.q)
        pa.verify(out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens,
                  case.scale, case.max_context_len, dc.k_scale, dc.v_scale, split_tokens=split)
        torch.cuda.synchronize()
        want = oracle.verify(case.q, case.k_cache, case.v_cache, case.block_tables,
                             case.context_lens, case.scale, "bf16", "int8", case.k_scale,
                             case.v_scale)
        err = max_abs_err(out, want, TOL["int8"])
        assert err < TOL["int8"], (split, err)


def _packed(case, counts):
    """Rows 0..T_b-1 of each sequence's q, packed; lengths moved so that they are the
    sequence's last positions (the poisoned slots stay past every length)."""
    T = case.q.shape[1]
    counts = np.asarray(counts, np.int64)
    qs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    qp = np.concatenate([case.q[b, :int(c)] for b, c in enumerate(counts)], axis=0)
    lens = (case.context_lens.astype(np.int64) - T + counts).astype(np.int32)
    return np.ascontiguousarray(qp), qs, lens


def test_int8_poison_verify_varlen():
    _say("int8 poison verify_varlen G 2 T 5")
    case = _case(2, 5, 61)
    dc = DevCase(case)
    counts = np.array([5, 0, 1, 3, 5, 2, 4, 5])
    qp, qs, lens = _packed(case, counts)
    q = dev(qp)
    out = torch.empty_like(q)
    pa.verify_varlen(out, q, dc.k_cache, dc.v_cache, dc.block_tables, dev(lens), dev(qs),
                     case.scale, case.max_context_len, 5, dc.k_scale, dc.v_scale)
    torch.cuda.synchronize()
    want = oracle.verify_varlen(qp, case.k_cache, case.v_cache, case.block_tables, lens, qs,
                                case.scale, "bf16", "int8", case.k_scale, case.v_scale)
    err = max_abs_err(out, want, TOL["int8"])
    assert err < TOL["int8"], err


@pytest.mark.parametrize("G", [2, 6])
def test_int8_poison_prefill(G):
    """The last 200 positions of each sequence as a prefill chunk."""
    _say("int8 poison prefill G", G)
    T = 200
    case = _case(G, 1, 70 + G)
    rng = np.random.default_rng(71 + G)
    q32 = rng.standard_normal((case.num_seqs * T, 2 * G, 128), dtype=np.float32)
    qp = wl.f32_to_bf16_bits(q32)
    qs = (np.arange(case.num_seqs + 1) * T).astype(np.int32)
    dc = DevCase(case)
    q = dev(qp)
    out = torch.empty_like(q)
    pa.prefill(out, q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, dev(qs),
               case.scale, T, dc.k_scale, dc.v_scale)
    torch.cuda.synchronize()
    want = oracle.verify_varlen(qp, case.k_cache, case.v_cache, case.block_tables,
                                case.context_lens, qs, case.scale, "bf16", "int8", case.k_scale,
                                case.v_scale)
    err = max_abs_err(out, want, TOL["int8"])
    assert err < TOL["int8"], err


@pytest.mark.parametrize("entry", ["decode", "verify", "verify_varlen", "prefill"])
@pytest.mark.parametrize("bad", ["short", "transposed"])
def test_int8_scale_shape_checked(entry, bad):
    """Every wrapper refuses scales that are not [kv_heads, num_blocks] before any launch
    (the kernels index them as k_scale[g * num_blocks + block])."""
    _say("int8 scale shape", entry, bad)
    case = _case(2, 5 if entry != "decode" else 1, 80)
    dc = DevCase(case)
    ks = dc.k_scale[:, :-1].contiguous() if bad == "short" else dc.k_scale.t().contiguous()
    out = torch.empty_like(dc.q)
    T = case.q.shape[1] if case.q.ndim == 4 else 1
    with pytest.raises(ValueError, match="k_scale must be"):
        if entry == "decode":
            pa.decode(out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens,
                      case.scale, case.max_context_len, ks, dc.v_scale)
        elif entry == "verify":
            pa.verify(out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens,
                      case.scale, case.max_context_len, ks, dc.v_scale)
        else:
            qs = dev((np.arange(case.num_seqs + 1) * T).astype(np.int32))
            q = dc.q.reshape(-1, *dc.q.shape[2:])
            o = torch.empty_like(q)
            if entry == "verify_varlen":
                pa.verify_varlen(o, q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens,
                                 qs, case.scale, case.max_context_len, T, ks, dc.v_scale)
            else:
                pa.prefill(o, q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, qs,
                           case.scale, T, ks, dc.v_scale)


@pytest.mark.parametrize("v_lo,v_hi", [(1e-6, 1e-6), (200.0, 250.0), (1e-4, 250.0), (1e-9, 1e4)])
def test_int8_v_scale_range(v_lo, v_hi):
    """V scales from tiny to large, mixed per block (the weights times the scale are
    bf16, so no scale over- or underflows them): decode, verify and prefill keep the
    oracle's values to 8e-3 of the output's magnitude (bf16 output rounding is 2^-9
    of it)."""
    _say("int8 v_scale range", v_lo, v_hi)
    case = _case(3, 5, 90)
    rng = np.random.default_rng(91)
    used = np.unique(case.block_tables[case.block_tables >= 0])
    case.v_scale[:, used] = np.exp(rng.uniform(np.log(v_lo), np.log(v_hi), size=(2, len(used))))
    dc = DevCase(case)

    def check(out, want):
        got = out.double().cpu().numpy()
        rel = float(np.abs(got - want).max() / np.abs(want).max())
        max_abs_err(got / np.abs(want).max(), want / np.abs(want).max(), 8e-3)
        assert rel < 8e-3, rel

    want = oracle.verify(case.q, case.k_cache, case.v_cache, case.block_tables,
                         case.context_lens, case.scale, "bf16", "int8", case.k_scale,
                         case.v_scale)
    out = torch.empty_like(dc.q)
    pa.verify(out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, case.scale,
              case.max_context_len, dc.k_scale, dc.v_scale, split_tokens=512)
    torch.cuda.synchronize()
    check(out, want)
    q1 = dc.q[:, 4].contiguous()
    out1 = torch.empty_like(q1)
    pa.decode(out1, q1, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, case.scale,
              case.max_context_len, dc.k_scale, dc.v_scale)
    torch.cuda.synchronize()
    check(out1, want[:, 4])
    qs = (np.arange(case.num_seqs + 1) * 5).astype(np.int32)
    qp = dc.q.reshape(-1, *dc.q.shape[2:])
    outp = torch.empty_like(qp)
    pa.prefill(outp, qp, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, dev(qs),
               case.scale, 5, dc.k_scale, dc.v_scale)
    torch.cuda.synchronize()
    check(outp, want.reshape(-1, *want.shape[2:]))
