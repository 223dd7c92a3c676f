"""GPU parity of pa_verify (k+1 speculative tokens, causal among themselves)."""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_gqa_pa_amd import _lib as pa
from paged_kv_gqa_pa_amd import workloads as wl
from tests.gpu_util import TOL, DevCase, host_bits, max_abs_err

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _verify(dc, split=0, max_len=None):
    case = dc.case
    out = torch.empty_like(dc.q)
    pa.verify(out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, case.scale,
              case.max_context_len if max_len is None else max_len, dc.k_scale, dc.v_scale,
              split_tokens=split)
    torch.cuda.synchronize()
    return out


def _oracle_verify(case):
    return oracle.verify(case.q, case.k_cache, case.v_cache, case.block_tables,
                         case.context_lens, case.scale, case.spec.q_dtype, case.spec.kv_dtype,
                         case.k_scale, case.v_scale)


@pytest.mark.parametrize("split", [0, 256])
def test_spec_verify_full_size(split):
    """64 sequences, 5 new tokens each written first, then verified."""
    _say("spec_verify_bf16 split", split)
    case = wl.build_case("spec_verify_bf16", poison=True)
    dc = DevCase(case)
    pa.reshape_and_cache(dc.new_k, dc.new_v, dc.k_cache, dc.v_cache, dc.slot_mapping)
    torch.cuda.synchronize()
    want_k, want_v = oracle.reshape_and_cache(case.new_k, case.new_v, case.k_cache,
                                              case.v_cache, case.slot_mapping)
    assert host_bits(dc.k_cache).tobytes() == want_k.tobytes()
    case.k_cache, case.v_cache = want_k, want_v
    out = _verify(dc, split)
    err = max_abs_err(out, _oracle_verify(case))
    assert err < TOL["bf16"], err


def _random_verify_case(rng, lens, Hkv, G, D, T, poison=False, kv="bf16"):
    lens = np.asarray(lens, np.int32)
    maxb = max(1, -(-int(lens.max()) // 16))
    need = int(sum(-(-int(L) // 16) for L in lens))
    nb = need + 5
    table = wl.assign_blocks(lens, rng.permutation(nb).astype(np.int32), maxb)
    k32 = rng.standard_normal((Hkv, nb, 16, D), dtype=np.float32)
    v32 = rng.standard_normal((Hkv, nb, 16, D), dtype=np.float32)
    if poison:
        used = np.unique(table[table >= 0])
        spare = np.setdiff1d(np.arange(nb), used)
        k32[:, spare] = np.nan
        v32[:, spare] = np.nan
        for b, L in enumerate(lens):
            if L % 16:
                phys = table[b, (int(L) - 1) // 16]
                k32[:, phys, L % 16:] = np.nan
                v32[:, phys, L % 16:] = np.nan
    q = wl.f32_to_bf16_bits(rng.standard_normal((len(lens), T, Hkv * G, D), dtype=np.float32))
    spec = wl.Spec("random_verify", 0, len(lens), Hkv * G, Hkv, D, nb, "bf16", kv,
                   max(16, int(lens.max())), num_query_tokens=T)
    if kv == "int8":
        # blocks quantised from their clean draws, then the int8 poison: spare blocks
        # at code 127 with scale 1e30, tails of partial last blocks at code 127
        kc, ks = wl.quantize_int8_blocks(np.nan_to_num(k32, nan=0.0))
        vc, vs = wl.quantize_int8_blocks(np.nan_to_num(v32, nan=0.0))
        if poison:
            wl.poison_int8(kc, ks, table, lens)
            wl.poison_int8(vc, vs, table, lens)
    else:
        kc, vc, ks, vs = wl.f32_to_bf16_bits(k32), wl.f32_to_bf16_bits(v32), None, None
    return wl.PagedCase(spec=spec, layer=0, context_lens=lens, block_tables=table, q=q,
                        k_cache=kc, v_cache=vc, k_scale=ks, v_scale=vs, new_k=None, new_v=None,
                        slot_mapping=None, scale=1.0 / np.sqrt(D))


EDGE = [0, 1, 2, 3, 4, 5, 6, 15, 16, 17, 21, 33, 100, 255, 256, 257, 700]


@pytest.mark.parametrize("kv", ["bf16", "int8"])
# up to 16 rows per (sequence, KV head): one row tile; 17..48: two or three row
# tiles; beyond 48 the prefill kernel
@pytest.mark.parametrize("G,T", [(1, 1), (1, 16), (2, 5), (3, 5), (2, 8), (8, 2), (16, 1), (6, 2),
                                 (4, 5), (6, 5), (8, 5), (16, 3), (3, 17), (16, 5), (8, 16)])
@pytest.mark.parametrize("D", [64, 128])
def test_verify_edges(G, T, D, kv):
    _say("verify edges", kv, "G", G, "T", T, "D", D)
    rng = np.random.default_rng(1000 + 10 * G + T + D)
    case = _random_verify_case(rng, EDGE, Hkv=2, G=G, D=D, T=T, poison=True, kv=kv)
    dc = DevCase(case)
    want = _oracle_verify(case)
    for split in (0, 32):
        out = _verify(dc, split)
        err = max_abs_err(out, want)
        assert err < TOL[kv], (split, err)
    got = out.float().cpu().numpy()
    # a row with no visible position (context shorter than the tokens before it) is zero
    for b, L in enumerate(case.context_lens):
        for t in range(T):
            if L - T + t < 0:
                assert (got[b, t] == 0).all()


def test_verify_rows_match_decode_at_shorter_contexts():
    """Row t of verify is decode with context L - T + t + 1 and that token's query."""
    _say("verify vs decode rows")
    rng = np.random.default_rng(7)
    T = 5
    case = _random_verify_case(rng, [40, 300, 517], Hkv=2, G=2, D=128, T=T)
    dc = DevCase(case)
    out = _verify(dc).float().cpu().numpy()
    for t in range(T):
        lens_t = (case.context_lens - T + t + 1).astype(np.int32)
        want = oracle.decode(np.ascontiguousarray(case.q[:, t]), case.k_cache, case.v_cache,
                             case.block_tables, lens_t, case.scale, "bf16", "bf16")
        dec = torch.empty_like(dc.q[:, t])
        pa.decode(dec, dc.q[:, t].contiguous(), dc.k_cache, dc.v_cache, dc.block_tables,
                  torch.from_numpy(lens_t).cuda(), case.scale, case.max_context_len)
        torch.cuda.synchronize()
        assert max_abs_err(out[:, t], want, TOL["bf16"]) < TOL["bf16"]
        assert max_abs_err(dec, want, TOL["bf16"]) < TOL["bf16"]


def test_verify_unsupported_shapes_rejected():
    rng = np.random.default_rng(3)
    case = _random_verify_case(rng, [20], Hkv=1, G=4, D=96, T=5)   # head_dim 96 is not built
    dc = DevCase(case)
    with pytest.raises(pa.PAError) as ei:
        _verify(dc)
    assert ei.value.status == pa.PA_ERR_UNSUPPORTED


@pytest.mark.parametrize("kv", ["bf16", "int8"])
@pytest.mark.parametrize("G,T", [(6, 5), (8, 5), (16, 5)])
def test_verify_many_rows_full_size(G, T, kv):
    """The speculative workload's sequences (64, context U{256..1024} + T) with group
    sizes whose rows fill two or three row tiles, or go to the prefill kernel (80 rows),
    on a poisoned cache; every output row against the oracle."""
    _say("verify many rows", kv, "G", G, "T", T)
    spec = wl.CONFIGS["spec_verify_bf16"]
    lens, _ = wl.structure(spec)
    lens = (lens - spec.num_query_tokens + T).astype(np.int32)
    rng = np.random.default_rng(1300 + G + T)
    case = _random_verify_case(rng, lens[:32], Hkv=2, G=G, D=128, T=T, poison=True, kv=kv)
    dc = DevCase(case)
    want = _oracle_verify(case)
    for split in (0, 256):
        err = max_abs_err(_verify(dc, split), want, TOL[kv])
        assert err < TOL[kv], (split, err)
