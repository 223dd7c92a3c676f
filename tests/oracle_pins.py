"""Pins of the CPU oracle to things other than itself.

Each ``pin_*`` function takes an oracle module (the real one, or a deliberately
broken copy in the mutation tests) and raises AssertionError when the oracle
disagrees with what the pages and the mathematics fix:

* pure-Python brute force on tiny inputs, walking the block table position by
  position with ``math.exp`` / ``math.fsum``;
* closed forms (one position returns its V row; equal keys or a zero scale
  return the mean of V; two positions give logistic weights);
* hand-derived worked examples under ``tests/golden/``;
* a library routine: torch's CPU ``scaled_dot_product_attention`` in float64
  on a dense context built independently of the paged layout, with K/V
  expanded per query head by ``repeat_interleave`` (grouped-query mapping);
* the causal mask of a verify step built the way the prefill code of
  "Anatomy of a Decode-Step Stall" (section "Full Source", engine.py) builds
  it: an upper-triangular -1e9 matrix sliced at the chunk start;
* invariants: physical placement of blocks does not matter; verify with one
  query token is decode; an int8 cache reads as code * per-block scale;
* visibility, not value, decides which keys count: NaN and infinite scores or
  values at visible positions propagate as the dense formula gives them, and
  positions past the context or past a token's causal edge never matter;
* variable-length verify against pure-Python loops over packed rows (with
  sequences of no query token and of more tokens than positions), equal
  counts against fixed-T verify, one token per sequence against decode;
* the cache write, checked against a flat one-index-per-slot view of the
  cache and for untouched bytes.
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch
import torch.nn.functional as F

from paged_kv_gqa_pa_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------------------
# helpers that build inputs (no attention arithmetic)
# ----------------------------------------------------------------------------
def _page_dense(dense, lens, num_blocks, rng, bs=16, max_blocks=None):
    """Scatter a dense per-sequence context [N, Hkv, Lmax, D] into a paged cache.

    Returns (cache [Hkv, num_blocks, bs, D], block_tables)."""
    N, Hkv, Lmax, D = dense.shape
    max_blocks = max_blocks or -(-Lmax // bs)
    perm = rng.permutation(num_blocks).astype(np.int32)
    table = wl.assign_blocks(lens, perm, max_blocks, bs)
    cache = np.zeros((Hkv, num_blocks, bs, D), dense.dtype)
    flat = cache.reshape(Hkv, num_blocks * bs, D)   # one index over the slots of a head
    for b in range(N):
        for j in range(int(lens[b])):
            slot = int(table[b, j // bs]) * bs + j % bs
            flat[:, slot, :] = dense[b, :, j, :]
    return cache, table


def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *rest = line.split()
            vals[key] = np.array([float(x) for x in rest], np.float64)
    return vals


def _sdpa(q, k, v, scale, mask=None):
    """torch CPU float64 SDPA; q [R, H, D] k/v [L, H, D] -> [R, H, D]."""
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))
    kt = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))
    vt = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))
    m = None if mask is None else torch.from_numpy(mask)
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=float(scale))
    return o.numpy().transpose(1, 0, 2)


# ----------------------------------------------------------------------------
# pins
# ----------------------------------------------------------------------------
def _brute_decode(q, kc, vc, table, lens, scale, G):
    """Pure-Python scalar loops over the paged cache (float32 stored inputs)."""
    N, Hq, D = q.shape
    bs = kc.shape[2]
    out = np.zeros((N, Hq, D))
    for b in range(N):
        L = int(lens[b])
        for h in range(Hq):
            g = h // G
            if L == 0:
                continue
            scores = []
            for j in range(L):
                blk = int(table[b][j // bs])
                off = j % bs
                scores.append(scale * math.fsum(float(q[b, h, d]) * float(kc[g, blk, off, d])
                                                for d in range(D)))
            mx = max(scores)
            w = [math.exp(s - mx) for s in scores]
            tot = math.fsum(w)
            for d in range(D):
                acc = []
                for j in range(L):
                    blk = int(table[b][j // bs])
                    acc.append(w[j] * float(vc[g, blk, j % bs, d]))
                out[b, h, d] = math.fsum(acc) / tot
    return out


def _brute_verify_varlen(q, kc, vc, table, lens, qs, scale, G):
    """Pure-Python loops: packed row r of sequence b (T_b rows from qs[b]) is query
    token t = r - qs[b], seeing positions j <= L_b - T_b + t."""
    total, Hq, D = q.shape
    bs = kc.shape[2]
    out = np.zeros((total, Hq, D))
    for b in range(len(qs) - 1):
        L = int(lens[b])
        Tb = int(qs[b + 1]) - int(qs[b])
        for t in range(Tb):
            r = int(qs[b]) + t
            last = L - Tb + t
            for h in range(Hq):
                g = h // G
                seen = [j for j in range(L) if j <= last]
                if not seen:
                    continue
                sc = []
                for j in seen:
                    blk = int(table[b][j // bs])
                    sc.append(scale * math.fsum(float(q[r, h, d]) * float(kc[g, blk, j % bs, d])
                                                for d in range(D)))
                mx = max(sc)
                w = [math.exp(x - mx) for x in sc]
                tot = math.fsum(w)
                for d in range(D):
                    out[r, h, d] = math.fsum(w[i] * float(vc[g, int(table[b][j // bs]), j % bs, d])
                                             for i, j in enumerate(seen)) / tot
    return out


def pin_verify_varlen(oracle):
    """Per-sequence query counts (none, fewer than the context, more than it) against
    brute force; equal counts reduce to fixed-T verify; one token per sequence is decode."""
    rng = np.random.default_rng(77)
    Hkv, G, D, nb = 2, 3, 4, 20
    lens = np.array([5, 0, 33, 3, 17, 2], np.int32)
    counts = np.array([2, 0, 4, 5, 1, 2], np.int64)       # sequence 3: more tokens than positions
    qs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    perm = rng.permutation(nb).astype(np.int32)
    table = wl.assign_blocks(lens, perm, 3)
    kc = rng.standard_normal((Hkv, nb, 16, D)).astype(np.float32)
    vc = rng.standard_normal((Hkv, nb, 16, D)).astype(np.float32)
    q = rng.standard_normal((int(qs[-1]), Hkv * G, D)).astype(np.float32)
    got = oracle.verify_varlen(q, kc, vc, table, lens, qs, 0.41, "f32", "f32")
    want = _brute_verify_varlen(q, kc, vc, table, lens, qs, 0.41, G)
    assert got.shape == want.shape
    assert np.abs(got - want).max() <= 1e-12, "varlen verify vs brute force"
    # equal counts: the fixed-T verify, packed
    T = 3
    lens2 = np.array([9, 40, 3], np.int32)
    table2 = wl.assign_blocks(lens2, rng.permutation(nb).astype(np.int32), 3)
    q2 = rng.standard_normal((3, T, Hkv * G, D)).astype(np.float32)
    qs2 = np.arange(4, dtype=np.int32) * T
    got2 = oracle.verify_varlen(q2.reshape(3 * T, Hkv * G, D), kc, vc, table2, lens2, qs2, 0.5, "f32", "f32")
    want2 = oracle.verify(q2, kc, vc, table2, lens2, 0.5, "f32", "f32").reshape(3 * T, Hkv * G, D)
    assert np.abs(got2 - want2).max() <= 1e-12, "equal counts vs fixed-T verify"
    # one token each: decode
    got3 = oracle.verify_varlen(q2[:, 0], kc, vc, table2, lens2, np.arange(4, dtype=np.int32), 0.5,
                                "f32", "f32")
    want3 = _brute_decode(q2[:, 0], kc, vc, table2, lens2, 0.5, G)
    assert np.abs(got3 - want3).max() <= 1e-12, "one token per sequence vs decode"


def pin_bruteforce_tiny(oracle):
    # The tiny fp32 workload itself, with its poisoned spare blocks.
    case = wl.build_case("tiny_fp32", poison=True)
    got = oracle.decode(case.q, case.k_cache, case.v_cache, case.block_tables,
                        case.context_lens, case.scale, "f32", "f32")
    want = _brute_decode(case.q, case.k_cache, case.v_cache, case.block_tables,
                         case.context_lens, case.scale, 2)
    assert np.abs(got - want).max() <= 1e-12, "tiny_fp32 vs brute force"
    # Random tiny shapes over G and D.
    rng = np.random.default_rng(1234)
    for (Hkv, G, D) in [(1, 1, 1), (2, 2, 4), (1, 3, 4), (2, 8, 4), (3, 1, 64), (2, 3, 64)]:
        N = 3
        lens = rng.integers(0, 40, size=N).astype(np.int32)
        nb = 12
        perm = rng.permutation(nb).astype(np.int32)
        table = wl.assign_blocks(lens, perm, 3)
        kc = rng.standard_normal((Hkv, nb, 16, D)).astype(np.float32)
        vc = rng.standard_normal((Hkv, nb, 16, D)).astype(np.float32)
        q = rng.standard_normal((N, Hkv * G, D)).astype(np.float32)
        sc = 0.37
        got = oracle.decode(q, kc, vc, table, lens, sc, "f32", "f32")
        want = _brute_decode(q, kc, vc, table, lens, sc, G)
        assert np.abs(got - want).max() <= 1e-12, f"brute force Hkv={Hkv} G={G} D={D}"


def pin_closed_forms(oracle):
    rng = np.random.default_rng(7)
    D, nb = 8, 6
    kc = rng.standard_normal((1, nb, 16, D)).astype(np.float32)
    vc = rng.standard_normal((1, nb, 16, D)).astype(np.float32)
    q = rng.standard_normal((1, 1, D)).astype(np.float32)
    table = np.array([[4, 1]], np.int32)
    # One position: the output is that position's V row, exactly.
    o = oracle.decode(q, kc, vc, table, np.array([1], np.int32), 0.5, "f32", "f32")
    assert np.array_equal(o[0, 0], vc[0, 4, 0].astype(np.float64)), "L=1 must return v0"
    # Zero scale: uniform weights, the mean of V over the context (20 positions).
    L = 20
    o = oracle.decode(q, kc, vc, table, np.array([L], np.int32), 0.0, "f32", "f32")
    rows = np.concatenate([vc[0, 4], vc[0, 1, :4]]).astype(np.float64)
    assert np.abs(o[0, 0] - rows.mean(0)).max() < 1e-12, "scale 0 -> mean of V"
    # Equal keys: the mean of V as well.
    kc2 = kc.copy()
    kc2[0, 4] = kc2[0, 4, 0]
    kc2[0, 1] = kc2[0, 4, 0]
    o = oracle.decode(q, kc2, vc, table, np.array([L], np.int32), 0.9, "f32", "f32")
    assert np.abs(o[0, 0] - rows.mean(0)).max() < 1e-12, "equal keys -> mean of V"
    # Two positions: logistic weights.
    o = oracle.decode(q, kc, vc, table, np.array([2], np.int32), 0.7, "f32", "f32")
    s0 = 0.7 * float(np.dot(q[0, 0].astype(np.float64), kc[0, 4, 0]))
    s1 = 0.7 * float(np.dot(q[0, 0].astype(np.float64), kc[0, 4, 1]))
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    want = w0 * vc[0, 4, 0].astype(np.float64) + (1 - w0) * vc[0, 4, 1].astype(np.float64)
    assert np.abs(o[0, 0] - want).max() < 1e-12, "L=2 logistic weights"
    # A negative scale is a scale like any other: two positions again, logistic weights
    # of the negated scores (a softmax over -s favours the smaller score).
    o = oracle.decode(q, kc, vc, table, np.array([2], np.int32), -0.7, "f32", "f32")
    w0n = 1.0 / (1.0 + math.exp(s0 - s1))
    want = w0n * vc[0, 4, 0].astype(np.float64) + (1 - w0n) * vc[0, 4, 1].astype(np.float64)
    assert np.abs(o[0, 0] - want).max() < 1e-12, "negative scale, L=2 logistic weights"
    # Empty context: zero row, no NaN.
    o = oracle.decode(q, kc, vc, table, np.array([0], np.int32), 0.7, "f32", "f32")
    assert np.array_equal(o, np.zeros_like(o)), "L=0 -> zeros"


def pin_golden(oracle):
    g = _read_golden("decode_two_keys.txt")
    kc = np.zeros((1, 7, 16, 2), np.float32)
    vc = np.zeros((1, 7, 16, 2), np.float32)
    kc[0, 5, 0], kc[0, 5, 1] = g["k0"], g["k1"]
    vc[0, 5, 0], vc[0, 5, 1] = g["v0"], g["v1"]
    q = g["q"].astype(np.float32).reshape(1, 1, 2)
    o = oracle.decode(q, kc, vc, np.array([[5]], np.int32), np.array([2], np.int32),
                      float(g["scale"][0]), "f32", "f32")
    assert np.abs(o[0, 0] - g["out"]).max() <= g["tol"][0], "golden decode_two_keys"

    g = _read_golden("verify_three_keys.txt")
    kc = np.zeros((1, 2, 16, 1), np.float32)
    vc = np.zeros((1, 2, 16, 1), np.float32)
    kc[0, 1, :3, 0] = g["keys"]
    vc[0, 1, :3, 0] = g["values"]
    q = g["q"].astype(np.float32).reshape(1, 2, 1, 1)
    o = oracle.verify(q, kc, vc, np.array([[1]], np.int32), np.array([3], np.int32),
                      float(g["scale"][0]), "f32", "f32")
    assert np.abs(o[0, :, 0, 0] - g["out"]).max() <= g["tol"][0], "golden verify_three_keys"


def pin_gqa_against_library(oracle):
    """Paged GQA decode == torch SDPA on the dense, repeat-interleaved context."""
    rng = np.random.default_rng(99)
    for (Hkv, G, D) in [(1, 2, 64), (2, 6, 16), (4, 2, 8), (2, 1, 8)]:
        N, Lmax = 3, 45
        lens = np.array([45, 17, 3], np.int32)
        dense_k = rng.standard_normal((N, Hkv, Lmax, D)).astype(np.float32)
        dense_v = rng.standard_normal((N, Hkv, Lmax, D)).astype(np.float32)
        q = rng.standard_normal((N, Hkv * G, D)).astype(np.float32)
        kc, table = _page_dense(dense_k, lens, 11, np.random.default_rng(5))
        vc, table_v = _page_dense(dense_v, lens, 11, np.random.default_rng(5))
        assert np.array_equal(table, table_v)
        got = oracle.decode(q, kc, vc, table, lens, 0.125, "f32", "f32")
        for b in range(N):
            L = int(lens[b])
            k = np.repeat(dense_k[b, :, :L].astype(np.float64), G, axis=0)   # [Hq, L, D]
            v = np.repeat(dense_v[b, :, :L].astype(np.float64), G, axis=0)
            want = _sdpa(q[b][None].astype(np.float64), k.transpose(1, 0, 2),
                         v.transpose(1, 0, 2), 0.125)[0]
            assert np.abs(got[b] - want).max() < 1e-12, f"GQA vs SDPA Hkv={Hkv} G={G}"


def pin_verify_prefill_mask(oracle):
    """Verify == SDPA with the prefill code's sliced upper-triangular mask."""
    rng = np.random.default_rng(3)
    Hkv, G, D, T = 2, 2, 16, 5
    lens = np.array([5, 23, 40], np.int32)
    N, Lmax = len(lens), 40
    dense_k = rng.standard_normal((N, Hkv, Lmax, D)).astype(np.float32)
    dense_v = rng.standard_normal((N, Hkv, Lmax, D)).astype(np.float32)
    q = rng.standard_normal((N, T, Hkv * G, D)).astype(np.float32)
    kc, table = _page_dense(dense_k, lens, 9, np.random.default_rng(8))
    vc, _ = _page_dense(dense_v, lens, 9, np.random.default_rng(8))
    got = oracle.verify(q, kc, vc, table, lens, 0.25, "f32", "f32")
    M = 64
    causal = np.triu(np.full((M, M), -1e9), k=1)
    for b in range(N):
        end = int(lens[b])
        start = end - T
        mask = causal[start:end, :end]                       # [T, L]
        k = np.repeat(dense_k[b, :, :end].astype(np.float64), G, axis=0).transpose(1, 0, 2)
        v = np.repeat(dense_v[b, :, :end].astype(np.float64), G, axis=0).transpose(1, 0, 2)
        want = _sdpa(q[b].astype(np.float64), k, v, 0.25, mask[None])
        assert np.abs(got[b] - want).max() < 1e-12, f"verify mask seq {b}"
    # One query token: verify is decode.
    q1 = q[:, :1]
    a = oracle.verify(q1, kc, vc, table, lens, 0.25, "f32", "f32")[:, 0]
    d = oracle.decode(q1[:, 0], kc, vc, table, lens, 0.25, "f32", "f32")
    assert np.array_equal(a, d), "verify with T=1 must equal decode"


def pin_placement_invariance(oracle):
    """Relabelling physical blocks (and the table) leaves the result unchanged."""
    case = wl.build_case("qwen2_1p5b_bf16")
    sel = slice(0, 6)
    lens = case.context_lens[sel]
    table = case.block_tables[sel]
    base = oracle.decode(case.q[sel], case.k_cache, case.v_cache, table, lens, case.scale,
                         "bf16", "bf16")
    relabel = np.random.default_rng(11).permutation(case.spec.num_blocks).astype(np.int32)
    kc2 = np.empty_like(case.k_cache)
    vc2 = np.empty_like(case.v_cache)
    kc2[:, relabel] = case.k_cache
    vc2[:, relabel] = case.v_cache
    table2 = np.where(table >= 0, relabel[np.maximum(table, 0)], -1).astype(np.int32)
    moved = oracle.decode(case.q[sel], kc2, vc2, table2, lens, case.scale, "bf16", "bf16")
    assert np.array_equal(base, moved), "placement invariance"


def pin_int8_dequant(oracle):
    """int8 cache reads as code * per-(kv_head, block) scale: SDPA on the dequantised context."""
    rng = np.random.default_rng(21)
    Hkv, G, D, nb = 2, 3, 16, 10
    lens = np.array([33, 7], np.int32)
    perm = rng.permutation(nb).astype(np.int32)
    table = wl.assign_blocks(lens, perm, 3)
    codes = rng.integers(-127, 128, size=(Hkv, nb, 16, D)).astype(np.int8)
    vcodes = rng.integers(-127, 128, size=(Hkv, nb, 16, D)).astype(np.int8)
    ks = rng.uniform(0.001, 0.05, size=(Hkv, nb)).astype(np.float32)
    vs = rng.uniform(0.001, 0.05, size=(Hkv, nb)).astype(np.float32)
    q32 = rng.standard_normal((2, Hkv * G, D)).astype(np.float32)
    q = wl.f32_to_bf16_bits(q32)
    got = oracle.decode(q, codes, vcodes, table, lens, 0.25, "bf16", "int8", ks, vs)
    tq = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).double().numpy()
    for b in range(2):
        L = int(lens[b])
        ks_full = torch.from_numpy(ks).double()[:, :, None, None]
        vs_full = torch.from_numpy(vs).double()[:, :, None, None]
        kd = (torch.from_numpy(codes).double() * ks_full).numpy()
        vd = (torch.from_numpy(vcodes).double() * vs_full).numpy()
        # dense context via the flat slot view
        slots = [int(table[b, j // 16]) * 16 + j % 16 for j in range(L)]
        k = kd.reshape(Hkv, nb * 16, D)[:, slots]           # [Hkv, L, D]
        v = vd.reshape(Hkv, nb * 16, D)[:, slots]
        k = np.repeat(k, G, axis=0).transpose(1, 0, 2)
        v = np.repeat(v, G, axis=0).transpose(1, 0, 2)
        want = _sdpa(tq[b][None], k, v, 0.25)[0]
        assert np.abs(got[b] - want).max() < 1e-12, "int8 dequant vs SDPA"


def pin_visible_nonfinite(oracle):
    """Visibility alone decides which keys count.  The dense formula (max-subtracted
    exponentials over every visible position) gives NaN for a row that sees a NaN
    score or a +inf score (inf - inf), weight 0 to a -inf score, and NaN in dimension
    d for a row that sees a V row with NaN in d; positions a row does not see never
    matter, whatever they hold."""
    rng = np.random.default_rng(41)
    D, nb = 4, 5
    kc = rng.standard_normal((1, nb, 16, D)).astype(np.float32)
    vc = rng.standard_normal((1, nb, 16, D)).astype(np.float32)
    q = np.abs(rng.standard_normal((1, 2, D))).astype(np.float32) + np.float32(0.5)  # q > 0
    table = np.array([[3, 1]], np.int32)
    L = np.array([20], np.int32)

    def with_key(pos, row):
        k = kc.copy()
        k[0, table[0, pos // 16], pos % 16] = row
        return k

    # NaN score at a visible position: every element of every head's row is NaN.
    k_nan = with_key(7, np.array([np.nan, 0, 0, 0], np.float32))
    o = oracle.decode(q, k_nan, vc, table, L, 0.5, "f32", "f32")
    assert np.isnan(o).all(), "a visible NaN score must give a NaN row"
    # +inf score (q > 0 times +inf): inf - inf in the exponent, NaN again.
    k_inf = with_key(18, np.array([np.inf, 0, 0, 0], np.float32))
    o = oracle.decode(q, k_inf, vc, table, L, 0.5, "f32", "f32")
    assert np.isnan(o).all(), "a visible +inf score must give a NaN row"
    # -inf score at the last position: weight exactly 0, so the row is that of the
    # context without it (brute force over the first L - 1 positions).
    k_ninf = with_key(19, np.array([-np.inf, 0, 0, 0], np.float32))
    o = oracle.decode(q, k_ninf, vc, table, L, 0.5, "f32", "f32")
    want = _brute_decode(q, kc, vc, table, L - 1, 0.5, 2)
    assert np.isfinite(o).all() and np.abs(o - want).max() <= 1e-12, "-inf score has weight 0"
    # NaN in dimension 2 of a visible V row: NaN in that dimension only.
    v_nan = vc.copy()
    v_nan[0, table[0, 0], 5, 2] = np.nan
    o = oracle.decode(q, kc, v_nan, table, L, 0.5, "f32", "f32")
    assert np.isnan(o[..., 2]).all() and np.isfinite(np.delete(o, 2, axis=-1)).all(), \
        "a visible NaN value poisons its dimension"
    # Verify: token t sees positions 0 .. L - T + t.  A NaN key at L - T + 1 reaches
    # tokens 1 and 2 only; token 0 is unchanged (and finite).
    T = 3
    qv = np.abs(rng.standard_normal((1, T, 2, D))).astype(np.float32)
    k_nan = with_key(int(L[0]) - T + 1, np.array([np.nan, 0, 0, 0], np.float32))
    o = oracle.verify(qv, k_nan, vc, table, L, 0.5, "f32", "f32")
    clean = oracle.verify(qv, kc, vc, table, L, 0.5, "f32", "f32")
    assert np.isnan(o[0, 1:]).all(), "tokens that see the NaN key must be NaN"
    assert np.array_equal(o[0, 0], clean[0, 0]), "a token that does not see it is unchanged"
    # Positions past the context never matter: a NaN key at position L is not read.
    k_past = with_key(int(L[0]), np.array([np.nan] * D, np.float32))
    o = oracle.decode(q, k_past, vc, table, L, 0.5, "f32", "f32")
    assert np.isfinite(o).all(), "a position past the context must not be read"


def pin_cache_write(oracle):
    rng = np.random.default_rng(5)
    Hkv, nb, D = 3, 7, 8
    kc = rng.standard_normal((Hkv, nb, 16, D)).astype(np.float32)
    vc = rng.standard_normal((Hkv, nb, 16, D)).astype(np.float32)
    key = rng.standard_normal((6, Hkv, D)).astype(np.float32)
    val = rng.standard_normal((6, Hkv, D)).astype(np.float32)
    slots = np.array([0, 17, -1, 111, 50, 16 * nb - 1], np.int64)
    nk, nv = oracle.reshape_and_cache(key, val, kc, vc, slots)
    ek = kc.copy().reshape(Hkv, nb * 16, D)
    ev = vc.copy().reshape(Hkv, nb * 16, D)
    for i, s in enumerate(slots):
        if s >= 0:
            ek[:, s] = key[i]
            ev[:, s] = val[i]
    assert nk.tobytes() == ek.tobytes() and nv.tobytes() == ev.tobytes(), "cache write"
    assert kc.tobytes() != nk.tobytes(), "inputs must not be modified in place"


PINS = [pin_bruteforce_tiny, pin_closed_forms, pin_golden, pin_gqa_against_library,
        pin_verify_prefill_mask, pin_placement_invariance, pin_int8_dequant, pin_cache_write,
        pin_verify_varlen, pin_visible_nonfinite]
