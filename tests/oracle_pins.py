"""Pins for the CPU oracle: checks against values fixed by the definitions and by
mathematics, never against the oracle itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError on a
mismatch.  ``tests/test_oracle_pins.py`` runs them on the oracle;
``tests/test_oracle_mutants.py`` runs them on deliberately broken copies of the
oracle source to show that each plausible mistake fails at least one pin.

Sources of truth used here:
* the hand-derived dequantisation table ``golden/dequant_bf16_table.txt``;
* exact rational arithmetic (``exact_rational.py``) on tiny inputs;
* closed forms (constant codes, one-hot activations, SiLU identities);
* an integer-exact regime where every binary32 partial sum is exact;
* library routines: torch's BF16 cast, its float8 (E4M3, E8M0) decoders for the MXFP4 value sets, numpy's
  matmul and bincount;
* invariants (token permutation, power-of-two scaling, empty experts) and the
  properties that fully determine the routing tensors.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

import exact_rational as X

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _bits_f32(a):
    return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(seed):
    return np.random.default_rng(seed)


def _bf16_of(vals):
    """BF16 bits of float values through torch's cast (a library routine)."""
    import torch

    t = torch.tensor(np.asarray(vals, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def load_dequant_table():
    rows = []
    with open(os.path.join(GOLDEN, "dequant_bf16_table.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            q, s, v, b = line.split()
            rows.append((int(q), int(s, 16), Fraction(v), int(b, 16)))
    return rows


# ------------------------------------------------------------------ dequant

def pin_dequant_table(o):
    rows = load_dequant_table()
    for q, s, exact, bits in rows:
        got = o.dequant_one(q, s)
        assert Fraction(got) == exact, ("dequant value", q, hex(s), got, exact)
        assert o.bf16_rne(got) == bits, ("dequant bf16", q, hex(s), hex(o.bf16_rne(got)), hex(bits))
    # the same table through the array routine, with codes carrying junk in the upper nibble
    by_scale = {}
    for q, s, exact, bits in rows:
        by_scale.setdefault(s, []).append((q, exact, bits))
    for s, entries in by_scale.items():
        K = 32
        codes = np.zeros((len(entries), K), np.uint8)
        for r, (q, _, _) in enumerate(entries):
            codes[r, :] = q | 0xA0  # upper nibble must be ignored
        scales = np.full((len(entries), 1), s, np.uint16)
        f, b = o.dequant(codes, scales)
        for r, (_, exact, bits) in enumerate(entries):
            assert np.all(f[r] == np.float32(float(exact))), ("array dequant", s, r)
            assert np.all(b[r] == bits), ("array dequant bf16", s, r)


def pin_dequant_groups(o):
    # group g covers k in [32g, 32g+32): distinct scales per group must land on the right k
    N, K = 3, 128
    codes = np.full((N, K), 9, np.uint8)                     # q - 8 = 1 -> w = s
    scale_vals = np.array([[0.5, 0.25, 2.0, 4.0], [1.0, 8.0, 0.125, 16.0], [3.0, 5.0, 6.0, 7.0]], np.float32)
    scales = _bf16_of(scale_vals).reshape(N, 4)
    f, _ = o.dequant(codes, scales)
    for n in range(N):
        for k in range(K):
            assert f[n, k] == scale_vals[n, k // 32], ("group index", n, k, f[n, k])


# ------------------------------------------------------------------ bf16 rounding

def pin_bf16_rounding(o):
    specials = [
        (1.0, 0x3F80), (-2.0, 0xC000), (0.0, 0x0000), (-0.0, 0x8000),
        (1.0 + 2.0 ** -8, 0x3F80),                 # tie, even stays
        (1.0 + 3 * 2.0 ** -8, 0x3F82),             # tie, odd rounds up
        (1.0 + 2.0 ** -8 + 2.0 ** -20, 0x3F81),    # just above the tie
        (1.0 + 2.0 ** -9, 0x3F80),                 # below the tie
        (float(np.finfo(np.float32).max), 0x7F80),  # rounds past the largest BF16 -> inf
        (float("inf"), 0x7F80), (float("-inf"), 0xFF80),
        (2.0 ** -133, 0x0001),                      # smallest BF16 subnormal
        (1.5 * 2.0 ** -133, 0x0002),                # subnormal tie -> even
        (2.0 ** -149, 0x0000),                      # far below half the smallest subnormal
    ]
    for v, bits in specials:
        got = o.bf16_rne(v)
        assert got == bits, ("bf16_rne special", v, hex(got), hex(bits))
    nan = o.bf16_rne(float("nan"))
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0, ("NaN must stay NaN", hex(nan))
    # random binary32 values against exact rational RNE and against torch's cast
    r = _rng(7)
    vals = np.concatenate([
        r.standard_normal(3000).astype(np.float32),
        (r.standard_normal(1000) * 1e-38).astype(np.float32),
        (r.standard_normal(1000) * 1e30).astype(np.float32),
        # exact ties: 8 significant bits plus a half ulp
        ((r.integers(128, 256, 1000) * 2 + 1).astype(np.float32) * np.float32(2.0 ** -9)),
    ])
    torch_bits = _bf16_of(vals)
    for v, tb in zip(vals, torch_bits):
        got = o.bf16_rne(float(v))
        assert got == int(tb), ("bf16_rne vs torch", float(v), hex(got), hex(int(tb)))
        ref = X.round_bf16(Fraction(float(v)))
        if ref is not X.INF:
            assert got == X.fraction_to_bf16_bits(ref) or (ref == 0 and got in (0, 0x8000)), \
                ("bf16_rne vs exact", float(v))
    # binary64 inputs that are not binary32 values (a two-step rounding would differ on some)
    d = np.concatenate([r.standard_normal(2000) * 3,
                        (1 + (2 * r.integers(0, 128, 500) + 1) / 256.0) * (1 - 2.0 ** -40)])
    for v in d:
        ref = X.round_bf16(Fraction(float(v)))
        assert o.bf16_rne_f64(float(v)) == X.fraction_to_bf16_bits(ref), ("bf16_rne_f64", float(v))


# ------------------------------------------------------------------ GEMM

def _gemm(o, A, a_row_div, codes, scales, ids, acc64=False):
    return o.grouped_gemm(A, a_row_div, codes, scales, ids, acc64=acc64, nthreads=2)


def pin_gemm_hand_cases(o):
    one = 0x3F80
    # all codes 15, scale 0.5, x = 1: every output = 32 * 7 * 0.5 = 112 exactly
    A = np.full((1, 32), one, np.uint16)
    codes = np.full((1, 4, 32), 15, np.uint8)
    scales = np.full((1, 4, 1), 0x3F00, np.uint16)
    acc, out = _gemm(o, A, 1, codes, scales, np.array([[0]], np.int32))
    assert np.all(acc == 112.0) and np.all(out == 0x42E0), ("all-15 case", acc, out)
    # all codes 8 -> zero
    acc, out = _gemm(o, A, 1, np.full((1, 4, 32), 8, np.uint8), scales, np.array([[0]], np.int32))
    assert np.all(acc == 0.0) and np.all(out == 0), "all-8 case"
    # one-hot activation at k=j across a group boundary (K=64, two scales per row)
    r = _rng(11)
    N, K = 8, 64
    codes = r.integers(0, 16, (1, N, K), dtype=np.uint8)
    sv = r.uniform(0.005, 0.02, (1, N, 2)).astype(np.float32)
    scales = _bf16_of(sv).reshape(1, N, 2)
    s_f = _bits_f32(scales)
    for j in (0, 5, 31, 32, 33, 63):
        xj = 1.5
        A = np.zeros((1, K), np.uint16)
        A[0, j] = _bf16_of([xj])[0]
        acc, out = _gemm(o, A, 1, codes, scales, np.array([[0]], np.int32))
        expect = np.array([xj * (int(codes[0, n, j]) - 8) * float(s_f[0, n, j // 32]) for n in range(N)])
        assert np.array_equal(acc[0], expect), ("one-hot", j, acc[0], expect)
    # route i reads A row i // a_row_div and expert topk_ids[i]
    E, T, k, N, K = 3, 3, 2, 4, 32
    codes = np.stack([np.full((N, K), 8 + e + 1, np.uint8) for e in range(E)])  # w = (e+1) * s
    scales = np.full((E, N, 1), 0x3F80, np.uint16)
    A = np.zeros((T, K), np.uint16)
    for t in range(T):
        A[t, 0] = _bf16_of([float(10 ** t)])[0]
    ids = np.array([[0, 2], [1, 0], [2, -1]], np.int32)
    acc, out = _gemm(o, A, k, codes, scales, ids)
    for i in range(T * k):
        e = ids.reshape(-1)[i]
        if e < 0:
            assert np.all(np.isnan(acc[i])) and np.all(out[i] == 0xFFFF), ("invalid route written", i)
        else:
            assert np.all(acc[i] == float(10 ** (i // k)) * (e + 1)), ("row/expert index", i, acc[i])
    # ids >= E are also not local
    acc, out = _gemm(o, A, k, codes, scales, np.array([[3, 7], [0, 0], [0, 0]], np.int32))
    assert np.all(out[0] == 0xFFFF) and np.all(out[1] == 0xFFFF) and np.all(out[2] != 0xFFFF)


def _tiny_draw(seed, T, E, k, N, K):
    r = _rng(seed)
    A = _bf16_of(r.standard_normal((T, K)))
    A = A.reshape(T, K)
    codes = r.integers(0, 16, (E, N, K), dtype=np.uint8)
    scales = _bf16_of(r.uniform(0.005, 0.02, E * N * (K // 32))).reshape(E, N, K // 32)
    ids = np.argsort(r.random((T, E)), axis=1)[:, :k].astype(np.int32)
    return A, codes, scales, ids


def pin_gemm_exact_rational(o):
    u = 2.0 ** -24
    for seed, (T, E, k, N, K) in enumerate([(2, 3, 2, 8, 32), (3, 4, 2, 6, 64), (4, 2, 1, 5, 96),
                                             (2, 4, 3, 4, 96)]):
        A, codes, scales, ids = _tiny_draw(100 + seed, T, E, k, N, K)
        acc32, out = _gemm(o, A, k, codes, scales, ids, acc64=False)
        acc64, _ = _gemm(o, A, k, codes, scales, ids, acc64=True)
        gamma = K * u / (1 - K * u)
        for i in range(T * k):
            e = int(ids.reshape(-1)[i])
            row = A[i // k]
            for n in range(N):
                terms = [X.bf16_bits_to_fraction(row[kk]) * X.dequant_exact(codes[e, n, kk], scales[e, n, kk // 32])
                         for kk in range(K)]
                exact = sum(terms, Fraction(0))
                if X.binary_span_bits(terms) <= 53:
                    assert Fraction(acc64[i, n]) == exact, ("fp64 accumulation not exact", i, n)
                bound = gamma * float(sum(abs(t) for t in terms))
                assert abs(Fraction(acc32[i, n]) - exact) <= Fraction(bound), ("fp32 error bound", i, n)
                # output bits: RNE of the exact value unless the binary32 error could cross a boundary
                ref = X.round_bf16(exact)
                lo, hi = X.round_bf16(exact - Fraction(bound)), X.round_bf16(exact + Fraction(bound))
                if lo == hi:
                    assert out[i, n] == X.fraction_to_bf16_bits(ref), ("bf16 output", i, n)


def pin_gemm_integer_exact(o):
    # s = 2^-4, x in {-2..2}: every product is a multiple of 2^-4 and every partial sum stays below 2^13,
    # so binary32 accumulation is exact in any order.
    r = _rng(5)
    T, E, k, N, K = 24, 6, 2, 40, 512
    x_int = r.integers(-2, 3, (T, K))
    A = _bf16_of(x_int.astype(np.float32)).reshape(T, K)
    codes = r.integers(0, 16, (E, N, K), dtype=np.uint8)
    scales = np.full((E, N, K // 32), 0x3D80, np.uint16)
    ids = np.argsort(r.random((T, E)), axis=1)[:, :k].astype(np.int32)
    acc, out = _gemm(o, A, k, codes, scales, ids)
    q = codes.astype(np.int64) - 8
    for i in range(T * k):
        e = ids.reshape(-1)[i]
        S = q[e] @ x_int[i // k].astype(np.int64)           # integer sums, numpy int64 matmul
        for n in range(N):
            exact = Fraction(int(S[n]), 16)
            assert Fraction(acc[i, n]) == exact, ("integer regime accumulator", i, n)
            assert out[i, n] == X.fraction_to_bf16_bits(X.round_bf16(exact)), ("integer regime bf16", i, n)


def pin_gemm_library_matmul(o):
    # one expert, every route valid: the grouped GEMM is x @ dequant(W)^T (numpy matmul in binary64)
    r = _rng(9)
    T, N, K = 6, 24, 256
    A = _bf16_of(r.standard_normal((T, K))).reshape(T, K)
    codes = r.integers(0, 16, (1, N, K), dtype=np.uint8)
    scales = _bf16_of(r.uniform(0.005, 0.02, N * K // 32)).reshape(1, N, K // 32)
    W, _ = o.dequant(codes[0], scales[0])
    ref = _bits_f32(A).astype(np.float64) @ W.astype(np.float64).T
    acc64, _ = _gemm(o, A, 1, codes, scales, np.zeros((T, 1), np.int32), acc64=True)
    assert np.allclose(acc64, ref, rtol=1e-12, atol=1e-12), "fp64 accumulation vs numpy matmul"
    acc32, _ = _gemm(o, A, 1, codes, scales, np.zeros((T, 1), np.int32))
    bound = K * 2.0 ** -24 * (np.abs(_bits_f32(A)).astype(np.float64) @ np.abs(W.astype(np.float64)).T)
    assert np.all(np.abs(acc32 - ref) <= bound * 1.01 + 1e-30), "fp32 accumulation vs numpy matmul"


def pin_gemm_invariants(o):
    r = _rng(21)
    T, E, k, N, K = 10, 5, 2, 12, 64
    A, codes, scales, ids = _tiny_draw(21, T, E, k, N, K)
    ids[3, 1] = -1
    ids[7, 0] = E + 3
    acc, out = _gemm(o, A, k, codes, scales, ids)
    # token permutation permutes outputs exactly
    perm = r.permutation(T)
    accp, outp = _gemm(o, A[perm], k, codes, scales, ids[perm])
    route_perm = (perm[:, None] * k + np.arange(k)[None, :]).reshape(-1)
    assert np.array_equal(outp, out[route_perm]), "permutation invariance (bf16)"
    assert np.array_equal(np.nan_to_num(accp, nan=7.0), np.nan_to_num(acc[route_perm], nan=7.0))
    # doubling x doubles every accumulator exactly
    A2 = _bf16_of(2.0 * _bits_f32(A)).reshape(A.shape)
    acc2, _ = _gemm(o, A2, k, codes, scales, ids)
    valid = ~np.isnan(acc)
    assert np.array_equal(acc2[valid], 2.0 * acc[valid]), "linearity in x"
    # doubling the scales doubles every accumulator exactly
    s2 = _bf16_of(2.0 * _bits_f32(scales)).reshape(scales.shape)
    acc3, _ = _gemm(o, A, k, codes, s2, ids)
    assert np.array_equal(acc3[valid], 2.0 * acc[valid]), "linearity in s"
    # invalid routes produce nothing
    assert np.all(out[3 * k + 1] == 0xFFFF) and np.all(out[7 * k + 0] == 0xFFFF)
    # an expert with no routes: changing its weights changes nothing
    used = set(ids.reshape(-1).tolist())
    empty = [e for e in range(E) if e not in used]
    ids_e = ids.copy()
    ids_e[ids_e == 4] = 0
    acc_a, out_a = _gemm(o, A, k, codes, scales, ids_e)
    c2 = codes.copy()
    c2[4] = 15 - c2[4]
    acc_b, out_b = _gemm(o, A, k, c2, scales, ids_e)
    assert np.array_equal(out_a, out_b), "weights of an empty expert leaked"
    del empty


# ------------------------------------------------------------------ routing

def check_route_properties(topk_ids, E, BM, res, bounds):
    """Properties that fully determine the routing tensors (R8 reading: stable, sentinel R)."""
    ids = np.asarray(topk_ids, np.int64).reshape(-1)
    R = ids.size
    valid = (ids >= 0) & (ids < E)
    counts = np.bincount(ids[valid], minlength=E)[:E] if E else np.zeros(0, np.int64)
    assert np.array_equal(res["counts"], counts), "counts"
    assert np.array_equal(res["expert_offsets"], np.concatenate([[0], np.cumsum(counts)])), "offsets"
    padded = (counts + BM - 1) // BM * BM
    ntp = int(padded.sum())
    assert res["num_tokens_padded"] == ntp and ntp % BM == 0, "num_tokens_padded"
    maxP, maxB = bounds
    s = np.asarray(res["sorted_ids"])
    b = np.asarray(res["expert_ids"])
    assert s.size == maxP and b.size == maxB and maxP == maxB * BM and maxP >= ntp, "bounds"
    pos = 0
    for e in range(E):
        seg = s[pos:pos + padded[e]]
        want = np.nonzero(valid & (ids == e))[0]
        assert np.array_equal(seg[:counts[e]], want), ("segment order", e)
        assert np.all(seg[counts[e]:] == R), ("segment sentinel", e)
        assert np.all(b[pos // BM:(pos + padded[e]) // BM] == e), ("block owner", e)
        pos += padded[e]
    assert np.all(s[ntp:] == R), "tail sentinel"
    assert np.all(b[ntp // BM:] == -1), "tail blocks"


def pin_route_prep(o):
    r = _rng(31)
    cases = [(16, 8, 2, 16), (64, 128, 8, 16), (33, 48, 8, 32), (7, 5, 3, 64), (1, 48, 8, 16), (0, 8, 2, 16),
             (300, 16, 4, 128), (5, 1, 1, 16)]
    for idx, (T, E, k, BM) in enumerate(cases):
        ids = np.argsort(r.random((T, max(E, k) + 4)), axis=1)[:, :k].astype(np.int32) - 2  # -2..E+1
        if idx == 2 and T:
            ids[:, :] = np.where(ids % 5 == 0, 3, ids)   # a hot expert
        res = o.route_prep(ids, E, BM)
        check_route_properties(ids, E, BM, res, o.route_bounds(T, k, E, BM))
    # worst case of the bound: every route to a distinct expert
    T, k, E, BM = 4, 4, 16, 16
    ids = np.arange(16, dtype=np.int32).reshape(4, 4)
    res = o.route_prep(ids, E, BM)
    assert res["num_tokens_padded"] == 16 * 16 == o.route_bounds(T, k, E, BM)[0]


# ------------------------------------------------------------------ activation and combine

def pin_silu(o):
    assert o.silu(0.0) == 0.0
    assert abs(o.silu(1.0) - 0.7310585786300049) < 1e-15          # e / (1 + e)
    assert abs(o.silu(-1.0) + 0.2689414213699951) < 1e-15         # -1 / (1 + e)
    for g in (0.3, 1.7, 4.0, 11.0):
        assert abs((o.silu(g) - o.silu(-g)) - g) < 1e-12 * max(1.0, g)   # silu(g) - silu(-g) = g
    assert o.silu(60.0) == 60.0 and abs(o.silu(-60.0)) < 1e-24
    # h = bf16(silu(g) * u); gate comes first in the row, up second
    gu = np.array([[0.0, 1.0, 5.0, 7.0], [2.0, -3.0, 0.0, 1.0], [60.0, 1.0, 0.5, 0.0]], np.float64)
    h = o.silu_mul(gu)
    assert h[0, 0] == 0 and h[0, 1] == X.fraction_to_bf16_bits(X.round_bf16(Fraction(7 * o.silu(1.0))))
    assert h[1, 0] == 0 and h[2, 1] == 0
    assert h[2, 0] == 0x41F0  # silu(60) * 0.5 = 30
    assert h[1, 1] == X.fraction_to_bf16_bits(X.round_bf16(Fraction(o.silu(-3.0))))


def pin_combine(o):
    T, k, H, E = 3, 2, 4, 4
    y = np.zeros((T * k, H), np.float64)
    y[0] = [1.0, 2.0, 3.0, 4.0]
    y[1] = [8.0, 8.0, 8.0, 8.0]
    y[2] = [5.0, -5.0, 0.5, 1.0]
    y[3] = [100.0, 100.0, 100.0, 100.0]          # its route is not local: must be ignored
    y[4] = [9.0, 9.0, 9.0, 9.0]                   # token 2: no valid route
    y[5] = [9.0, 9.0, 9.0, 9.0]
    tw = np.array([[0.25, 0.75], [2.0, 3.0], [1.0, 1.0]], np.float32)
    ids = np.array([[0, 1], [2, -1], [E, -3]], np.int32)
    out, acc = o.combine(y, tw, ids, E, with_acc=True)
    assert np.array_equal(acc[0], [6.25, 6.5, 6.75, 7.0]) and np.array_equal(acc[2], [0.0] * 4), acc
    assert np.array_equal(_bits_f32(out[0]), np.float32([6.25, 6.5, 6.75, 7.0])), out[0]
    assert np.array_equal(_bits_f32(out[1]), np.float32([10.0, -10.0, 1.0, 2.0])), out[1]
    assert np.all(out[2] == 0), "token without local routes must be zero"
    # k=1, weight 1: the combine is the BF16 rounding of y
    yv = _rng(3).standard_normal((5, 7)).astype(np.float32).astype(np.float64)
    out = o.combine(yv, np.ones((5, 1), np.float32), np.zeros((5, 1), np.int32), 1)
    assert np.array_equal(out, _bf16_of(yv.astype(np.float32)).reshape(5, 7))


def pin_fused_composition(o):
    # fused MLP = gate_up (fp32 acc) -> silu*mul (bf16) -> down (fp32 acc) -> combine
    r = _rng(41)
    T, E, k, H, I = 5, 4, 2, 64, 32
    x = _bf16_of(r.standard_normal((T, H))).reshape(T, H)
    c13 = r.integers(0, 16, (E, 2 * I, H), dtype=np.uint8)
    s13 = _bf16_of(r.uniform(0.005, 0.02, E * 2 * I * H // 32)).reshape(E, 2 * I, H // 32)
    c2 = r.integers(0, 16, (E, H, I), dtype=np.uint8)
    s2 = _bf16_of(r.uniform(0.005, 0.02, E * H * I // 32)).reshape(E, H, I // 32)
    ids = np.argsort(r.random((T, E)), axis=1)[:, :k].astype(np.int32)
    ids[4, :] = -1
    ids[1, 1] = E
    tw = r.uniform(0.1, 1.0, (T, k)).astype(np.float32)
    out, h, y = o.fused_moe(x, ids, tw, c13, s13, c2, s2, nthreads=2)
    gu, _ = o.grouped_gemm(x, k, c13, s13, ids, nthreads=2)
    valid = (ids.reshape(-1) >= 0) & (ids.reshape(-1) < E)
    h_ref = o.silu_mul(np.nan_to_num(gu, nan=0.0))
    assert np.array_equal(h[valid], h_ref[valid]), "h"
    y_ref, _ = o.grouped_gemm(h_ref, 1, c2, s2, ids, nthreads=2)
    assert np.array_equal(y[valid], y_ref[valid]), "y"
    out_ref, acc_ref = o.combine(np.nan_to_num(y_ref, nan=0.0), tw, ids, E, with_acc=True)
    assert np.array_equal(out, out_ref), "combine"
    assert np.array_equal(o.last_out_acc, acc_ref), "combine accumulators"
    assert np.array_equal(_bf16_of(acc_ref.astype(np.float32)).reshape(out.shape), out), "acc rounds to out"
    assert np.all(out[4] == 0), "token without local routes"
    # gate rows come first: swapping the gate and up halves of w13 changes h
    c13s = np.concatenate([c13[:, I:], c13[:, :I]], axis=1)
    s13s = np.concatenate([s13[:, I:], s13[:, :I]], axis=1)
    _, h_s, _ = o.fused_moe(x, ids, tw, c13s, s13s, c2, s2, nthreads=2)
    assert not np.array_equal(h_s[valid], h[valid])
    # independent check of h on one route: silu(g) * u from exact gate/up sums rounded once
    i = 0
    e = int(ids.reshape(-1)[i])
    for c in (0, 7, I - 1):
        g = X.gemm_exact(x, k, c13, s13, ids, i, c)
        u_ = X.gemm_exact(x, k, c13, s13, ids, i, I + c)
        want = float(g) / (1.0 + math.exp(-float(g))) * float(u_)
        got = float(_bits_f32(np.array([h[i, c]], np.uint16))[0])
        assert abs(got - want) <= abs(want) * 2.0 ** -7 + 1e-6, ("h vs exact", c, got, want)
    del e


# ------------------------------------------------------------------ MXFP4

def e2m1_via_e4m3():
    """The 16 E2M1 values, each re-encoded bit-wise as the E4M3 value it equals and decoded by torch's float8
    cast (a library routine).  E2M1: bit 3 sign, bits 2..1 exponent with bias 1 (0: subnormal, value m/2),
    bit 0 mantissa; E4M3 has bias 7 and three mantissa bits, so a normal E2M1 (e, m) is E4M3 (e + 6, 4m) and
    the subnormal 0.5 is 2^-1 = E4M3 exponent 6."""
    import torch

    codes = []
    for c in range(16):
        sgn, ex, m = c >> 3, (c >> 1) & 3, c & 1
        if ex == 0:
            mag = 0x30 if m else 0x00
        else:
            mag = ((ex + 6) << 3) | (m << 2)
        codes.append((sgn << 7) | mag)
    t = torch.tensor(codes, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float32)
    return t.numpy().astype(np.float64)


def e8m0_via_torch():
    import torch

    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e8m0fnu).to(torch.float32).numpy()


def mxfp4_exact(table, c, e):
    return Fraction(float(table[c & 15])) * Fraction(2) ** (int(e) - 127)


def pin_mxfp4_values(o):
    table = e2m1_via_e4m3()
    for c in range(16):
        got = o.e2m1(c)
        assert got == table[c] and math.copysign(1.0, got) == math.copysign(1.0, table[c]), ("e2m1", c, got)
    scale = e8m0_via_torch()
    for e in range(255):
        assert o.e8m0(e) == float(scale[e]), ("e8m0", e)
    assert math.isnan(o.e8m0(255)) and math.isnan(float(scale[255]))
    # every code at every scale from 2^-127 to 2^125 (above, 6 * 2^126 leaves binary32): the weight is the exact
    # product
    for e in range(0, 253):
        for c in range(16):
            assert Fraction(o.dequant_mxfp4_one(c | 0xA0, e)) == mxfp4_exact(table, c, e), ("product", c, e)


def pin_mxfp4_dequant_groups(o):
    # group g covers k in [32g, 32g+32) of its row; the BF16 image is the same value (at most 2 significant bits)
    table = e2m1_via_e4m3()
    r = _rng(61)
    N, K = 5, 160
    codes = r.integers(0, 256, (N, K), dtype=np.uint8)          # upper nibble must be ignored
    scales = r.integers(100, 150, (N, K // 32), dtype=np.uint8)
    f, b = o.dequant_mxfp4(codes, scales)
    for n in range(N):
        for k in range(K):
            want = mxfp4_exact(table, codes[n, k], scales[n, k // 32])
            assert Fraction(float(f[n, k])) == want, ("f32", n, k)
            assert Fraction(float(_bits_f32(np.array([b[n, k]], np.uint16))[0])) == want, ("bf16", n, k)


def _mx_draw(seed, T, E, k, N, K):
    r = _rng(seed)
    A = _bf16_of(r.standard_normal((T, K))).reshape(T, K)
    codes = r.integers(0, 16, (E, N, K), dtype=np.uint8)
    scales = r.integers(118, 130, (E, N, K // 32), dtype=np.uint8)
    ids = np.argsort(r.random((T, E)), axis=1)[:, :k].astype(np.int32)
    return A, codes, scales, ids


def pin_mxfp4_gemm_exact_rational(o):
    table = e2m1_via_e4m3()
    u = 2.0 ** -24
    for seed, (T, E, k, N, K) in enumerate([(2, 3, 2, 6, 32), (3, 2, 2, 4, 96)]):
        A, codes, scales, ids = _mx_draw(300 + seed, T, E, k, N, K)
        acc32, out = o.grouped_gemm(A, k, codes, scales, ids, fmt="mxfp4", nthreads=2)
        acc64, _ = o.grouped_gemm(A, k, codes, scales, ids, acc64=True, fmt="mxfp4", nthreads=2)
        gamma = K * u / (1 - K * u)
        for i in range(T * k):
            e = int(ids.reshape(-1)[i])
            for n in range(N):
                terms = [X.bf16_bits_to_fraction(A[i // k][kk]) * mxfp4_exact(table, codes[e, n, kk],
                                                                              scales[e, n, kk // 32])
                         for kk in range(K)]
                exact = sum(terms, Fraction(0))
                if X.binary_span_bits(terms) <= 53:
                    assert Fraction(acc64[i, n]) == exact, ("fp64 accumulation not exact", i, n)
                bound = gamma * float(sum(abs(t) for t in terms))
                assert abs(Fraction(acc32[i, n]) - exact) <= Fraction(bound), ("fp32 error bound", i, n)
                lo, hi = X.round_bf16(exact - Fraction(bound)), X.round_bf16(exact + Fraction(bound))
                if lo == hi:
                    assert out[i, n] == X.fraction_to_bf16_bits(X.round_bf16(exact)), ("bf16 output", i, n)


def pin_mxfp4_gemm_library_matmul(o):
    # one expert, every route valid: x @ W^T with W from the library-decoded value tables (numpy, binary64)
    table = e2m1_via_e4m3()
    scale = e8m0_via_torch().astype(np.float64)
    r = _rng(62)
    T, N, K = 5, 20, 192
    A = _bf16_of(r.standard_normal((T, K))).reshape(T, K)
    codes = r.integers(0, 16, (1, N, K), dtype=np.uint8)
    scales = r.integers(110, 140, (1, N, K // 32), dtype=np.uint8)
    W = table[codes[0]] * np.repeat(scale[scales[0]], 32, axis=1)
    ref = _bits_f32(A).astype(np.float64) @ W.T
    acc64, _ = o.grouped_gemm(A, 1, codes, scales, np.zeros((T, 1), np.int32), acc64=True, fmt="mxfp4")
    assert np.allclose(acc64, ref, rtol=1e-12, atol=1e-30), "fp64 accumulation vs numpy matmul"


def pin_mxfp4_fused_composition(o):
    r = _rng(63)
    T, E, k, H, I = 4, 3, 2, 64, 32
    x = _bf16_of(r.standard_normal((T, H))).reshape(T, H)
    c13 = r.integers(0, 16, (E, 2 * I, H), dtype=np.uint8)
    s13 = r.integers(120, 128, (E, 2 * I, H // 32), dtype=np.uint8)
    c2 = r.integers(0, 16, (E, H, I), dtype=np.uint8)
    s2 = r.integers(120, 128, (E, H, I // 32), dtype=np.uint8)
    ids = np.argsort(r.random((T, E)), axis=1)[:, :k].astype(np.int32)
    ids[3, 0] = -1
    tw = r.uniform(0.1, 1.0, (T, k)).astype(np.float32)
    out, h, y = o.fused_moe(x, ids, tw, c13, s13, c2, s2, nthreads=2, fmt="mxfp4")
    gu, _ = o.grouped_gemm(x, k, c13, s13, ids, nthreads=2, fmt="mxfp4")
    valid = (ids.reshape(-1) >= 0) & (ids.reshape(-1) < E)
    h_ref = o.silu_mul(np.nan_to_num(gu, nan=0.0))
    assert np.array_equal(h[valid], h_ref[valid]), "h"
    y_ref, _ = o.grouped_gemm(h_ref, 1, c2, s2, ids, nthreads=2, fmt="mxfp4")
    assert np.array_equal(y[valid], y_ref[valid]), "y"
    out_ref, _ = o.combine(np.nan_to_num(y_ref, nan=0.0), tw, ids, E, with_acc=True)
    assert np.array_equal(out, out_ref), "combine"


ALL_PINS = [pin_dequant_table, pin_dequant_groups, pin_bf16_rounding, pin_gemm_hand_cases,
            pin_gemm_exact_rational, pin_gemm_integer_exact, pin_gemm_library_matmul, pin_gemm_invariants,
            pin_route_prep, pin_silu, pin_combine, pin_fused_composition, pin_mxfp4_values,
            pin_mxfp4_dequant_groups, pin_mxfp4_gemm_exact_rational, pin_mxfp4_gemm_library_matmul,
            pin_mxfp4_fused_composition]
