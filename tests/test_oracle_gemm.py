"""Pins for the oracle's GEMMs.

The oracle is the plain matrix product.  It is pinned here by things other
than itself:

* brute force on tiny shapes against exact Python integers (int32, reduced
  modulo 2**32) and exact rational sums (``fractions.Fraction``) of values
  decoded by numpy, not by the oracle's codec;
* closed forms: identity, all-ones (= K), rank one, K = 0;
* a library routine: numpy's int64 and float64 matrix products (a different
  summation order, so float results agree within the binary64 error bound);
* the acceptance check itself: it must pass correctly rounded results and
  reject results that carry a planted pipelining mistake (a K tile read from
  the wrong ring slot, a dropped tile).

Shapes are chosen with M, N and K all different so that a transposed
operand or swapped index cannot pass.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from software_pipelined_tiled_pipeline_amd import inputs

U = 2.0 ** -53


def wrap32(v: int) -> int:
    return ((v + 2 ** 31) % 2 ** 32) - 2 ** 31


def f16_vals(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def bf16_vals(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def tiny_shapes():
    rng = np.random.default_rng(7)
    shapes = [(1, 1, 1), (8, 8, 8), (3, 5, 7), (7, 2, 5), (1, 8, 3), (8, 1, 8)]
    shapes += [tuple(int(x) for x in rng.integers(1, 9, 3)) for _ in range(30)]
    return shapes


# ------------------------------------------------------------------ int32

@pytest.mark.parametrize("M,N,K", tiny_shapes())
def test_s32_brute_force(M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    pool = np.array([-2 ** 31, 2 ** 31 - 1, -1, 0, 1, 46341, -46341, 2 ** 30], np.int64)
    A = np.where(rng.random((M, K)) < 0.3, rng.choice(pool, (M, K)),
                 rng.integers(-2 ** 31, 2 ** 31, (M, K))).astype(np.int32)
    B = np.where(rng.random((K, N)) < 0.3, rng.choice(pool, (K, N)),
                 rng.integers(-2 ** 31, 2 ** 31, (K, N))).astype(np.int32)
    got = oracle.gemm_s32_nn(A, B)
    for m in range(M):
        for n in range(N):
            exact = sum(int(A[m, k]) * int(B[k, n]) for k in range(K))
            assert got[m, n] == wrap32(exact)


def test_s32_config_shape_vs_numpy_int64():
    # 128 x 256 x 256 with entries in -8..8: no wrap; numpy's int64 product is exact.
    A, B = inputs.make_operands("s32_nn", 128, 256, 256, inputs.workload_seed(1))
    ref = A.astype(np.int64) @ B.astype(np.int64)
    assert np.array_equal(oracle.gemm_s32_nn(A, B), ref.astype(np.int32))


def test_s32_wrap_vs_numpy_int64():
    rng = np.random.default_rng(3)
    A = rng.integers(-2 ** 31, 2 ** 31, (33, 65)).astype(np.int32)
    B = rng.integers(-2 ** 31, 2 ** 31, (65, 17)).astype(np.int32)
    with np.errstate(over="ignore"):
        ref = (A.astype(np.int64) @ B.astype(np.int64))  # int64 wraps modulo 2**64
    assert np.array_equal(oracle.gemm_s32_nn(A, B), ref.astype(np.int32))


def test_s32_closed_forms():
    K = 37
    I = np.eye(K, dtype=np.int32)
    A = inputs.int32_uniform8((11, K), 5, 0)
    assert np.array_equal(oracle.gemm_s32_nn(A, I), A)
    ones = oracle.gemm_s32_nn(np.ones((4, K), np.int32), np.ones((K, 6), np.int32))
    assert np.all(ones == K)
    u = np.arange(1, 6, dtype=np.int32).reshape(5, 1)
    v = np.arange(-3, 4, dtype=np.int32).reshape(1, 7)
    assert np.array_equal(oracle.gemm_s32_nn(u, v), u * v)
    assert np.array_equal(oracle.gemm_s32_nn(np.zeros((3, 0), np.int32), np.zeros((0, 4), np.int32)),
                          np.zeros((3, 4), np.int32))


# -------------------------------------------------------------- f16 / bf16

def _exact_nt(av, bv):
    M, K = av.shape
    N = bv.shape[0]
    ref = np.empty((M, N), dtype=object)
    mag = np.empty((M, N), dtype=object)
    for m in range(M):
        for n in range(N):
            ps = [Fraction(float(av[m, k])) * Fraction(float(bv[n, k])) for k in range(K)]
            ref[m, n] = sum(ps, Fraction(0))
            mag[m, n] = sum((abs(p) for p in ps), Fraction(0))
    return ref, mag


@pytest.mark.parametrize("M,N,K", tiny_shapes())
def test_f16_brute_force_exact(M, N, K):
    # Values in [-1, 1] are multiples of 2**-24, so every partial sum is a
    # multiple of 2**-48 below 2**5 in magnitude: binary64 holds it exactly and
    # the oracle must equal the rational sum bit for bit.
    seed = M * 100 + N * 10 + K
    A = inputs.f16_uniform1((M, K), seed, 0)
    B = inputs.f16_uniform1((N, K), seed, 1)
    # sprinkle subnormals and exact +-1
    sprinkle = np.array([0x0001, 0x83FF, 0x3C00, 0xBC00, 0x0200], np.uint16)
    idx = np.arange(0, A.size, 5)
    A.flat[idx] = sprinkle[np.arange(idx.size) % sprinkle.size]
    ref, mag = oracle.gemm_nt("f16", A, B)
    eref, emag = _exact_nt(f16_vals(A), f16_vals(B))
    for m in range(M):
        for n in range(N):
            assert Fraction(ref[m, n]) == eref[m, n]
            assert Fraction(mag[m, n]) == emag[m, n]


@pytest.mark.parametrize("M,N,K", tiny_shapes()[:12])
def test_f16_brute_force_extremes(M, N, K):
    # Full binary16 range (subnormals to 65504): binary64 is no longer exact,
    # but sequential summation stays within K * 2**-53 * sum|a*b|.
    rng = np.random.default_rng(M + 10 * N + 100 * K)
    A = rng.integers(0, 0x7C00, (M, K)).astype(np.uint16) | (rng.integers(0, 2, (M, K)) << 15).astype(np.uint16)
    B = rng.integers(0, 0x7C00, (N, K)).astype(np.uint16) | (rng.integers(0, 2, (N, K)) << 15).astype(np.uint16)
    ref, mag = oracle.gemm_nt("f16", A, B)
    eref, emag = _exact_nt(f16_vals(A), f16_vals(B))
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(ref[m, n]) - eref[m, n]) <= Fraction(K * U) * emag[m, n]
            assert abs(Fraction(mag[m, n]) - emag[m, n]) <= Fraction(K * U) * emag[m, n]


@pytest.mark.parametrize("M,N,K", tiny_shapes()[:12])
def test_bf16_brute_force(M, N, K):
    A = inputs.bf16_normal((M, K), 11 + K, 0)
    B = inputs.bf16_normal((N, K), 11 + K, 1)
    ref, mag = oracle.gemm_nt("bf16", A, B)
    eref, emag = _exact_nt(bf16_vals(A), bf16_vals(B))
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(ref[m, n]) - eref[m, n]) <= Fraction(K * U) * emag[m, n]
            assert abs(Fraction(mag[m, n]) - emag[m, n]) <= Fraction(K * U) * emag[m, n]


@pytest.mark.parametrize("fmt,vals", [("f16", f16_vals), ("bf16", bf16_vals)])
def test_nt_vs_numpy_float64(fmt, vals):
    M, N, K = 45, 67, 300
    kind = "f16_nt" if fmt == "f16" else "bf16_nt"
    A, B = inputs.make_operands(kind, M, N, K, 99)
    ref, mag = oracle.gemm_nt(fmt, A, B)
    av, bv = vals(A), vals(B)
    np_ref = av @ bv.T
    np_mag = np.abs(av) @ np.abs(bv).T
    assert np.all(np.abs(ref - np_ref) <= 2 * K * U * np_mag)
    assert np.all(np.abs(mag - np_mag) <= 2 * K * U * np_mag)


def test_nt_closed_forms():
    K = 24
    A = inputs.f16_uniform1((9, K), 4, 0)
    I = np.where(np.eye(K, dtype=bool), np.uint16(0x3C00), np.uint16(0))
    ref, mag = oracle.gemm_nt("f16", A, I)                 # lhs * I^T = lhs
    assert np.array_equal(ref, f16_vals(A))
    assert np.array_equal(mag, np.abs(f16_vals(A)))
    for fmt, one in (("f16", 0x3C00), ("bf16", 0x3F80)):
        for K in (1, 7, 1000, 4096):
            ref, mag = oracle.gemm_nt(fmt, np.full((2, K), one, np.uint16), np.full((3, K), one, np.uint16))
            assert np.all(ref == K) and np.all(mag == K)
    # rank one, K = 1: one exact product; its RNE encoding is numpy's float16 of it
    u = inputs.f16_uniform1((13, 1), 8, 0)
    v = inputs.f16_uniform1((17, 1), 8, 1)
    ref, _ = oracle.gemm_nt("f16", u, v)
    prod = f16_vals(u) @ f16_vals(v).T
    assert np.array_equal(ref, prod)
    assert np.array_equal(oracle.encode("f16", ref), prod.astype(np.float16).view(np.uint16))
    # power-of-two constant rank one over long K: K * u * v exactly
    ref, _ = oracle.gemm_nt("f16", np.full((3, 16384), 0x3800, np.uint16), np.full((2, 16384), 0xB400, np.uint16))
    assert np.all(ref == 16384 * 0.5 * -0.25)
    # K = 0
    ref, mag = oracle.gemm_nt("bf16", np.zeros((3, 0), np.uint16), np.zeros((5, 0), np.uint16))
    assert ref.shape == (3, 5) and np.all(ref == 0) and np.all(mag == 0)


def test_entries_match_full():
    M, N, K = 37, 29, 77
    A, B = inputs.make_operands("bf16_nt", M, N, K, 5)
    ref, mag = oracle.gemm_nt("bf16", A, B)
    rng = np.random.default_rng(0)
    mi = rng.integers(0, M, 200)
    ni = rng.integers(0, N, 200)
    r2, m2 = oracle.gemm_nt_entries("bf16", A, B, mi, ni)
    assert np.array_equal(r2, ref[mi, ni]) and np.array_equal(m2, mag[mi, ni])
    with pytest.raises(IndexError):
        oracle.gemm_nt_entries("bf16", A, B, np.array([M]), np.array([0]))


# ------------------------------------------------------- acceptance check

def test_check_accepts_correct_rounding():
    M, N, K = 64, 80, 1000
    for fmt, kind in (("f16", "f16_nt"), ("bf16", "bf16_nt")):
        A, B = inputs.make_operands(kind, M, N, K, 12)
        ref, mag = oracle.gemm_nt(fmt, A, B)
        bad, worst = oracle.check_nt(fmt, oracle.encode(fmt, ref), ref, mag)
        assert bad == 0 and worst <= 0.5 + 1e-12
        # fp32 accumulation in a different order (numpy, float32, k-blocked) also passes
        vals = f16_vals if fmt == "f16" else bf16_vals
        av, bv = vals(A).astype(np.float32), vals(B).astype(np.float32)
        acc = np.zeros((M, N), np.float32)
        for k0 in range(0, K, 32):
            acc += av[:, k0:k0 + 32] @ bv[:, k0:k0 + 32].T
        got = oracle.encode(fmt, acc.astype(np.float64))
        assert oracle.check_nt(fmt, got, ref, mag)[0] == 0


def test_check_rejects_planted_ring_mistakes():
    # A ring-slot race sums the wrong K tile; an early release drops one.
    # Both must be flagged across the output, with the bound at rel = 1e-3.
    M, N, K, BK = 48, 64, 2048, 64
    A, B = inputs.make_operands("f16_nt", M, N, K, 21)
    av, bv = f16_vals(A), f16_vals(B)
    ref, mag = oracle.gemm_nt("f16", A, B)
    t = 7
    stale = av[:, (t - 1) * BK:t * BK] @ bv[:, (t - 1) * BK:t * BK].T
    fresh = av[:, t * BK:(t + 1) * BK] @ bv[:, t * BK:(t + 1) * BK].T
    wrong_slot = oracle.encode("f16", ref - fresh + stale)
    dropped = oracle.encode("f16", ref - fresh)
    assert oracle.check_nt("f16", wrong_slot, ref, mag)[0] > M * N // 4
    assert oracle.check_nt("f16", dropped, ref, mag)[0] > M * N // 4
    # a transposed output fails too
    assert oracle.check_nt("f16", oracle.encode("f16", ref.T.copy().reshape(M, N)), ref, mag)[0] > M * N // 2
    # and NaN is never accepted
    got = oracle.encode("f16", ref)
    got[3, 4] = 0x7E00
    assert oracle.check_nt("f16", got, ref, mag)[0] == 1


# ------------------------------------------- special values (IEEE 754)

F16_INF, F16_NINF, F16_NAN, F16_MAX = 0x7C00, 0xFC00, 0x7E00, 0x7BFF
BF16_INF, BF16_NINF, BF16_NAN, BF16_MAX = 0x7F80, 0xFF80, 0x7FC0, 0x7F7F
NAN, INF = float("nan"), float("inf")
# (ref, mag, output bits, accepted?) -- overflow threshold 65520 for
# binary16 (65504 plus half its top-binade spacing of 32), 2**128 - 2**119
# for bfloat16 (255 * 2**120 plus half of 2**120)
CHECK_CASES = {
    "f16": [
        (NAN, NAN, F16_NAN, True), (NAN, NAN, F16_INF, False), (NAN, NAN, 0x3C00, False),
        (INF, INF, F16_INF, True), (INF, INF, F16_NINF, False), (INF, INF, F16_MAX, False), (INF, INF, F16_NAN, False),
        (-INF, INF, F16_NINF, True), (-INF, INF, F16_INF, False),
        (1e6, 1e6, F16_INF, True), (1e6, 1e6, F16_MAX, False), (1e6, 1e6, F16_NINF, False), (1e6, 1e6, F16_NAN, False),
        (-1e6, 1e6, F16_NINF, True), (-1e6, 1e6, F16_INF, False),
        (65520.0, 0.0, F16_INF, True), (65520.0, 0.0, F16_MAX, True),    # the threshold itself rounds up
        (65519.0, 0.0, F16_INF, True), (65519.0, 0.0, F16_MAX, True),    # one spacing below
        (65400.0, 0.0, F16_INF, False), (65400.0, 0.0, F16_MAX, False),  # RNE is 65408: three spacings off
        (60000.0, 60000.0, F16_INF, False), (70000.0, 70000.0, F16_MAX, False),
        (1.0, 1.0, F16_NAN, False),
    ],
    "bf16": [
        (NAN, NAN, BF16_NAN, True), (NAN, NAN, BF16_INF, False),
        (INF, INF, BF16_INF, True), (INF, INF, BF16_NINF, False), (INF, INF, BF16_MAX, False),
        (1e39, 1e39, BF16_INF, True), (1e39, 1e39, BF16_MAX, False), (-1e39, 1e39, BF16_NINF, True),
        (2.0 ** 128 - 2.0 ** 119, 0.0, BF16_INF, True),
        (3e38, 3e38, BF16_INF, False), (3.385e38, 0.0, BF16_MAX, True), (3.3e38, 0.0, BF16_MAX, False),
        (1.0, 1.0, BF16_NAN, False),
    ],
}


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_check_special_values(fmt):
    for r, m, bits, want in CHECK_CASES[fmt]:
        bad, worst = oracle.check_nt(fmt, np.array([bits], np.uint16), np.array([r]), np.array([m]))
        assert (bad == 0) == want, (fmt, r, m, hex(bits), want)
        if not want:
            assert worst == INF
    # all at once: the failures are counted, not stopped at
    rows = CHECK_CASES[fmt]
    bad, _ = oracle.check_nt(fmt, np.array([b for _, _, b, _ in rows], np.uint16), np.array([r for r, _, _, _ in rows]),
                             np.array([m for _, m, _, _ in rows]))
    assert bad == sum(1 for *_, w in rows if not w)


def test_oracle_special_products():
    # IEEE 754 arithmetic fixes these: inf * 0 = NaN, inf - inf = NaN, NaN
    # propagates, an infinity plus finite terms stays that infinity
    one, two, five = 0x3C00, 0x4000, 0x4500
    A = np.array([[F16_INF, one, two], [F16_INF, F16_NINF, 0], [F16_NAN, one, one]], np.uint16)
    B = np.array([[0, one, one], [one, one, one], [0xBC00, 0, 0], [one, 0xBC00, five]], np.uint16)
    ref, mag = oracle.gemm_nt("f16", A, B)
    assert np.isnan(ref[0, 0]) and np.isnan(mag[0, 0])
    assert ref[0, 1] == INF and mag[0, 1] == INF
    assert ref[0, 2] == -INF
    assert ref[0, 3] == INF                      # inf*1 + 1*(-1) + 2*5
    assert np.isnan(ref[1, 1])                   # inf + (-inf)
    assert ref[1, 3] == INF                      # inf*1 + (-inf)*(-1)
    assert np.isnan(ref[1, 2])                   # inf*(-1) + (-inf)*0
    assert np.all(np.isnan(ref[2]))
    assert oracle.encode("f16", ref[0:2, 0:4]).tolist() == [[F16_NAN, F16_INF, F16_NINF, F16_INF],
                                                             [F16_NAN, F16_NAN, F16_NAN, F16_INF]]
    # subnormal operands count at their value; their products are exact in binary64
    ref, _ = oracle.gemm_nt("f16", np.array([[0x0001, 0x03FF]], np.uint16), np.array([[0x0001, 0x3C00]], np.uint16))
    assert ref[0, 0] == 2.0 ** -48 + 1023 * 2.0 ** -24
    ref, _ = oracle.gemm_nt("bf16", np.array([[0x0001, 0x007F]], np.uint16), np.array([[0x0001, 0x4F80]], np.uint16))
    assert ref[0, 0] == 2.0 ** -266 + 127 * 2.0 ** -133 * 2.0 ** 32
    # zero products: the sum starts at +0, so only +0 comes out
    ref, mag = oracle.gemm_nt("f16", np.full((1, 4), 0x8000, np.uint16), np.full((1, 4), one, np.uint16))
    assert ref[0, 0] == 0 and not np.signbit(ref[0, 0]) and mag[0, 0] == 0
    assert oracle.encode("f16", ref).tolist() == [[0]]
