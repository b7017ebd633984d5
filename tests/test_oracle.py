"""Pins for the CPU oracle, against things other than the oracle itself.

The pages print no worked numeric example for the GEMM+ReLU program, so the
oracle is pinned by
  * library routines for the fp16 codec (numpy's float16 conversions),
  * an independent exact model (Python Fractions, exact sums, exact
    round-half-even) on tiny shapes,
  * math.fsum (correctly rounded sums) on a mid-size problem,
  * closed forms (ones, identity, permutation, integer matrices, ties,
    subnormals, overflow) and invariants (C >= 0, scaling, layout padding).
A dropped term, a wrong sign, a transposed operand, an index slip, a flushed
subnormal or a truncating store each fails at least one of these.
"""

import json
import math
import os
from bisect import bisect_right
from fractions import Fraction

import numpy as np
import pytest

import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def bits_to_f64(b):
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float64)


# --------------------------------------------------------------------------- codec


def test_dec16_exhaustive(oracle_lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle_lib.dec16(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signs of zero survive
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def _enc_candidates():
    finite = np.arange(0x7C00, dtype=np.uint16)          # +0 .. 65504
    v = finite.view(np.float16).astype(np.float64)
    mids = (v[:-1] + v[1:]) / 2                            # exact in binary64
    up = np.nextafter(mids, np.inf)
    dn = np.nextafter(mids, -np.inf)
    special = np.array([65504.0, 65519.99, np.nextafter(65520.0, 0), 65520.0, 65536.0, 1e9,
                        2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14, np.nextafter(2.0 ** -14, 0),
                        np.nextafter(2.0 ** -25, 0), np.nextafter(2.0 ** -25, 1), 2.0 ** -26,
                        2.0 ** -24 * 1.5, 2.0 ** -24 * 2.5, 1e-300, 5e-324, 0.0, np.inf])
    x = np.concatenate([v, mids, up, dn, special])
    return np.concatenate([x, -x])


def test_enc16_matches_numpy_at_values_midpoints_and_neighbours(oracle_lib):
    x = _enc_candidates()
    got = oracle_lib.enc16(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(x[i], hex(got[i]), hex(ref[i])) for i in bad[:10]]


def test_enc16_ties_go_to_even_by_hand(oracle_lib):
    # 1 + 2^-11 lies halfway between 1 (mantissa 0, even) and 1 + 2^-10 (odd)
    assert oracle_lib.enc16([1 + 2.0 ** -11])[0] == 0x3C00
    # 1 + 3*2^-11 lies halfway between 1 + 2^-10 (odd) and 1 + 2^-9 (even)
    assert oracle_lib.enc16([1 + 3 * 2.0 ** -11])[0] == 0x3C02
    # overflow boundary: 65520 ties to the even neighbour 2^16 = inf
    assert oracle_lib.enc16([65520.0])[0] == 0x7C00
    assert oracle_lib.enc16([65519.0])[0] == 0x7BFF
    # subnormal grid: 2^-25 ties to 0, 3*2^-26 rounds up to 2^-24
    assert oracle_lib.enc16([2.0 ** -25])[0] == 0x0000
    assert oracle_lib.enc16([3 * 2.0 ** -26])[0] == 0x0001
    # the largest subnormal rounding up into the smallest normal
    assert oracle_lib.enc16([2.0 ** -14 - 2.0 ** -26])[0] == 0x0400


def test_relu_store(oracle_lib):
    x = np.array([-1.0, -0.0, 0.0, 2.0 ** -30, 2.0 ** -25, 1.0, -65504.0, np.nan, 1e6])
    got = oracle_lib.relu_store(x)
    assert list(got) == [0, 0, 0, 0, 0, 0x3C00, 0, 0, 0x7C00]


# ----------------------------------------------------------------- exact brute force

_POS_F16 = [Fraction(float(v)) for v in np.arange(0x7C00, dtype=np.uint16).view(np.float16)]


def _rne_fraction(r: Fraction) -> int:
    """Exact round-half-even of a rational to fp16 bits, after ReLU."""
    if r <= 0:
        return 0
    if r >= 65520:
        return 0x7C00
    k = bisect_right(_POS_F16, r) - 1
    if k == len(_POS_F16) - 1:
        return k
    lo, hi = _POS_F16[k], _POS_F16[k + 1]
    dl, dh = r - lo, hi - r
    if dl < dh:
        return k
    if dh < dl:
        return k + 1
    return k if k % 2 == 0 else k + 1


def _exact_gemm_relu(a_bits, b_bits, M, N, K):
    av = [Fraction(float(x)) for x in bits_to_f64(a_bits)]
    bv = [Fraction(float(x)) for x in bits_to_f64(b_bits)]
    out = np.zeros(M * N, dtype=np.uint16)
    for i in range(M):
        for j in range(N):
            s = sum((av[i * K + k] * bv[k * N + j] for k in range(K)), Fraction(0))
            out[i * N + j] = _rne_fraction(s)
    return out


@pytest.mark.parametrize("seed", range(12))
def test_bruteforce_exact_small(oracle_lib, seed):
    rng = np.random.default_rng(1000 + seed)
    M, N, K = (int(x) for x in rng.integers(1, 9, 3))
    # magnitudes in [2^-8, 1] with random signs: every binary64 partial sum is
    # exact, so the oracle must equal the exact model bit for bit
    mag = 2.0 ** rng.uniform(-8, 0, M * K)
    a = f16(mag * rng.choice([-1.0, 1.0], M * K))
    mag = 2.0 ** rng.uniform(-8, 0, K * N)
    b = f16(mag * rng.choice([-1.0, 1.0], K * N))
    got = oracle_lib.gemm_relu(a, b, M, N, K)
    ref = _exact_gemm_relu(a, b, M, N, K)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("seed", range(6))
def test_bruteforce_exact_wide_range(oracle_lib, seed):
    # any finite fp16 inputs (subnormals included), scaled so sums stay finite
    rng = np.random.default_rng(2000 + seed)
    M, N, K = 5, 7, 6
    a = rng.integers(0, 0x7C00, M * K).astype(np.uint16) | (
        rng.integers(0, 2, M * K).astype(np.uint16) << 15)
    b = f16(rng.uniform(-1, 1, K * N) * 2.0 ** rng.integers(-20, 0, K * N))
    a = f16(np.clip(bits_to_f64(a), -4, 4))
    got = oracle_lib.gemm_relu(a, b, M, N, K)
    ref = _exact_gemm_relu(a, b, M, N, K)
    assert np.array_equal(got, ref)


def test_zero_iff_sum_at_most_half_min_subnormal(oracle_lib):
    # C_ij == 0 exactly when the exact sum is <= 2^-25 (ReLU, then the tie at
    # 2^-25 goes to the even neighbour 0)
    rng = np.random.default_rng(7)
    M, N, K = 6, 6, 4
    a = f16(rng.uniform(-1, 1, M * K) * 2.0 ** -12)
    b = f16(rng.uniform(-1, 1, K * N) * 2.0 ** -12)
    got = oracle_lib.gemm_relu(a, b, M, N, K)
    av, bv = bits_to_f64(a).reshape(M, K), bits_to_f64(b).reshape(K, N)
    for i in range(M):
        for j in range(N):
            s = sum(Fraction(float(av[i, k])) * Fraction(float(bv[k, j])) for k in range(K))
            assert (got[i * N + j] == 0) == (s <= Fraction(1, 2 ** 25))


# ------------------------------------------------------------------ fsum cross-check


def test_fsum_cross_check_mid_size(oracle_lib):
    M, N, K = 96, 80, 512
    a, b = wl.generate_dense(M, N, K, "uniform", 11)
    got, S, Sabs = oracle_lib.gemm_relu(a, b, M, N, K, want_sums=True)
    av = bits_to_f64(a).reshape(M, K)
    bv = bits_to_f64(b).reshape(K, N)
    exact = np.array([[math.fsum(av[i] * bv[:, j]) for j in range(N)] for i in range(M)])
    # binary64 recursive summation bound: |s - exact| <= (K-1) u sum|p|
    u = 2.0 ** -53
    assert np.all(np.abs(S[0] - exact) <= (K - 1) * u * Sabs[0] + 1e-300)
    ref = f16(np.where(exact > 0, exact, 0.0))
    mism = np.nonzero(got.reshape(M, N) != ref)
    # a mismatch is only allowed where the exact value sits within the
    # summation error of a rounding boundary; with these inputs there is none
    assert mism[0].size == 0


# ------------------------------------------------------------------- closed forms

ONE, MINUS_ONE = 0x3C00, 0xBC00


@pytest.mark.parametrize("K", [1, 7, 1000, 2048, 8192])
def test_ones_give_K(oracle_lib, K):
    M, N = 3, 5
    a = np.full(M * K, ONE, np.uint16)
    b = np.full(K * N, ONE, np.uint16)
    got = oracle_lib.gemm_relu(a, b, M, N, K)
    assert np.all(got == f16(float(K)))


def test_minus_ones_give_zero(oracle_lib):
    M, N, K = 4, 4, 33
    a = np.full(M * K, MINUS_ONE, np.uint16)
    b = np.full(K * N, ONE, np.uint16)
    assert np.all(oracle_lib.gemm_relu(a, b, M, N, K) == 0)


def _relu_bits(bits):
    v = bits_to_f64(bits)
    return np.where(v > 0, bits, 0).astype(np.uint16)


def test_identity_left_and_right(oracle_lib):
    rng = np.random.default_rng(3)
    n, N = 24, 17
    eye = f16(np.eye(n)).reshape(-1)
    b = f16(rng.uniform(-1, 1, n * N))
    assert np.array_equal(oracle_lib.gemm_relu(eye, b, n, N, n), _relu_bits(b))
    a = f16(rng.uniform(-1, 1, N * n))
    assert np.array_equal(oracle_lib.gemm_relu(a, eye, N, n, n), _relu_bits(a))


def test_permutation_permutes_rows(oracle_lib):
    rng = np.random.default_rng(4)
    n, N = 16, 9
    perm = rng.permutation(n)
    P = np.zeros((n, n))
    P[np.arange(n), perm] = 1.0
    b = f16(rng.uniform(-1, 1, n * N)).reshape(n, N)
    got = oracle_lib.gemm_relu(f16(P).reshape(-1), b.reshape(-1), n, N, n).reshape(n, N)
    assert np.array_equal(got, _relu_bits(b[perm]))


def test_integer_matrices_exact(oracle_lib):
    # entries in {-1,0,1}: every sum is an integer of magnitude <= K, exact in
    # fp16 for K <= 2048; compare with integer matmul
    M, N, K = 37, 29, 2048
    rng = np.random.default_rng(5)
    ai = rng.integers(-1, 2, (M, K))
    bi = rng.integers(-1, 2, (K, N))
    got = oracle_lib.gemm_relu(f16(ai).reshape(-1), f16(bi).reshape(-1), M, N, K)
    ref = np.maximum(ai @ bi, 0)
    assert np.array_equal(bits_to_f64(got).reshape(M, N), ref.astype(np.float64))


def test_scaling_by_two_is_exact(oracle_lib):
    M, N, K = 20, 24, 64
    a, b = wl.generate_dense(M, N, K, "uniform", 6)
    c1 = oracle_lib.gemm_relu(a, b, M, N, K)
    a2 = f16(bits_to_f64(a) * 2)
    c2 = oracle_lib.gemm_relu(a2, b, M, N, K)
    v1, v2 = bits_to_f64(c1), bits_to_f64(c2)
    normal = (v1 >= 2.0 ** -14) | (v1 == 0)
    assert np.array_equal(v2[normal], 2 * v1[normal])


def test_zero_row_gives_zero_row(oracle_lib):
    M, N, K = 8, 12, 40
    a, b = wl.generate_dense(M, N, K, "uniform", 8)
    a = a.reshape(M, K).copy()
    a[3] = 0
    got = oracle_lib.gemm_relu(a.reshape(-1), b, M, N, K).reshape(M, N)
    assert np.all(got[3] == 0)


def test_transpose_is_not_symmetric(oracle_lib):
    # C(A,B) must use B as (K,N) row-major: swapping in B^T changes the result
    M = N = K = 16
    a, b = wl.generate_dense(M, N, K, "uniform", 9)
    c = oracle_lib.gemm_relu(a, b, M, N, K)
    bt = b.reshape(K, N).T.copy().reshape(-1)
    ct = oracle_lib.gemm_relu(a, bt, M, N, K)
    assert not np.array_equal(c, ct)
    av, bv = bits_to_f64(a).reshape(M, K), bits_to_f64(b).reshape(K, N)
    ref = f16(np.maximum(av @ bv, 0)).reshape(-1)       # fp64 BLAS, then RNE
    assert np.mean(c == ref) > 0.99


# ------------------------------------------------------------------- probes (golden)


def test_golden_probes(oracle_lib):
    with open(os.path.join(GOLDEN, "probes.json")) as f:
        probes = json.load(f)["probes"]
    for p in probes:
        M, N, K = p["M"], p["N"], p["K"]
        a = f16(np.array(p["A"], dtype=np.float64)).reshape(-1)
        b = f16(np.array(p["B"], dtype=np.float64)).reshape(-1)
        got = oracle_lib.gemm_relu(a, b, M, N, K)
        assert [int(x) for x in got] == [int(x, 16) for x in p["C_bits"]], p["name"]


# ------------------------------------------------------------------- layouts, batch


def test_padding_and_ld_do_not_leak(oracle_lib):
    M, N, K = 13, 11, 19
    lda, ldb, ldc = 24, 16, 20
    a, b = wl.generate_dense(M, N, K, "uniform", 10)
    dense = oracle_lib.gemm_relu(a, b, M, N, K)
    ap = wl.pad_rows(a, M, K, lda)          # NaN in the pad columns
    bp = wl.pad_rows(b, K, N, ldb)
    C = np.full(M * ldc + 40, 0x7E00, np.uint16)
    oracle_lib.gemm_relu(ap, bp, M, N, K, lda, ldb, ldc, C=C)
    C2 = C[: M * ldc].reshape(M, ldc)
    assert np.array_equal(C2[:, :N].reshape(-1), dense)
    assert np.all(C2[:, N:] == 0x7E00) and np.all(C[M * ldc:] == 0x7E00)


def test_batched_slices_match_single(oracle_lib):
    M, N, K, B = 9, 10, 11, 5
    a, b = wl.generate_dense(M, N, K, "uniform", 12, batch=B)
    c = oracle_lib.gemm_relu(a, b, M, N, K, batch=B).reshape(B, M * N)
    for i in range(B):
        ci = oracle_lib.gemm_relu(a[i * M * K:(i + 1) * M * K], b[i * K * N:(i + 1) * K * N],
                                  M, N, K)
        assert np.array_equal(c[i], ci)
    # broadcast B (batch stride 0)
    c0 = oracle_lib.gemm_relu(a, b[:K * N], M, N, K, batch=B, sB=0).reshape(B, M * N)
    for i in range(B):
        assert np.array_equal(c0[i], oracle_lib.gemm_relu(a[i * M * K:(i + 1) * M * K],
                                                          b[:K * N], M, N, K))


def test_empty_and_k0(oracle_lib):
    a = np.zeros(0, np.uint16)
    assert oracle_lib.gemm_relu(a, a, 0, 5, 3).size == 0
    c = oracle_lib.gemm_relu(a, a, 3, 4, 0)
    assert c.size == 12 and np.all(c == 0)


def test_threads_do_not_change_result(oracle_lib):
    M, N, K = 33, 21, 70
    a, b = wl.generate_dense(M, N, K, "normal_invsqrtk", 13)
    c1 = oracle_lib.gemm_relu(a, b, M, N, K, threads=1)
    c8 = oracle_lib.gemm_relu(a, b, M, N, K, threads=8)
    assert np.array_equal(c1, c8)


def test_sampled_matches_full(oracle_lib):
    w = wl.Workload("t", 70, 90, 130, "uniform", 14, batch=3)
    a, b = wl.generate(w)
    full, S, Sa = oracle_lib.gemm_relu(a, b, w.M, w.N, w.K, batch=3, want_sums=True)
    idx = wl.sample_positions(w, 200)
    got, s, sa = oracle_lib.gemm_relu_sampled(a, b, w.K, w.lda_, w.ldb_, idx, w.sA, w.sB)
    full = full.reshape(3, w.M, w.N)
    for q, (bb, i, j) in enumerate(idx):
        assert got[q] == full[bb, i, j]
        assert s[q] == S[bb, i, j] and sa[q] == Sa[bb, i, j]


def test_small_workload_output_hash(oracle_lib):
    with open(os.path.join(GOLDEN, "oracle_outputs_sha256.json")) as f:
        want = json.load(f)
    w = wl.WORKLOADS["small_512"]
    a, b = wl.generate(w)
    c = oracle_lib.gemm_relu(a, b, w.M, w.N, w.K)
    assert wl.sha256_of(c) == want["small_512"]
