"""Pins for the oracle's weight-only int4 GEMM (W_INT4 / A_FP16).

  * nibble decoding against numpy integer arithmetic on every byte value,
  * with power-of-two scales every dequantized weight s * q is an exact fp16
    value, so the int4 oracle must equal the dense oracle (already pinned) on
    the dequantized (N,K) weight bit for bit: this fixes the row, group and
    nibble indexing and the sign of q,
  * an exact Fraction model with arbitrary scales on tiny shapes,
  * closed forms: q = 1 everywhere gives s-weighted row sums.
A swapped nibble order, a group index off by one, an unsigned nibble or a
transposed weight each fails one of them.
"""

from fractions import Fraction

import numpy as np
import pytest

import workloads as wl


def f16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def f16v(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def pack(q):
    """(N, K) ints in -8..7 -> (N, K/2) bytes, even k in the low nibble."""
    u = (np.asarray(q) & 15).astype(np.uint8)
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


def test_nibble_decoding_every_byte(oracle_lib):
    b = np.arange(256, dtype=np.uint8)
    lo, hi = oracle_lib.s4_decode(b)
    ref_lo = ((b.astype(np.int16) & 15) ^ 8) - 8
    ref_hi = ((b.astype(np.int16) >> 4) ^ 8) - 8
    assert np.array_equal(lo, ref_lo) and np.array_equal(hi, ref_hi)


@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("act", ["none", "relu"])
def test_power_of_two_scales_match_the_dense_oracle(oracle_lib, G, act):
    rng = np.random.default_rng(G)
    M, N, K = 7, 40, 256
    q = rng.integers(-8, 8, (N, K))
    e = rng.integers(-12, -4, (N, K // G))
    s = 2.0 ** e                                   # fp16-exact, and so is s * q
    a = f16(rng.uniform(-1, 1, M * K))
    bias = f16(rng.uniform(-0.1, 0.1, N))
    wdeq = (np.repeat(s, G, axis=1) * q)           # (N, K), exact in fp16
    w16 = f16(wdeq)
    assert np.array_equal(f16v(w16).reshape(N, K), wdeq)
    ref = oracle_lib.gemm_ex(a, w16, M, N, K, bias=bias, b_layout="nk", act=act)
    got = oracle_lib.gemm_w4(a, pack(q), f16(s), M, N, K, G, bias=bias, act=act)
    assert np.array_equal(got, ref)


def _exact_w4(a, q, s, bias, M, N, K, G, act):
    av = [Fraction(float(x)) for x in f16v(a)]
    sv = [[Fraction(float(x)) for x in row] for row in f16v(s).reshape(N, K // G)]
    bv = [Fraction(float(x)) for x in f16v(bias)] if bias is not None else None
    out = np.zeros(M * N, np.uint16)
    vals = f16v(np.arange(0x7C00, dtype=np.uint16))
    for i in range(M):
        for n in range(N):
            t = sum((av[i * K + k] * sv[n][k // G] * int(q[n, k]) for k in range(K)), Fraction(0))
            if bv is not None:
                t += bv[n]
            if act == "relu" and t <= 0:
                t = Fraction(0)
            # exact round-half-even to fp16 by neighbour search
            sign = 0x8000 if t < 0 else 0
            x = abs(t)
            k = int(np.searchsorted(vals, float(x), side="right")) - 1
            k = max(k, 0)
            while k + 1 < len(vals) and Fraction(float(vals[k + 1])) <= x:
                k += 1
            while k > 0 and Fraction(float(vals[k])) > x:
                k -= 1
            if k + 1 < len(vals):
                dl = x - Fraction(float(vals[k]))
                dh = Fraction(float(vals[k + 1])) - x
                if dh < dl or (dh == dl and k % 2 == 1):
                    k += 1
            out[i * N + n] = (sign | k) if t != 0 else 0
    return out


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("act", ["none", "relu"])
def test_bruteforce_exact_any_scales(oracle_lib, seed, act):
    rng = np.random.default_rng(500 + seed)
    M, N, K, G = 3, 5, 64, 32
    q = rng.integers(-8, 8, (N, K))
    # scales and A in [2^-6, 1]: every product and partial sum is exact in
    # binary64, so the oracle must equal the exact model
    s = f16(2.0 ** rng.uniform(-6, 0, N * (K // G)))
    a = f16(2.0 ** rng.uniform(-6, 0, M * K) * rng.choice([-1.0, 1.0], M * K))
    bias = f16(rng.uniform(-1, 1, N)) if seed % 2 else None
    got = oracle_lib.gemm_w4(a, pack(q), s, M, N, K, G, bias=bias, act=act)
    ref = _exact_w4(a, q, s, bias, M, N, K, G, act)
    assert np.array_equal(got, ref)


def test_unit_weights_give_scaled_row_sums(oracle_lib):
    M, N, K, G = 4, 16, 256, 64
    q = np.ones((N, K), int)
    s = f16(np.tile([0.5, 0.25, 0.125, 1.0], N))     # per (n, group)
    a = f16(np.tile(np.arange(K) % 3 - 1.0, M))        # -1, 0, 1, ...
    got = f16v(oracle_lib.gemm_w4(a, pack(q), s, M, N, K, G, act="none")).reshape(M, N)
    av = f16v(a).reshape(M, K)
    sv = f16v(s).reshape(N, K // G)
    want = np.array([[sum(sv[n, g] * av[i, g * G:(g + 1) * G].sum() for g in range(K // G))
                      for n in range(N)] for i in range(M)])
    assert np.array_equal(got, want)


def test_padded_rows_and_nan_padding_do_not_leak(oracle_lib):
    rng = np.random.default_rng(9)
    M, N, K, G = 5, 24, 128, 64
    q = rng.integers(-8, 8, (N, K))
    wq = pack(q)
    s = f16(rng.uniform(0.01, 0.02, N * (K // G)))
    a = f16(rng.uniform(-1, 1, M * K))
    ref = oracle_lib.gemm_w4(a, wq, s, M, N, K, G)
    ldw, lds, lda = K // 2 + 16, K // G + 3, K + 8
    wq_p = np.full((N, ldw), 0x88, np.uint8)
    wq_p[:, :K // 2] = wq
    s_p = np.full((N, lds), 0x7E00, np.uint16)
    s_p[:, :K // G] = s.reshape(N, K // G)
    a_p = wl.pad_rows(a, M, K, lda)
    got = oracle_lib.gemm_w4(a_p, wq_p, s_p, M, N, K, G, lda=lda, ldw=ldw, lds=lds)
    assert np.array_equal(got, ref)


def test_generator_shapes_and_range(oracle_lib):
    wq, s = wl.generate_w4(64, 512, 128, 3)
    assert wq.dtype == np.uint8 and wq.size == 64 * 256 and s.size == 64 * 4
    lo, hi = oracle_lib.s4_decode(wq)
    assert lo.min() >= -8 and hi.max() <= 7 and set(np.unique(lo)) == set(range(-8, 8))
