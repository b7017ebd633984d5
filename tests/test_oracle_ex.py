"""Pins for the oracle's variants: bf16 storage, B stored as (N,K), a
per-column bias, and no activation.

Each is pinned against something other than the oracle:
  * the bf16 codec against numpy's float32 view (decode, exhaustive), torch's
    float32 -> bfloat16 conversion (encode, values exactly representable in
    float32) and an exact rational round-half-even (encode, arbitrary binary64
    values, midpoints and their neighbours),
  * the (N,K) layout against the (K,N) layout on the transposed array,
  * bias and activation against an exact Fraction model on tiny shapes and
    closed forms (A = 0 gives act(bias); ones give K + bias; -ones keep their
    sign without the ReLU).
A bias read at the row instead of the column, a dropped bias, a ReLU applied
when it should not be, a transposed B or a bf16 rounding slip each fails one.
"""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch


def f16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def bf16_bits_to_f64(b):
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def bf16_of_float32(x32):
    """torch's float32 -> bfloat16 conversion (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------- exact rounding


def rne_bf16(r: Fraction) -> int:
    """Exact round-half-even of a rational to bf16 bits (sign kept)."""
    if r == 0:
        return 0
    sign = 0x8000 if r < 0 else 0
    a = abs(r)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e <= a:        # make 2^(e-1) <= a < 2^e
        e += 1
    while Fraction(2) ** (e - 1) > a:
        e -= 1
    qe = max(e - 8, -133)               # quantum of the binade (or subnormals)
    scaled = a / Fraction(2) ** qe
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    value = Fraction(n) * Fraction(2) ** qe
    if value >= Fraction(2) ** 128:
        return sign | 0x7F80
    bits = int(np.float32(float(value)).view(np.uint32)) >> 16   # exact: value is a bf16
    return sign | (bits & 0x7FFF)


_F16_ALL = np.arange(0x7C00, dtype=np.uint16)
_F16_POS = [Fraction(float(v)) for v in _F16_ALL.view(np.float16).astype(np.float64)]


def rne_f16(r: Fraction) -> int:
    """Exact round-half-even of a rational to fp16 bits (sign kept)."""
    if r == 0:
        return 0
    sign = 0x8000 if r < 0 else 0
    a = abs(r)
    if a >= 65520:
        return sign | 0x7C00
    lo, hi = 0, len(_F16_POS) - 1
    while lo < hi:                      # largest k with value_k <= a
        mid = (lo + hi + 1) // 2
        if _F16_POS[mid] <= a:
            lo = mid
        else:
            hi = mid - 1
    k = lo
    if k == len(_F16_POS) - 1:
        return sign | k
    dl, dh = a - _F16_POS[k], _F16_POS[k + 1] - a
    if dh < dl or (dh == dl and k % 2 == 1):
        k += 1
    return sign | k


# ------------------------------------------------------------------ bf16 codec


def test_decbf16_exhaustive(oracle_lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle_lib.decbf16(bits)
    ref = bf16_bits_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def test_encbf16_round_trips_every_finite_value(oracle_lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = (bits & 0x7F80) != 0x7F80
    v = bf16_bits_to_f64(bits[finite])
    assert np.array_equal(oracle_lib.encbf16(v), bits[finite])


def test_encbf16_matches_torch_on_float32_values(oracle_lib):
    rng = np.random.default_rng(77)
    u = rng.integers(0, 2 ** 32, 400000, dtype=np.uint64).astype(np.uint32)
    x32 = u.view(np.float32)
    x32 = x32[np.isfinite(x32)]
    # every float32 subnormal and tie pattern near the bottom too
    tiny = (np.arange(0, 1 << 16, dtype=np.uint32)).view(np.float32)
    x32 = np.concatenate([x32, tiny, -tiny])
    got = oracle_lib.encbf16(x32.astype(np.float64))
    ref = bf16_of_float32(x32)
    assert np.array_equal(got, ref)


def test_encbf16_matches_exact_rounding_on_binary64_values(oracle_lib):
    rng = np.random.default_rng(78)
    x = rng.uniform(1, 2, 3000) * 2.0 ** rng.integers(-140, 129, 3000)
    x *= rng.choice([-1.0, 1.0], x.size)
    # midpoints between neighbouring bf16 values and one binary64 ulp either side
    b = rng.integers(0, 0x7F7F, 2000).astype(np.uint16)
    lo = bf16_bits_to_f64(b)
    hi = bf16_bits_to_f64(b + 1)
    mid = (lo + hi) / 2
    x = np.concatenate([x, mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf)])
    got = oracle_lib.encbf16(x)
    ref = np.array([rne_bf16(Fraction(float(v))) for v in x], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_encbf16_special_points(oracle_lib):
    maxf = bf16_bits_to_f64(np.array([0x7F7F], np.uint16))[0]
    over_mid = maxf + 2.0 ** (127 - 8)            # midpoint to 2^128: ties to inf
    cases = [
        (0.0, 0x0000), (-0.0, 0x8000), (1.0, 0x3F80), (-2.0, 0xC000),
        (1 + 2.0 ** -8, 0x3F80),                  # tie: even neighbour 1.0
        (1 + 3 * 2.0 ** -8, 0x3F82),              # tie: even neighbour 1 + 2^-6
        (2.0 ** -133, 0x0001), (2.0 ** -134, 0x0000), (3 * 2.0 ** -134, 0x0002),
        (2.0 ** -126, 0x0080), (maxf, 0x7F7F), (over_mid, 0x7F80),
        (np.nextafter(over_mid, 0), 0x7F7F), (np.inf, 0x7F80), (1e300, 0x7F80),
        (-1e300, 0xFF80),
    ]
    got = oracle_lib.encbf16(np.array([c[0] for c in cases]))
    assert [int(g) for g in got] == [c[1] for c in cases]


# ------------------------------------------------------------- (N,K) B layout


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_nk_layout_is_the_transposed_kn(oracle_lib, dtype):
    rng = np.random.default_rng(5)
    M, N, K = 13, 17, 29
    a = rng.integers(0, 0x3C00, M * K).astype(np.uint16)          # finite, |x| < 1-ish
    b = rng.integers(0, 0x3C00, K * N).astype(np.uint16)
    if dtype == "bf16":
        a = (a >> 3) + 0x3000
        b = (b >> 3) + 0x3000
    a |= (rng.integers(0, 2, M * K).astype(np.uint16) << 15)
    b |= (rng.integers(0, 2, K * N).astype(np.uint16) << 15)
    ref = oracle_lib.gemm_ex(a, b, M, N, K, dtype=dtype, b_layout="kn", act="none")
    ldb = K + 3
    bt = np.full(N * ldb, 0x7E00, np.uint16)                      # NaN in the padding
    bt.reshape(N, ldb)[:, :K] = b.reshape(K, N).T
    got = oracle_lib.gemm_ex(a, bt, M, N, K, ldb=ldb, dtype=dtype, b_layout="nk", act="none")
    assert np.array_equal(got, ref)


# ---------------------------------------------------- bias, activation: exact


def _exact_ex(a, b, bias, M, N, K, dtype, act):
    dec = bf16_bits_to_f64 if dtype == "bf16" else (
        lambda x: np.asarray(x, np.uint16).view(np.float16).astype(np.float64))
    rne = rne_bf16 if dtype == "bf16" else rne_f16
    av = [Fraction(float(x)) for x in dec(a)]
    bv = [Fraction(float(x)) for x in dec(b)]
    cv = [Fraction(float(x)) for x in dec(bias)] if bias is not None else None
    out = np.zeros(M * N, dtype=np.uint16)
    for i in range(M):
        for j in range(N):
            s = sum((av[i * K + k] * bv[k * N + j] for k in range(K)), Fraction(0))
            if cv is not None:
                s += cv[j]
            if act == "relu" and s <= 0:
                s = Fraction(0)
            out[i * N + j] = rne(s)
    return out


def _small_operands(rng, n, dtype):
    """Values with magnitudes in [2^-8, 1] and random signs: every binary64
    partial sum of a few products is exact."""
    v = 2.0 ** rng.uniform(-8, 0, n) * rng.choice([-1.0, 1.0], n)
    if dtype == "bf16":
        return bf16_of_float32(v.astype(np.float32))
    return f16(v)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("act", ["none", "relu"])
@pytest.mark.parametrize("with_bias", [False, True])
@pytest.mark.parametrize("seed", range(3))
def test_bruteforce_exact_ex(oracle_lib, dtype, act, with_bias, seed):
    rng = np.random.default_rng(3000 + seed)
    M, N, K = (int(x) for x in rng.integers(1, 8, 3))
    N += 1                                   # M != N most of the time: bias[i] vs bias[j]
    a = _small_operands(rng, M * K, dtype)
    b = _small_operands(rng, K * N, dtype)
    bias = _small_operands(rng, N, dtype) if with_bias else None
    got = oracle_lib.gemm_ex(a, b, M, N, K, bias=bias, dtype=dtype, act=act)
    ref = _exact_ex(a, b, bias, M, N, K, dtype, act)
    assert np.array_equal(got, ref)
    if act == "none" and not with_bias:
        # without the ReLU some outputs are negative
        assert np.any(ref & 0x8000) or M * N < 4


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("act", ["none", "relu"])
def test_zero_a_gives_activation_of_bias(oracle_lib, dtype, act):
    M, N, K = 5, 24, 16
    vals = np.linspace(-3, 3, N)
    bias = bf16_of_float32(vals.astype(np.float32)) if dtype == "bf16" else f16(vals)
    a = np.zeros(M * K, np.uint16)
    rng = np.random.default_rng(1)
    b = _small_operands(rng, K * N, dtype)
    got = oracle_lib.gemm_ex(a, b, M, N, K, bias=bias, dtype=dtype, act=act).reshape(M, N)
    want = bias.copy()
    if act == "relu":
        want[(want & 0x8000) != 0] = 0
    want[want == 0x8000] = 0                 # 0 + (-0) is +0
    assert np.array_equal(got, np.tile(want, (M, 1)))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_ones_plus_integer_bias(oracle_lib, dtype):
    M, N, K = 3, 8, 100
    one = 0x3F80 if dtype == "bf16" else 0x3C00
    a = np.full(M * K, one, np.uint16)
    b = np.full(K * N, one, np.uint16)
    vals = np.arange(N, dtype=np.float64) - 150.0            # K + bias from -50 to -43 ..
    bias = bf16_of_float32(vals.astype(np.float32)) if dtype == "bf16" else f16(vals)
    for act in ("none", "relu"):
        got = oracle_lib.gemm_ex(a, b, M, N, K, bias=bias, dtype=dtype, act=act)
        exact = K + vals
        if act == "relu":
            exact = np.maximum(exact, 0)
        want = bf16_of_float32(exact.astype(np.float32)) if dtype == "bf16" else f16(exact)
        want[want == 0x8000] = 0
        assert np.array_equal(got.reshape(M, N), np.tile(want, (M, 1)))


def test_minus_ones_keep_their_sign_without_relu(oracle_lib):
    M, N, K = 4, 6, 10
    a = np.full(M * K, 0xBC00, np.uint16)                    # -1
    b = np.full(K * N, 0x3C00, np.uint16)                    # +1
    assert np.all(oracle_lib.gemm_ex(a, b, M, N, K, act="none") == f16(-10.0))
    assert np.all(oracle_lib.gemm_ex(a, b, M, N, K, act="relu") == 0)


def test_zero_bias_is_the_plain_relu(oracle_lib):
    rng = np.random.default_rng(11)
    M, N, K = 37, 40, 72
    a = _small_operands(rng, M * K, "f16")
    b = _small_operands(rng, K * N, "f16")
    ref = oracle_lib.gemm_relu(a, b, M, N, K)
    got = oracle_lib.gemm_ex(a, b, M, N, K, bias=np.zeros(N, np.uint16), act="relu")
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("dtype,layout,act", [("f16", "nk", "none"), ("bf16", "kn", "relu"),
                                              ("bf16", "nk", "none")])
def test_sampled_ex_matches_full_ex(oracle_lib, dtype, layout, act):
    rng = np.random.default_rng(12)
    M, N, K, batch = 9, 24, 40, 2
    lda, ldb, ldc = K + 2, (N + 3 if layout == "kn" else K + 5), N + 1
    rows_b = K if layout == "kn" else N
    sA, sB, sC = M * lda + 4, rows_b * ldb + 2, M * ldc + 3
    a = _small_operands(rng, (batch - 1) * sA + M * lda, dtype)
    b = _small_operands(rng, (batch - 1) * sB + rows_b * ldb, dtype)
    bias = _small_operands(rng, N, dtype)
    full, S, Sa = oracle_lib.gemm_ex(a, b, M, N, K, lda, ldb, ldc, batch, sA, sB, sC,
                                     bias=bias, dtype=dtype, b_layout=layout, act=act,
                                     want_sums=True)
    idx = np.array([(bb, i, j) for bb in range(batch) for i in range(0, M, 2)
                    for j in range(0, N, 3)])
    out, s, sa = oracle_lib.gemm_ex_sampled(a, b, K, lda, ldb, idx, sA, sB, bias=bias,
                                            dtype=dtype, b_layout=layout, act=act)
    want = np.array([full[bb * sC + i * ldc + j] for bb, i, j in idx], dtype=np.uint16)
    assert np.array_equal(out, want)
    assert np.array_equal(s, np.array([S[bb, i, j] for bb, i, j in idx]))
    assert np.array_equal(sa, np.array([Sa[bb, i, j] for bb, i, j in idx]))


def test_bad_modes_are_rejected(oracle_lib):
    a = np.zeros(4, np.uint16)
    with pytest.raises(KeyError):
        oracle_lib.gemm_ex(a, a, 2, 2, 2, dtype="f32")
    with pytest.raises(KeyError):
        oracle_lib.gemm_ex(a, a, 2, 2, 2, act="gelu")


def test_fsum_cross_check_bf16_with_bias(oracle_lib):
    # mid-size bf16 problem: every output against a correctly rounded sum
    rng = np.random.default_rng(13)
    M, N, K = 24, 20, 700
    a = bf16_of_float32(rng.uniform(-1, 1, M * K).astype(np.float32))
    b = bf16_of_float32(rng.uniform(-1, 1, K * N).astype(np.float32))
    bias = bf16_of_float32(rng.uniform(-4, 4, N).astype(np.float32))
    got = oracle_lib.gemm_ex(a, b, M, N, K, bias=bias, dtype="bf16", act="none")
    av = bf16_bits_to_f64(a).reshape(M, K)
    bv = bf16_bits_to_f64(b).reshape(K, N)
    cv = bf16_bits_to_f64(bias)
    mism = 0
    for i in range(M):
        for j in range(N):
            s = math.fsum(list(av[i] * bv[:, j]) + [cv[j]])
            mism += int(got[i * N + j]) != rne_bf16(Fraction(s))
    # the binary64 sum differs from the correctly rounded one by far less than
    # a bf16 rounding boundary is likely to be crossed: allow none
    assert mism == 0
