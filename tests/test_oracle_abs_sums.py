"""Pins for the oracle's second output: S_ij = sum_k |A_ik * B_kj| (+ |bias_j|).

This sum sets the per-element error bound of the G2 gate (the fp32
recursive-summation bound, "tilelang practitioner's notes" section 3.2 on fp32
accumulation and section 5.3 on checking numerics against a reference), so an
inflated value would loosen G2 silently.  Here it is compared with an
independent computation: numpy decodes the operands (np.float16 views, bf16 by
shifting into binary32) and forms |A| @ |B| in float64 with its own BLAS
product, no code shared with the oracle.  Both sides sum exact binary64
products of non-negative terms, so they agree to a few float64 ulps whatever
the summation order.  Covered: fp16 and bf16, (K,N) and (N,K) B, with and
without bias, strided batches with padded leading dimensions, the sampled
entry points and the int4-weight GEMM (weights dequantized by numpy integer
arithmetic).  The last tests plant the plausible mistakes (a stray factor 2,
an accumulator not reset between outputs, the bias term dropped) in the
oracle's output and check that the comparison rejects each.
"""

import numpy as np
import pytest

import workloads as wl
from parity import gate

RTOL = 1e-12   # far above float64 order effects (K <= 4096: < 1e-12), far below any slip


def f16v(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def bf16v(bits):
    u = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def vals(bits, dtype):
    return bf16v(bits) if dtype == "bf16" else f16v(bits)


def abs_sums_numpy(a, b, M, N, K, dtype="f16", b_layout="kn", bias=None, lda=None, ldb=None,
                   batch=1, sA=None, sB=None):
    """|A| @ |B| (+ |bias|) per batch in float64, shaped (batch, M, N)."""
    lda = K if lda is None else lda
    ldb = (N if b_layout == "kn" else K) if ldb is None else ldb
    sA = M * lda if sA is None else sA
    sB = (K * ldb if b_layout == "kn" else N * ldb) if sB is None else sB
    av, bv = vals(a, dtype), vals(b, dtype)
    out = np.empty((batch, M, N))
    for t in range(batch):
        A = av[t * sA:t * sA + M * lda].reshape(M, lda)[:, :K]
        if b_layout == "kn":
            B = bv[t * sB:t * sB + K * ldb].reshape(K, ldb)[:, :N]
        else:
            B = bv[t * sB:t * sB + N * ldb].reshape(N, ldb)[:, :K].T
        out[t] = np.abs(A) @ np.abs(B)
        if bias is not None:
            out[t] += np.abs(vals(bias, dtype)[:N])[None, :]
    return out


def assert_abs_sums(got, ref):
    got = np.asarray(got, np.float64).reshape(-1)
    ref = np.asarray(ref, np.float64).reshape(-1)
    assert got.shape == ref.shape
    assert np.all(np.abs(got - ref) <= RTOL * ref + 1e-300), \
        f"max rel diff {np.max(np.abs(got - ref) / np.maximum(ref, 1e-300)):.3g}"


@pytest.mark.parametrize("dist", ["uniform", "normal_invsqrtk", "int3"])
def test_gemm_relu_abs_sums(oracle_lib, dist):
    M, N, K = 37, 45, 300
    a, b = wl.generate_dense(M, N, K, dist, 41)
    _, _, Sa = oracle_lib.gemm_relu(a, b, M, N, K, want_sums=True)
    assert_abs_sums(Sa, abs_sums_numpy(a, b, M, N, K))


def test_gemm_relu_abs_sums_batched_padded(oracle_lib):
    M, N, K, bt = 19, 23, 77, 3
    lda, ldb = K + 5, N + 3
    a, b = wl.generate_dense(M, N, K, "uniform", 42, batch=bt)
    a = wl.pad_rows(a, M, K, lda, bt, fill=0x3C00)   # pads hold 1.0: must not be summed
    b = wl.pad_rows(b, K, N, ldb, bt, fill=0x3C00)
    sA, sB = M * lda, K * ldb
    _, _, Sa = oracle_lib.gemm_relu(a, b, M, N, K, lda, ldb, N, bt, sA, sB, M * N,
                                    want_sums=True)
    ref = abs_sums_numpy(a, b, M, N, K, lda=lda, ldb=ldb, batch=bt, sA=sA, sB=sB)
    assert_abs_sums(Sa, ref)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("b_layout", ["kn", "nk"])
@pytest.mark.parametrize("with_bias", [False, True])
@pytest.mark.parametrize("act", ["none", "relu"])
def test_gemm_ex_abs_sums(oracle_lib, dtype, b_layout, with_bias, act):
    M, N, K, bt = 21, 34, 136, 2
    a, b = wl.generate_dense(M, N, K, "uniform", 43, batch=bt, dtype=dtype)
    if b_layout == "nk":
        b = wl.transpose_bits(b, K, N, bt)
    bias = wl.generate_bias(N, 43, dtype) if with_bias else None
    _, _, Sa = oracle_lib.gemm_ex(a, b, M, N, K, batch=bt, bias=bias, dtype=dtype,
                                  b_layout=b_layout, act=act, want_sums=True)
    ref = abs_sums_numpy(a, b, M, N, K, dtype, b_layout, bias, batch=bt)
    assert_abs_sums(Sa, ref)


def test_sampled_abs_sums(oracle_lib):
    w = wl.Workload("t", 150, 130, 260, "uniform", 44, batch=2)
    a, b = wl.generate(w)
    idx = wl.sample_positions(w, 300)
    _, _, sa = oracle_lib.gemm_relu_sampled(a, b, w.K, w.lda_, w.ldb_, idx, w.sA, w.sB)
    ref = abs_sums_numpy(a, b, w.M, w.N, w.K, batch=2)
    assert_abs_sums(sa, ref[idx[:, 0], idx[:, 1], idx[:, 2]])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("b_layout", ["kn", "nk"])
def test_sampled_ex_abs_sums(oracle_lib, dtype, b_layout):
    M, N, K = 90, 70, 200
    a, b = wl.generate_dense(M, N, K, "uniform", 45, dtype=dtype)
    if b_layout == "nk":
        b = wl.transpose_bits(b, K, N)
    bias = wl.generate_bias(N, 45, dtype)
    w = wl.Workload("t", M, N, K, "uniform", 45)
    idx = wl.sample_positions(w, 200)
    ldb = N if b_layout == "kn" else K
    _, _, sa = oracle_lib.gemm_ex_sampled(a, b, K, K, ldb, idx, bias=bias, dtype=dtype,
                                          b_layout=b_layout)
    ref = abs_sums_numpy(a, b, M, N, K, dtype, b_layout, bias)
    assert_abs_sums(sa, ref[0, idx[:, 1], idx[:, 2]])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("with_bias", [False, True])
def test_gemm_w4_abs_sums(oracle_lib, dtype, with_bias):
    M, N, K, G = 9, 40, 256, 64
    a, _ = wl.generate_dense(M, 8, K, "uniform", 46, dtype=dtype)
    wq, s = wl.generate_w4(N, K, G, 46, dtype)
    bias = wl.generate_bias(N, 46, dtype) if with_bias else None
    _, _, Sa = oracle_lib.gemm_w4(a, wq, s, M, N, K, G, bias=bias, dtype=dtype, want_sums=True)
    # dequantize with numpy integer arithmetic: low nibble = even k, two's complement
    byt = wq.reshape(N, K // 2).astype(np.int16)
    q = np.empty((N, K), np.int16)
    q[:, 0::2] = ((byt & 15) ^ 8) - 8
    q[:, 1::2] = ((byt >> 4) ^ 8) - 8
    wdeq = np.repeat(vals(s, dtype).reshape(N, K // G), G, axis=1) * q   # (N, K)
    ref = np.abs(vals(a, dtype).reshape(M, K)) @ np.abs(wdeq).T
    if bias is not None:
        ref += np.abs(vals(bias, dtype))[None, :]
    assert_abs_sums(Sa, ref)


# ---------------------------------------------------- the check catches slips


def _sums(oracle_lib):
    M, N, K = 24, 32, 200
    a, b = wl.generate_dense(M, N, K, "uniform", 47)
    bias = wl.generate_bias(N, 47)
    _, _, Sa = oracle_lib.gemm_ex(a, b, M, N, K, bias=bias, want_sums=True)
    return Sa, abs_sums_numpy(a, b, M, N, K, bias=bias), (M, N, K, a, b, bias)


def test_check_rejects_doubled_sums(oracle_lib):
    Sa, ref, _ = _sums(oracle_lib)
    assert_abs_sums(Sa, ref)
    with pytest.raises(AssertionError):
        assert_abs_sums(2.0 * Sa, ref)


def test_check_rejects_accumulator_not_reset(oracle_lib):
    Sa, ref, _ = _sums(oracle_lib)
    carried = np.cumsum(Sa.reshape(-1))      # each output adds the previous ones
    with pytest.raises(AssertionError):
        assert_abs_sums(carried, ref)


def test_check_rejects_dropped_bias_or_last_k(oracle_lib):
    Sa, ref, (M, N, K, a, b, bias) = _sums(oracle_lib)
    with pytest.raises(AssertionError):
        assert_abs_sums(Sa - np.abs(f16v(bias))[None, None, :], ref)
    last = np.abs(f16v(a).reshape(M, K)[:, -1:]) @ np.abs(f16v(b).reshape(K, N)[-1:, :])
    with pytest.raises(AssertionError):
        assert_abs_sums(Sa - last[None], ref)


def test_g2_alone_catches_one_dropped_chunk():
    """One 64-wide K tile dropped from a single output at the skinny
    workload's shape and scale (what a pipeline stage read before it landed
    would do) stays under the contract tolerance and under G1 over the whole
    output, but exceeds that element's G2 bound: G2 is the gate that sees it,
    which is why its input sum is pinned above."""
    rng = np.random.default_rng(48)
    M, N, K = 16, 16384, 8192
    a = (rng.uniform(-1, 1, (M, K)) / np.sqrt(K)).astype(np.float16).astype(np.float64)
    b = (rng.uniform(-1, 1, (K, N)) / np.sqrt(K)).astype(np.float16).astype(np.float64)
    s = a @ b
    sa = np.abs(a) @ np.abs(b)
    ref = np.maximum(s, 0).astype(np.float16).view(np.uint16).reshape(-1)
    part = a[:, 64:128] @ b[64:128, :]
    bound = 2.0 * K * 2.0 ** -24 * sa
    # a positive output whose dropped tile is about twice its G2 bound
    score = np.where((s > 0) & (s - part > 0), np.abs(np.abs(part) - 2.0 * bound), np.inf)
    i, j = np.unravel_index(np.argmin(score), s.shape)
    bad_s = s.copy()
    bad_s[i, j] -= part[i, j]
    bad = np.maximum(bad_s, 0).astype(np.float16).view(np.uint16).reshape(-1)
    rep = gate(bad, ref, K, sa)
    assert rep.contract_fail == 0 and rep.g1 <= 1e-3, str(rep)
    assert rep.g2_fail == 1, str(rep)
    # with the bound's sum inflated fourfold the same slip would pass every gate
    assert gate(bad, ref, K, 4.0 * sa).ok
