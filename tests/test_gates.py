"""The parity gates themselves, on the CPU: correct results pass and planted
mistakes (made in the oracle's output on the CPU) fail."""

import numpy as np

import workloads as wl
from parity import gate


def _case(oracle_lib, M=64, N=48, K=256, dist="uniform", seed=21):
    a, b = wl.generate_dense(M, N, K, dist, seed)
    c, S, Sa = oracle_lib.gemm_relu(a, b, M, N, K, want_sums=True)
    return a, b, c, S, Sa


def test_identical_passes(oracle_lib):
    _, _, c, _, Sa = _case(oracle_lib)
    rep = gate(c, c, 256, Sa)
    assert rep.ok and rep.bit_exact_frac == 1.0


def test_fp32_rounded_result_passes(oracle_lib):
    # an fp32-accumulated result (what the kernels compute) passes every gate
    M, N, K = 64, 48, 256
    a, b, c, S, Sa = _case(oracle_lib, M, N, K)
    av = a.view(np.float16).astype(np.float32).reshape(M, K)
    bv = b.view(np.float16).astype(np.float32).reshape(K, N)
    s32 = np.zeros((M, N), np.float32)
    for k in range(K):
        s32 += np.outer(av[:, k], bv[k])
    got = np.maximum(s32, 0).astype(np.float16).view(np.uint16)
    rep = gate(got, c, K, Sa)
    assert rep.ok, str(rep)


def test_dropped_k_chunk_fails_supplementary_gates(oracle_lib):
    # the skinny workload's scale: a dropped 1/8 of K can slip under the
    # contract's absolute tolerance but not under G1/G2
    M, N, K = 16, 256, 8192
    a, b = wl.generate_dense(M, N, K, "uniform_invsqrtk", 3)
    c, S, Sa = oracle_lib.gemm_relu(a, b, M, N, K, want_sums=True)
    a2 = a.reshape(M, K).copy()
    a2[:, :K // 8] = 0
    bad = oracle_lib.gemm_relu(a2.reshape(-1), b, M, N, K)
    rep = gate(bad, c, K, Sa)
    assert not rep.ok
    assert rep.g1 > 1e-3 or rep.g2_fail > 0


def test_sign_and_nan_fail(oracle_lib):
    _, _, c, _, Sa = _case(oracle_lib)
    bad = c.copy()
    bad[0] = 0x8000            # -0.0
    assert gate(bad, c, 256, Sa).negative == 1
    bad = c.copy()
    bad[5] = 0x7E00
    assert not gate(bad, c, 256, Sa).ok


def test_transposed_output_fails(oracle_lib):
    M = N = 64
    a, b, c, _, Sa = _case(oracle_lib, M, N, 128)
    bad = c.reshape(M, N).T.copy().reshape(-1)
    assert not gate(bad, c, 128, Sa).ok


def test_truncating_store_shows_in_bit_exact_fraction(oracle_lib):
    # round-toward-zero instead of nearest-even passes the loose contract gate
    # (the GPU tie probe catches it bit-exactly); the gate's bit-exact fraction
    # over the positive outputs exposes it
    M, N, K = 64, 48, 256
    a, b, c, S, Sa = _case(oracle_lib, M, N, K)
    s = S.reshape(-1)
    r = np.maximum(s, 0).astype(np.float32)
    bits = r.view(np.uint32)
    # truncate the fp32 value to 11 significant bits, then convert (exact)
    trunc = (bits & ~np.uint32((1 << 13) - 1)).view(np.float32)
    got = trunc.astype(np.float16).view(np.uint16)
    pos = c != 0
    rep = gate(got[pos], c[pos], K, Sa.reshape(-1)[pos])
    assert rep.bit_exact_frac < 0.6
