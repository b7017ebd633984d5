"""Pins for the attention oracle (softmax(scale Q K^T) V, fp16 storage).

  * against an independent vectorized numpy float64 implementation (matmul,
    exp) on random shapes, causal or not, Sq != Sk: the same binary64 values
    up to summation order, so the fp16 outputs agree within one ulp and are
    almost all identical,
  * closed forms: Q = 0 gives the mean of the visible V rows; the first causal
    query sees only key 0 and gets V[0]; a dominant score selects its V row;
    a query with no visible key gets 0,
  * invariants: heads and batches are independent; permuting keys together
    with values does not change a non-causal output.
A transposed Q K^T, a missing scale, a causal mask off by one, a softmax over
the wrong axis or a mixed-up head layout each fails one of them.
"""

import numpy as np
import pytest


def f16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def v16(b):
    return np.asarray(b, np.uint16).view(np.float16).astype(np.float64)


def numpy_attention(q, k, v, B, Sq, Sk, H, D, scale, causal):
    Q = v16(q).reshape(B, Sq, H, D).transpose(0, 2, 1, 3)
    K = v16(k).reshape(B, Sk, H, D).transpose(0, 2, 1, 3)
    V = v16(v).reshape(B, Sk, H, D).transpose(0, 2, 1, 3)
    S = scale * (Q @ K.transpose(0, 1, 3, 2))                     # (B, H, Sq, Sk)
    if causal:
        i = np.arange(Sq)[:, None]
        j = np.arange(Sk)[None, :]
        S = np.where(j <= i + (Sk - Sq), S, -np.inf)
    mx = S.max(axis=-1, keepdims=True)
    mx = np.where(np.isfinite(mx), mx, 0.0)
    P = np.exp(S - mx)
    den = P.sum(axis=-1, keepdims=True)
    P = np.where(den > 0, P / np.where(den > 0, den, 1.0), 0.0)
    O = P @ V                                                      # (B, H, Sq, D)
    return O.transpose(0, 2, 1, 3).reshape(-1)


def rand_qkv(rng, B, Sq, Sk, H, D, spread=1.0):
    q = f16(rng.uniform(-spread, spread, B * Sq * H * D))
    k = f16(rng.uniform(-spread, spread, B * Sk * H * D))
    v = f16(rng.uniform(-1, 1, B * Sk * H * D))
    return q, k, v


@pytest.mark.parametrize("B,Sq,Sk,H,D,causal", [
    (1, 7, 7, 1, 8, False), (2, 9, 13, 3, 16, False), (1, 16, 16, 2, 64, True),
    (2, 5, 11, 2, 32, True), (1, 12, 5, 1, 8, True), (1, 33, 40, 4, 128, False)])
def test_matches_numpy_float64(oracle_lib, B, Sq, Sk, H, D, causal):
    rng = np.random.default_rng(Sq * 100 + Sk)
    q, k, v = rand_qkv(rng, B, Sq, Sk, H, D, spread=2.0)
    scale = 1.0 / np.sqrt(D)
    got = oracle_lib.attention(q, k, v, B, Sq, Sk, H, D, scale, causal)
    ref = numpy_attention(q, k, v, B, Sq, Sk, H, D, scale, causal)
    ref16 = f16(ref)
    gv = v16(got)
    ulp = np.spacing(np.abs(ref16.view(np.float16))).astype(np.float64)
    assert np.all(np.abs(gv - v16(ref16)) <= ulp)
    assert np.mean(got == ref16) > 0.99


def test_zero_queries_average_the_visible_values(oracle_lib):
    # 1/n and the sums are exact for n = 4 keys and values in eighths
    B, S, H, D = 1, 4, 2, 8
    rng = np.random.default_rng(1)
    q = np.zeros(B * S * H * D, np.uint16)
    k = f16(rng.uniform(-1, 1, B * S * H * D))
    v = f16(rng.integers(-8, 9, B * S * H * D) / 8.0)
    got = v16(oracle_lib.attention(q, k, v, B, S, S, H, D, 0.7)).reshape(B, S, H, D)
    want = v16(v).reshape(B, S, H, D).mean(axis=1)
    for i in range(S):
        assert np.array_equal(got[:, i], want)
    # causal: query i averages keys 0..i
    got = v16(oracle_lib.attention(q, k, v, B, S, S, H, D, 0.7, causal=True)).reshape(B, S, H, D)
    vv = v16(v).reshape(B, S, H, D)
    for i in (0, 1, 3):                       # counts 1, 2, 4: exact reciprocals
        assert np.array_equal(got[:, i], vv[:, :i + 1].mean(axis=1).astype(np.float16))


def test_first_causal_query_sees_only_the_first_key(oracle_lib):
    rng = np.random.default_rng(2)
    B, S, H, D = 2, 6, 3, 16
    q, k, v = rand_qkv(rng, B, S, S, H, D)
    got = oracle_lib.attention(q, k, v, B, S, S, H, D, 0.25, causal=True).reshape(B, S, H, D)
    assert np.array_equal(got[:, 0], v.reshape(B, S, H, D)[:, 0])


def test_dominant_score_selects_its_value_row(oracle_lib):
    B, S, H, D = 1, 8, 1, 16
    rng = np.random.default_rng(3)
    k = f16(rng.uniform(-0.01, 0.01, S * D))
    kk = v16(k).reshape(S, D)
    kk[5] = 1.0                                   # key 5 aligns with every query
    k = f16(kk.reshape(-1))
    q = f16(np.ones(S * D))
    v = f16(rng.uniform(-1, 1, S * D))
    got = oracle_lib.attention(q, k, v, B, S, S, H, D, 100.0).reshape(S, D)
    # exp(-100 * 16 * 0.99) underflows: the weight of key 5 is 1 exactly
    assert np.array_equal(got, np.tile(v.reshape(S, D)[5], (S, 1)))


def test_no_visible_key_gives_zero(oracle_lib):
    # causal with Sk < Sq: query i sees keys j <= i - (Sq - Sk)
    B, Sq, Sk, H, D = 1, 6, 2, 1, 8
    rng = np.random.default_rng(4)
    q, k, v = rand_qkv(rng, B, Sq, Sk, H, D)
    got = oracle_lib.attention(q, k, v, B, Sq, Sk, H, D, 0.3, causal=True).reshape(Sq, D)
    assert np.all(got[:4] == 0)
    assert np.array_equal(got[4], v.reshape(Sk, D)[0])


def test_heads_and_batches_are_independent(oracle_lib):
    B, S, H, D = 2, 9, 3, 16
    rng = np.random.default_rng(5)
    q, k, v = rand_qkv(rng, B, S, S, H, D)
    full = oracle_lib.attention(q, k, v, B, S, S, H, D, 0.5, causal=True).reshape(B, S, H, D)
    for b in range(B):
        for h in range(H):
            sl = lambda t: np.ascontiguousarray(t.reshape(B, S, H, D)[b, :, h, :]).reshape(-1)
            one = oracle_lib.attention(sl(q), sl(k), sl(v), 1, S, S, 1, D, 0.5, causal=True)
            assert np.array_equal(one.reshape(S, D), full[b, :, h, :])


def test_key_permutation_invariance(oracle_lib):
    B, Sq, Sk, H, D = 1, 5, 12, 2, 32
    rng = np.random.default_rng(6)
    q, k, v = rand_qkv(rng, B, Sq, Sk, H, D)
    perm = rng.permutation(Sk)
    kp = k.reshape(B, Sk, H, D)[:, perm].reshape(-1)
    vp = v.reshape(B, Sk, H, D)[:, perm].reshape(-1)
    a = v16(oracle_lib.attention(q, k, v, B, Sq, Sk, H, D, 0.4))
    b = v16(oracle_lib.attention(q, kp, vp, B, Sq, Sk, H, D, 0.4))
    ulp = np.spacing(np.abs(a.astype(np.float16))).astype(np.float64)
    assert np.all(np.abs(a - b) <= ulp)


def test_row_statistics(oracle_lib):
    B, S, H, D = 1, 6, 1, 8
    rng = np.random.default_rng(7)
    q, k, v = rand_qkv(rng, B, S, S, H, D)
    _, mx, sm = oracle_lib.attention(q, k, v, B, S, S, H, D, 0.5, causal=True, want_stats=True)
    Q = v16(q).reshape(S, D)
    K = v16(k).reshape(S, D)
    for i in range(S):
        s = 0.5 * (K[:i + 1] @ Q[i])
        assert np.isclose(mx[0, 0, i], s.max(), rtol=0, atol=1e-12)
        assert np.isclose(sm[0, 0, i], np.exp(s - s.max()).sum(), rtol=1e-12)


def numpy_attention_gqa(q, k, v, B, Sq, Sk, H, Hkv, D, scale, causal):
    # independent reference: repeat each key/value head over its group of
    # query heads, then plain multi-head attention in numpy
    g = H // Hkv
    K = v16(k).reshape(B, Sk, Hkv, D).repeat(g, axis=2)
    V = v16(v).reshape(B, Sk, Hkv, D).repeat(g, axis=2)
    return numpy_attention(q, f16(K.reshape(-1)), f16(V.reshape(-1)), B, Sq, Sk, H, D, scale,
                           causal)


@pytest.mark.parametrize("B,Sq,Sk,H,Hkv,D,causal", [
    (1, 7, 9, 4, 2, 8, False), (2, 5, 11, 6, 3, 16, True), (1, 1, 33, 8, 1, 32, False),
    (2, 12, 12, 4, 4, 16, True), (1, 3, 20, 6, 2, 64, True)])
def test_grouped_query_heads_match_numpy(oracle_lib, B, Sq, Sk, H, Hkv, D, causal):
    rng = np.random.default_rng(Sq * 31 + H)
    q = f16(rng.uniform(-2, 2, B * Sq * H * D))
    k = f16(rng.uniform(-2, 2, B * Sk * Hkv * D))
    v = f16(rng.uniform(-1, 1, B * Sk * Hkv * D))
    scale = 1.0 / np.sqrt(D)
    got = oracle_lib.attention(q, k, v, B, Sq, Sk, H, D, scale, causal, kv_heads=Hkv)
    ref16 = f16(numpy_attention_gqa(q, k, v, B, Sq, Sk, H, Hkv, D, scale, causal))
    ulp = np.spacing(np.abs(ref16.view(np.float16))).astype(np.float64)
    assert np.all(np.abs(v16(got) - v16(ref16)) <= ulp)
    assert np.mean(got == ref16) > 0.99


def test_query_heads_of_a_group_share_keys_and_values(oracle_lib):
    # two query heads with identical queries in one group give identical
    # outputs; the same queries in another group (other keys) differ
    B, Sq, Sk, H, Hkv, D = 1, 4, 10, 4, 2, 16
    rng = np.random.default_rng(21)
    qh = f16(rng.uniform(-1, 1, Sq * D)).reshape(Sq, 1, D)
    q = np.repeat(qh, H, axis=1).reshape(-1)
    k = f16(rng.uniform(-1, 1, B * Sk * Hkv * D))
    v = f16(rng.uniform(-1, 1, B * Sk * Hkv * D))
    o = oracle_lib.attention(q, k, v, B, Sq, Sk, H, D, 0.5, kv_heads=Hkv).reshape(Sq, H, D)
    assert np.array_equal(o[:, 0], o[:, 1]) and np.array_equal(o[:, 2], o[:, 3])
    assert not np.array_equal(o[:, 0], o[:, 2])


def test_grouped_query_bad_group_is_rejected(oracle_lib):
    z = np.zeros(64, np.uint16)
    with pytest.raises(ValueError):
        oracle_lib.attention(z, z, z, 1, 1, 1, 3, 8, 1.0, kv_heads=2)
