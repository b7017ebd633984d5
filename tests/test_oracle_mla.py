"""Pins for the latent-attention decode oracle (one query per sequence, heads
sharing one cached row per token: the first 512 values are key and value, the
last 64 a rotary key part).

  * reduction: the decode is attention with one query position, one
    key/value head of size 576 and V = K, whose first 512 output columns it
    keeps; the attention oracle (pinned on its own against numpy, closed forms
    and invariants) gives the same bits, with and without ragged lengths,
  * closed forms: two visible tokens whose scores differ by ln 3 give weights
    3/4 and 1/4 exactly, with the difference carried by the rotary part or by
    the latent part (a dropped term or swapped weights fails); one visible
    token returns its latent row; a zero scale averages the visible latent
    rows; no visible token gives 0,
  * invariants: tokens past a sequence's length never matter (even NaN);
    heads are independent and permute with Q; visible tokens may be reordered.
"""

import math

import numpy as np
import pytest

DL, DR = 512, 64
DQ = DL + DR


def f16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def v16(b):
    return np.asarray(b, np.uint16).view(np.float16).astype(np.float64)


def inputs(B, H, Sk, seed):
    rng = np.random.default_rng(50_000 + seed)
    q = f16(rng.normal(0, 1, B * H * DQ))
    kv = f16(rng.normal(0, 1, B * Sk * DQ))
    return q, kv


@pytest.mark.parametrize("B,H,Sk", [(1, 1, 1), (2, 3, 70), (3, 16, 130)])
def test_is_attention_with_one_shared_head_and_v_equal_k(oracle_lib, B, H, Sk):
    q, kv = inputs(B, H, Sk, B + H + Sk)
    scale = 1.0 / math.sqrt(192)
    got = oracle_lib.mla_decode(q, kv, B, H, Sk, scale).reshape(B, H, DL)
    ref = oracle_lib.attention(q, kv, kv, B, 1, Sk, H, DQ, scale, kv_heads=1).reshape(B, H, DQ)
    assert np.array_equal(got, ref[:, :, :DL])


def test_ragged_lengths_match_attention_on_the_truncated_cache(oracle_lib):
    B, H, Sk = 4, 5, 90
    q, kv = inputs(B, H, Sk, 7)
    lens = [90, 1, 37, 64]
    got = oracle_lib.mla_decode(q, kv, B, H, Sk, 0.2, seqlens=lens).reshape(B, H, DL)
    Q = q.reshape(B, H, DQ)
    C = kv.reshape(B, Sk, DQ)
    for b, n in enumerate(lens):
        c = np.ascontiguousarray(C[b, :n])
        ref = oracle_lib.attention(np.ascontiguousarray(Q[b]), c, c, 1, 1, n, H, DQ, 0.2,
                                   kv_heads=1).reshape(H, DQ)
        assert np.array_equal(got[b], ref[:, :DL]), b


@pytest.mark.parametrize("where", [DL, DL + DR - 1, 0, 300])
@pytest.mark.parametrize("first_wins", [True, False])
def test_two_tokens_three_to_one(oracle_lib, where, first_wins):
    # q is one unit vector; token w has a 1 at that position, the other a 0,
    # so with scale ln 3 the weights are exactly 3/4 and 1/4
    rng = np.random.default_rng(3)
    u = rng.integers(-40, 40, DL).astype(np.float64)
    w = rng.integers(-40, 40, DL).astype(np.float64)
    q = np.zeros(DQ)
    q[where] = 1.0
    c = np.zeros((2, DQ))
    c[0, :DL], c[1, :DL] = 4 * u, 4 * w
    win = 0 if first_wins else 1
    c[win, where] = 1.0                         # the scores: 1 and 0 (may overwrite
    c[1 - win, where] = 0.0                     # one latent value of each token)
    lat = c[:, :DL]
    out = v16(oracle_lib.mla_decode(f16(q), f16(c.reshape(-1)), 1, 1, 2, math.log(3.0)))
    want = 0.75 * lat[win] + 0.25 * lat[1 - win]
    assert np.array_equal(out, want)


def test_one_visible_token_returns_its_latent_row(oracle_lib):
    B, H, Sk = 2, 4, 9
    q, kv = inputs(B, H, Sk, 11)
    kv = kv.reshape(B, Sk, DQ).copy()
    kv[np.abs(v16(kv)) == 0.0] = f16(0.5)        # no zeros: -0 would come back as +0
    got = oracle_lib.mla_decode(q, kv.reshape(-1), B, H, Sk, 0.3, seqlens=[1, 1])
    got = got.reshape(B, H, DL)
    for b in range(B):
        for h in range(H):
            assert np.array_equal(got[b, h], kv[b, 0, :DL])


def test_zero_scale_averages_the_visible_rows(oracle_lib):
    B, H, Sk = 2, 3, 12
    q, kv = inputs(B, H, Sk, 12)
    lens = [8, 4]                                 # powers of two: exact weights
    got = oracle_lib.mla_decode(q, kv, B, H, Sk, 0.0, seqlens=lens).reshape(B, H, DL)
    C = v16(kv).reshape(B, Sk, DQ)
    for b, n in enumerate(lens):
        mean = C[b, :n, :DL].sum(axis=0) / n
        for h in range(H):
            assert np.array_equal(got[b, h], oracle_lib.enc16(mean))


def test_no_visible_token_gives_zero(oracle_lib):
    q, kv = inputs(2, 3, 5, 13)
    got = oracle_lib.mla_decode(q, kv, 2, 3, 5, 0.1, seqlens=[0, 5]).reshape(2, 3, DL)
    assert not got[0].any() and got[1].any()
    assert not oracle_lib.mla_decode(q, kv, 2, 3, 0, 0.1).any()


def test_tokens_past_the_length_are_ignored(oracle_lib):
    B, H, Sk = 2, 3, 40
    q, kv = inputs(B, H, Sk, 14)
    lens = [17, 33]
    a = oracle_lib.mla_decode(q, kv, B, H, Sk, 0.1, seqlens=lens)
    poisoned = kv.reshape(B, Sk, DQ).copy()
    for b, n in enumerate(lens):
        poisoned[b, n:] = 0x7E00                  # NaN
    b_ = oracle_lib.mla_decode(q, poisoned.reshape(-1), B, H, Sk, 0.1, seqlens=lens)
    assert np.array_equal(a, b_)


def test_heads_are_independent_and_permute_with_q(oracle_lib):
    B, H, Sk = 1, 6, 50
    q, kv = inputs(B, H, Sk, 15)
    perm = np.array([3, 0, 5, 1, 4, 2])
    a = oracle_lib.mla_decode(q, kv, B, H, Sk, 0.1).reshape(H, DL)
    qp = q.reshape(H, DQ)[perm].reshape(-1)
    b_ = oracle_lib.mla_decode(qp, kv, B, H, Sk, 0.1).reshape(H, DL)
    assert np.array_equal(b_, a[perm])


def test_visible_tokens_may_be_reordered(oracle_lib):
    B, H, Sk = 1, 4, 64
    q, kv = inputs(B, H, Sk, 16)
    perm = np.random.default_rng(0).permutation(Sk)
    a = v16(oracle_lib.mla_decode(q, kv, B, H, Sk, 0.15))
    kvp = kv.reshape(Sk, DQ)[perm].reshape(-1)
    b_ = v16(oracle_lib.mla_decode(q, kvp, B, H, Sk, 0.15))
    ulp = np.spacing(np.abs(a).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(a - b_) <= ulp)


def test_stats_and_bad_lengths(oracle_lib):
    B, H, Sk = 2, 2, 6
    q, kv = inputs(B, H, Sk, 17)
    _, mx, sm = oracle_lib.mla_decode(q, kv, B, H, Sk, 0.5, want_stats=True)
    S = 0.5 * np.einsum("bhd,bkd->bhk", v16(q).reshape(B, H, DQ), v16(kv).reshape(B, Sk, DQ))
    assert np.allclose(mx, S.max(axis=-1), rtol=1e-12, atol=1e-12)
    assert np.all(sm >= 1.0) and np.all(sm <= Sk)
    with pytest.raises(ValueError):
        oracle_lib.mla_decode(q, kv, B, H, Sk, 0.5, seqlens=[7, 1])
    with pytest.raises(ValueError):
        oracle_lib.mla_decode(q, kv, B, H, Sk, 0.5, seqlens=[-1, 1])
