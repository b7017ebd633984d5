"""GPU parity of the latent-attention decode (tg_mla_decode_f16) against the
CPU oracle, through the C ABI.

Tolerance, from the kernel's arithmetic (as for the attention forward):
scores and sums are fp32, each probability is rounded to fp16 before the
value product (relative error <= 2^-11, so the output moves by at most
2^-11 * max|V| from the probabilities and as much again from the normalizer);
with several key ranges each range's normalised output (a convex combination
of cached values, so at most max|V| in size) is rounded to fp16, at most
2^-11 * max|V| more, and the ranges are combined with fp32 weights; the
output is rounded to fp16 once: |O_gpu - O_ref| <= 2^-9 * max|V| +
ulp16(O_ref), V the latent parts of the visible rows.
"""

import math
import sys

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DL, DQ = 512, 576
SCALE = 1.0 / math.sqrt(192)


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def tg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiled_dense_gemm_05_amd as tg
    return tg


@pytest.fixture(autouse=True)
def _default_splits(tg):
    yield
    tg.tg_set_mla_splits(-1)


def dev(bits) -> "torch.Tensor":
    x = np.asarray(bits, dtype=np.uint16).reshape(-1)
    return torch.from_numpy(x.view(np.int16).copy()).to("cuda")


def host(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def v16(b):
    return np.asarray(b, np.uint16).view(np.float16).astype(np.float64)


def inputs(B, H, Sk, seed, spread=1.0):
    rng = np.random.default_rng(70_000 + seed)
    q = np.asarray(rng.normal(0, spread, B * H * DQ)).astype(np.float16).view(np.uint16)
    kv = np.asarray(rng.normal(0, 1, B * Sk * DQ)).astype(np.float16).view(np.uint16)
    return q, kv


def check(got, ref, kv, B, Sk, lens=None):
    g, r = v16(got), v16(ref)
    assert not np.any(np.isnan(g)), "NaN in the output"
    c = v16(kv).reshape(B, Sk, DQ)[:, :, :DL] if Sk else np.zeros((B, 0, DL))
    vmax = 0.0
    for b in range(B):
        n = Sk if lens is None else max(0, min(Sk, int(lens[b])))
        if n:
            vmax = max(vmax, float(np.abs(c[b, :n]).max()))
    ulp = np.spacing(np.abs(r).astype(np.float16)).astype(np.float64)
    err = np.abs(g - r)
    bad = int((err > 2.0 ** -9 * vmax + ulp).sum())
    assert bad == 0, f"{bad} outputs beyond the bound, max err {err.max():.3g}"


def run(tg, q, kv, B, H, Sk, scale, lens=None, ws_bytes=None):
    q_d = dev(q)
    kv_d = dev(kv) if kv.size else dev(np.zeros(8))
    o_d = dev(np.full(B * H * DL + 64, 0x7E00, np.uint16))
    sl_d = torch.tensor(np.asarray(lens, np.int32), device="cuda") if lens is not None else None
    need = tg.tg_mla_decode_workspace_bytes(B, H, Sk)
    assert need >= 0
    nb = need if ws_bytes is None else ws_bytes
    ws = torch.full((nb + 64,), 0x55, dtype=torch.uint8, device="cuda") if nb else None
    st = tg.tg_mla_decode_f16(q_d.data_ptr(), kv_d.data_ptr(), o_d.data_ptr(),
                              sl_d.data_ptr() if sl_d is not None else 0, B, H, Sk, scale,
                              ws.data_ptr() if ws is not None else 0, nb,
                              torch.cuda.current_stream().cuda_stream)
    assert st == tg.TG_OK, tg.tg_status_string(st)
    torch.cuda.synchronize()
    out = host(o_d)
    assert np.all(out[B * H * DL:] == 0x7E00), "wrote past O"
    assert tg.tg_path_name(tg.tg_last_path()) == "mla"
    if ws is not None:
        assert np.all(ws[nb:].cpu().numpy() == 0x55), "wrote past the workspace"
    return out[:B * H * DL]


CASES = [
    (1, 1, 1), (1, 16, 70), (2, 64, 32), (3, 128, 257), (2, 130, 1000), (1, 128, 4096),
    (5, 3, 300), (1, 64, 0),
]


@pytest.mark.parametrize("splits", [-1, 1, 2, 5])
@pytest.mark.parametrize("B,H,Sk", CASES)
def test_mla_matches_oracle(tg, oracle_lib, splits, B, H, Sk):
    q, kv = inputs(B, H, Sk, B * 7 + H + Sk)
    ref = oracle_lib.mla_decode(q, kv, B, H, Sk, SCALE)
    say(f"mla B={B} H={H} Sk={Sk} splits={splits}")
    tg.tg_set_mla_splits(splits)
    need = tg.tg_mla_decode_workspace_bytes(B, H, Sk)
    per = B * H * (DL + 2) * 4
    ws = max(need, per * max(splits, 1))
    check(run(tg, q, kv, B, H, Sk, SCALE, ws_bytes=ws), ref, kv, B, Sk)


@pytest.mark.parametrize("splits", [1, 3])
def test_ragged_lengths_and_junk_past_them(tg, oracle_lib, splits):
    # lengths 0, 1, a tile edge, mid-tile and full; rows past a length hold NaN
    B, H, Sk = 6, 80, 300
    lens = [0, 1, 32, 33, 299, 300]
    q, kv = inputs(B, H, Sk, 3)
    ref = oracle_lib.mla_decode(q, kv, B, H, Sk, SCALE, seqlens=lens)
    junk = kv.reshape(B, Sk, DQ).copy()
    for b, n in enumerate(lens):
        junk[b, n:] = 0x7E00
    say(f"mla ragged splits={splits}")
    tg.tg_set_mla_splits(splits)
    got = run(tg, q, junk.reshape(-1), B, H, Sk, SCALE, lens=lens,
              ws_bytes=B * H * (DL + 2) * 4 * splits)
    check(got, ref, kv, B, Sk, lens)
    o = v16(got).reshape(B, H, DL)
    assert np.all(o[0] == 0.0), "a sequence with no visible token must give 0"


def test_lengths_outside_the_cache_are_clamped(tg, oracle_lib):
    B, H, Sk = 3, 8, 100
    q, kv = inputs(B, H, Sk, 4)
    ref = oracle_lib.mla_decode(q, kv, B, H, Sk, SCALE, seqlens=[0, 100, 100])
    say("mla clamped lengths")
    check(run(tg, q, kv, B, H, Sk, SCALE, lens=[-5, 100, 1 << 30]), ref, kv, B, Sk)


@pytest.mark.parametrize("spread,scale", [(3.0, 0.5), (0.01, 1.0), (1.0, -SCALE), (1.0, 0.0)])
def test_sharp_flat_negative_and_zero_scale(tg, oracle_lib, spread, scale):
    B, H, Sk = 2, 64, 700
    q, kv = inputs(B, H, Sk, 5, spread=spread)
    ref = oracle_lib.mla_decode(q, kv, B, H, Sk, scale)
    say(f"mla spread={spread} scale={scale}")
    tg.tg_set_mla_splits(3)
    check(run(tg, q, kv, B, H, Sk, scale, ws_bytes=B * H * (DL + 2) * 4 * 3), ref, kv, B, Sk)


def test_small_workspace_lowers_the_split_count(tg, oracle_lib):
    B, H, Sk = 1, 64, 4096
    q, kv = inputs(B, H, Sk, 6)
    ref = oracle_lib.mla_decode(q, kv, B, H, Sk, SCALE)
    per = B * H * (DL + 2) * 4
    say("mla workspace sizes")
    outs = [run(tg, q, kv, B, H, Sk, SCALE, ws_bytes=w) for w in (0, per, 3 * per + 17, None)]
    for o in outs:
        check(o, ref, kv, B, Sk)


def test_deterministic(tg):
    B, H, Sk = 4, 128, 2000
    q, kv = inputs(B, H, Sk, 8)
    say("mla determinism")
    a = run(tg, q, kv, B, H, Sk, SCALE)
    b = run(tg, q, kv, B, H, Sk, SCALE)
    assert np.array_equal(a, b)


def test_rejects_bad_arguments(tg):
    q = torch.zeros(2 * 4 * DQ, dtype=torch.float16, device="cuda")
    kv = torch.zeros(2 * 8 * DQ, dtype=torch.float16, device="cuda")
    o = torch.zeros(2 * 4 * DL + 8, dtype=torch.float16, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    bad = tg.TG_ERR_INVALID_ARG
    assert tg.tg_mla_decode_f16(0, kv.data_ptr(), o.data_ptr(), 0, 2, 4, 8, 0.1, 0, 0, s) == bad
    assert tg.tg_mla_decode_f16(q.data_ptr(), kv.data_ptr(), o.data_ptr() + 2, 0, 2, 4, 8, 0.1,
                                0, 0, s) == bad
    assert tg.tg_mla_decode_f16(q.data_ptr(), kv.data_ptr(), o.data_ptr(), 0, 2, 4, 8,
                                float("nan"), 0, 0, s) == bad
    assert tg.tg_mla_decode_f16(q.data_ptr(), kv.data_ptr(), o.data_ptr(), 0, -1, 4, 8, 0.1,
                                0, 0, s) == bad
    assert tg.tg_mla_decode_f16(q.data_ptr(), kv.data_ptr(), o.data_ptr(), 0, 0, 4, 8, 0.1,
                                0, 0, s) == tg.TG_OK


def test_torch_helper(tg, oracle_lib):
    B, H, Sk = 2, 16, 333
    q, kv = inputs(B, H, Sk, 9)
    ref = oracle_lib.mla_decode(q, kv, B, H, Sk, SCALE, seqlens=[333, 100])
    qt = dev(q).view(torch.float16).reshape(B, H, DQ)
    kvt = dev(kv).view(torch.float16).reshape(B, Sk, DQ)
    lens = torch.tensor([333, 100], dtype=torch.int32, device="cuda")
    say("mla torch helper")
    o = tg.mla_decode(qt, kvt, SCALE, seqlens=lens)
    torch.cuda.synchronize()
    check(o.view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1), ref, kv, B, Sk,
          [333, 100])


@pytest.mark.parametrize("B,H,Sk", [(1, 128, 65536), (3, 256, 1000), (300, 8, 40)])
def test_long_wide_and_many(tg, oracle_lib, B, H, Sk):
    # one long sequence (the most key ranges: 256 of 256 keys), four head
    # blocks, and more sequences than the chip has compute units
    q, kv = inputs(B, H, Sk, B + H)
    ref = oracle_lib.mla_decode(q, kv, B, H, Sk, SCALE)
    say(f"mla long/wide B={B} H={H} Sk={Sk}")
    check(run(tg, q, kv, B, H, Sk, SCALE), ref, kv, B, Sk)


def test_benchmark_shape_sampled(tg, oracle_lib):
    # the benchmark workload (64 sequences x 8192 tokens, 128 heads) in the
    # launch configuration the benchmark times; the oracle computes three
    # whole sequences
    w = workloads.MLA_WORKLOAD
    B, H, Sk = w["B"], w["H"], w["Sk"]
    q, kv = workloads.generate_mla(B, H, Sk, w["seed"])
    say("mla benchmark shape")
    got = run(tg, q, kv, B, H, Sk, SCALE).reshape(B, H, DL)
    o = v16(got)
    assert np.all(np.isfinite(o))
    for b in (0, 37, B - 1):
        qb = q.reshape(B, H, DQ)[b].reshape(-1)
        kb = kv.reshape(B, Sk, DQ)[b].reshape(-1)
        ref = oracle_lib.mla_decode(qb, kb, 1, H, Sk, SCALE)
        check(got[b].reshape(-1), ref, kb, 1, Sk)
