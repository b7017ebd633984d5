"""GPU parity of the split-K skinny GEMM+ReLU (tg_gemm_relu_f16_splitk) against
the CPU oracle, through the C ABI: the same contract gates as the single-pass
path (per-element tolerance, relative error, fp32 summation bound, no negative
or NaN output), canaries around C and past the workspace, and bitwise
determinism."""

import sys

import numpy as np
import pytest

import workloads as wl
from parity import gate

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SENTINEL = 0x7E00


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def tg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiled_dense_gemm_05_amd as tg
    return tg


def dev(bits) -> "torch.Tensor":
    x = np.asarray(bits, dtype=np.uint16).reshape(-1)
    return torch.from_numpy(x.view(np.int16).copy()).to("cuda")


def host(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def run(tg, a, b, M, N, K, lda, ldb, ldc, splits, guard=64):
    csize = (M - 1) * ldc + N if M and N else 0
    a_d = dev(a if a.size else np.zeros(8, np.uint16))
    b_d = dev(b if b.size else np.zeros(8, np.uint16))
    c_d = dev(np.full(csize + guard, SENTINEL, np.uint16))
    nb = tg.tg_gemm_splitk_workspace_bytes(M, N, splits)
    assert nb >= 0
    ws = torch.full((nb + 256,), 0x55, dtype=torch.uint8, device="cuda")
    st = tg.tg_gemm_relu_f16_splitk(a_d.data_ptr(), b_d.data_ptr(), c_d.data_ptr(), M, N, K, lda,
                                    ldb, ldc, splits, ws.data_ptr(), nb,
                                    torch.cuda.current_stream().cuda_stream)
    assert st == tg.TG_OK, tg.tg_status_string(st)
    torch.cuda.synchronize()
    assert np.all(ws[nb:].cpu().numpy() == 0x55), "wrote past the workspace"
    out = host(c_d)
    assert np.all(out[csize:] == SENTINEL), "wrote past C"
    return out[:csize]


CASES = [
    (16, 1024, 8192, 1), (16, 1024, 8192, 2), (16, 1024, 8192, 8), (1, 264, 520, 3),
    (7, 1000, 136, 2), (17, 512, 1000, 4), (64, 520, 2056, 5), (33, 96, 64, 2), (48, 8, 8, 1),
]


@pytest.mark.parametrize("M,N,K,splits", CASES)
def test_splitk_matches_oracle(tg, oracle_lib, M, N, K, splits):
    a, b = wl.generate_dense(M, N, K, "uniform", M + N + splits)
    ref, S, Sa = oracle_lib.gemm_relu(a, b, M, N, K, want_sums=True)
    say(f"splitk M={M} N={N} K={K} splits={splits}")
    got = run(tg, a, b, M, N, K, K, N, N, splits)
    rep = gate(got, ref, K, Sa.reshape(-1))
    assert rep.ok, str(rep)


def test_padded_leading_dimensions(tg, oracle_lib):
    M, N, K, lda, ldb, ldc = 13, 264, 1000, 1032, 272, 280
    a, b = wl.generate_dense(M, N, K, "uniform", 3)
    a = wl.pad_rows(a, M, K, lda)
    b = wl.pad_rows(b, K, N, ldb)
    csize = (M - 1) * ldc + N
    ref = np.full(csize, SENTINEL, np.uint16)
    ref, S, Sa = oracle_lib.gemm_relu(a, b, M, N, K, lda, ldb, ldc, C=ref, want_sums=True)
    say("splitk padded")
    got = run(tg, a, b, M, N, K, lda, ldb, ldc, 3)
    win = np.zeros(csize, bool)
    win[(np.arange(M)[:, None] * ldc + np.arange(N)[None, :]).reshape(-1)] = True
    assert np.all(got[~win] == SENTINEL), "wrote outside the M x N window"
    rep = gate(got[win], ref[win], K, Sa.reshape(-1))
    assert rep.ok, str(rep)


def test_k_zero_writes_zeros(tg):
    say("splitk K=0")
    got = run(tg, np.zeros(0, np.uint16), np.zeros(0, np.uint16), 4, 64, 0, 8, 64, 64, 1)
    assert np.all(got == 0)


def test_same_as_single_pass_within_the_gate_and_deterministic(tg, oracle_lib):
    w = wl.WORKLOADS["skinny_16x16384x8192"]
    a, b = wl.generate(w)
    say("splitk on the 16 x 16384 x 8192 workload, splits 4")
    x = run(tg, a, b, w.M, w.N, w.K, w.K, w.N, w.N, 4)
    y = run(tg, a, b, w.M, w.N, w.K, w.K, w.N, w.N, 4)
    assert np.array_equal(x, y)
    idx = wl.sample_positions(w, 4000)
    ref, _, sa = oracle_lib.gemm_relu_sampled(a, b, w.K, w.lda_, w.ldb_, idx)
    got = x.reshape(w.M, w.N)[idx[:, 1], idx[:, 2]]
    vals = x.view(np.float16).astype(np.float64)
    assert np.all(vals >= 0) and not np.any(np.isnan(vals))
    rep = gate(got, ref, w.K, sa)
    assert rep.ok, str(rep)
