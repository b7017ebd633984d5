"""GPU parity at the edges of the launch and addressing limits: batches past
the 65535 grid rows a launch takes, leading dimensions at and past the limit
of the 32-bit buffer offsets, long K, and very wide N.  Inputs are seeded,
expected values come from the oracle."""

import sys

import numpy as np
import pytest

import workloads as wl
from parity import gate

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


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
def _auto_path(tg):
    tg.tg_set_path(tg.TG_PATH_AUTO)
    yield
    tg.tg_set_path(tg.TG_PATH_AUTO)


def dev(bits) -> "torch.Tensor":
    x = np.asarray(bits, dtype=np.uint16).reshape(-1)
    return torch.from_numpy(x.view(np.int16).copy()).to("cuda")


def host(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def call(tg, a_d, b_d, c_d, M, N, K, lda, ldb, ldc, sA=0, sB=0, sC=0, batch=1):
    s = torch.cuda.current_stream().cuda_stream
    if batch == 1:
        st = tg.tg_gemm_relu_f16(a_d.data_ptr(), b_d.data_ptr(), c_d.data_ptr(), M, N, K, lda,
                                 ldb, ldc, s)
    else:
        st = tg.tg_gemm_relu_f16_strided_batched(a_d.data_ptr(), b_d.data_ptr(), c_d.data_ptr(),
                                                 M, N, K, lda, ldb, ldc, sA, sB, sC, batch, s)
    assert st == tg.TG_OK, tg.tg_status_string(st)
    torch.cuda.synchronize()
    return tg.tg_path_name(tg.tg_last_path())


@pytest.mark.parametrize("path,M,N,K", [("tile128", 16, 16, 16), ("generic", 9, 13, 11),
                                        ("skinny", 16, 24, 40), ("naive", 3, 8, 8)])
def test_batch_beyond_one_launch(tg, oracle_lib, path, M, N, K):
    # 70000 slices: the launchers split the batch into grids of at most
    # 65535 rows; the slices past the split must be computed too
    batch = 70000
    a, b = wl.generate_dense(M, N, K, "uniform", 31, batch=batch)
    # one thread: the oracle would otherwise start its threads once per slice
    ref, _, Sa = oracle_lib.gemm_relu(a, b, M, N, K, batch=batch, want_sums=True, threads=1)
    assert tg.tg_set_path(getattr(tg, f"TG_PATH_{path.upper()}")) >= 0
    a_d, b_d = dev(a), dev(b)
    c_d = dev(np.full(batch * M * N, 0x7E00, np.uint16))
    say(f"limits batch={batch} {M}x{N}x{K} path={path}")
    used = call(tg, a_d, b_d, c_d, M, N, K, K, N, N, M * K, K * N, M * N, batch)
    assert used == path
    rep = gate(host(c_d), ref, K, Sa.reshape(-1))
    assert rep.ok, str(rep)


@pytest.mark.parametrize("ldb,expect", [(1 << 21, "tile128"), ((1 << 21) + 8, "generic")])
def test_leading_dimension_at_the_offset_limit(tg, oracle_lib, ldb, expect):
    # the direct-to-LDS kernels address a B panel with 32-bit byte offsets and
    # take ldb <= 2^21; one step past it the any-layout kernel serves the call
    M, N, K = 200, 264, 72
    a, b = wl.generate_dense(M, N, K, "uniform", 32)
    b = wl.pad_rows(b, K, N, ldb)
    ref, _, Sa = oracle_lib.gemm_relu(a, b, M, N, K, K, ldb, N, want_sums=True)
    a_d, b_d = dev(a), dev(b)
    c_d = dev(np.zeros(M * N, np.uint16))
    say(f"limits ldb={ldb} {M}x{N}x{K}")
    used = call(tg, a_d, b_d, c_d, M, N, K, K, ldb, N)
    assert used == expect
    rep = gate(host(c_d), ref, K, Sa.reshape(-1))
    assert rep.ok, str(rep)


@pytest.mark.parametrize("path", ["tile128", "tile256", "skinny", "generic"])
def test_long_k(tg, oracle_lib, path):
    # 2^17-long sums: the fp32 accumulation bound (G2) at its widest
    M, N, K = (48 if path == "skinny" else 136), 128, 1 << 17
    a, b = wl.generate_dense(M, N, K, "uniform_invsqrtk", 33)
    ref, _, Sa = oracle_lib.gemm_relu(a, b, M, N, K, want_sums=True)
    assert tg.tg_set_path(getattr(tg, f"TG_PATH_{path.upper()}")) >= 0
    a_d, b_d = dev(a), dev(b)
    c_d = dev(np.zeros(M * N, np.uint16))
    say(f"limits long K={K} {M}x{N} path={path}")
    used = call(tg, a_d, b_d, c_d, M, N, K, K, N, N)
    assert used == path
    rep = gate(host(c_d), ref, K, Sa.reshape(-1))
    assert rep.ok, str(rep)


def test_very_wide_n_skinny(tg, oracle_lib):
    # one row of A against 2^20 columns: 16384 column slices
    M, N, K = 1, 1 << 20, 64
    a, b = wl.generate_dense(M, N, K, "uniform_invsqrtk", 34)
    ref, _, Sa = oracle_lib.gemm_relu(a, b, M, N, K, want_sums=True)
    a_d, b_d = dev(a), dev(b)
    c_d = dev(np.zeros(M * N, np.uint16))
    say(f"limits wide N={N} M={M} K={K}")
    used = call(tg, a_d, b_d, c_d, M, N, K, K, N, N)
    assert used == "skinny"
    rep = gate(host(c_d), ref, K, Sa.reshape(-1))
    assert rep.ok, str(rep)
