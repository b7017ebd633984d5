"""GPU parity of the weight-only int4 GEMM (tg_gemm_w4) against the CPU oracle,
through the C ABI.  Every case prints its name before touching the GPU."""

import sys

import numpy as np
import pytest

import workloads as wl
from parity import gate

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DT = {"f16": 0, "bf16": 1}
ACT = {"none": 0, "relu": 1}


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


def dev(x, dtype=np.uint16) -> "torch.Tensor":
    a = np.ascontiguousarray(np.asarray(x, dtype=dtype).reshape(-1))
    if dtype == np.uint8:
        return torch.from_numpy(a.copy()).to("cuda")
    return torch.from_numpy(a.view(np.int16).copy()).to("cuda")


def host(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def w4_case(tg, oracle_lib, M, N, K, G, dtype="f16", act="relu", bias=False, pad=(0, 0, 0, 0),
            forced=None, seed=0, dist="uniform"):
    """One call against the oracle; pad = extra (lda, ldw bytes, lds, ldc)."""
    lda, ldw, lds, ldc = K + pad[0], K // 2 + pad[1], K // G + pad[2], N + pad[3]
    a, _ = wl.generate_dense(M, 8, K, dist, seed, dtype=dtype)
    a = wl.pad_rows(a, M, K, lda)
    wq, s = wl.generate_w4(N, K, G, seed, dtype=dtype)
    wq_p = np.full((N, ldw), 0x88, np.uint8)                     # padding: -8s
    wq_p[:, :K // 2] = wq.reshape(N, K // 2)
    s_p = np.full((N, lds), 0x7E00, np.uint16)                    # padding: NaN (fp16)
    s_p[:, :K // G] = s.reshape(N, K // G)
    b = wl.generate_bias(N, seed, dtype=dtype) if bias else None
    ref, _, Sa = oracle_lib.gemm_w4(a, wq_p, s_p, M, N, K, G, lda, ldw, lds, ldc, bias=b,
                                    dtype=dtype, act=act, want_sums=True)
    csize = (M - 1) * ldc + N
    if forced is not None:
        assert tg.tg_set_path(forced) >= 0
    a_d, w_d, s_d = dev(a), dev(wq_p, np.uint8), dev(s_p)
    b_d = dev(b) if bias else None
    c_d = dev(np.full(csize + 64, 0x7E00, np.uint16))
    say(f"w4 {dtype} M={M} N={N} K={K} G={G} act={act} bias={bias} pad={pad} forced={forced}")
    st = tg.tg_gemm_w4(DT[dtype], ACT[act], a_d.data_ptr(), w_d.data_ptr(), s_d.data_ptr(),
                       c_d.data_ptr(), b_d.data_ptr() if bias else 0, M, N, K, G, lda, ldw, lds,
                       ldc, torch.cuda.current_stream().cuda_stream)
    assert st == tg.TG_OK, tg.tg_status_string(st)
    torch.cuda.synchronize()
    used = tg.tg_path_name(tg.tg_last_path())
    out = host(c_d)
    assert np.all(out[csize:] == 0x7E00), "wrote past C"
    idx = (np.arange(M)[:, None] * ldc + np.arange(N)[None, :]).reshape(-1)
    win = np.zeros(csize, bool)
    win[idx] = True
    assert np.all(out[:csize][~win] == 0x7E00), "wrote outside the M x N window"
    rep = gate(out[idx], ref[idx], K, Sa.reshape(-1), dtype=dtype, relu=(act == "relu"))
    assert rep.ok, f"{used}: {rep}"
    return used, out[idx]


SHAPES = [(16, 1024, 1024, 128), (1, 64, 256, 32), (7, 200, 512, 64), (33, 520, 768, 256),
          (64, 128, 2048, 128), (100, 256, 512, 128), (16, 256, 384, 128), (16, 256, 96, 32),
          (48, 4096, 512, 64)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("act", ["none", "relu"])
@pytest.mark.parametrize("M,N,K,G", SHAPES)
def test_w4_matches_oracle(tg, oracle_lib, dtype, act, M, N, K, G):
    used, _ = w4_case(tg, oracle_lib, M, N, K, G, dtype=dtype, act=act, bias=(M % 2 == 0),
                      seed=M + N)
    assert used == "w4"


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("M,N,K,G", [(16, 1024, 1024, 128), (5, 130, 96, 32),
                                     (70, 256, 512, 64)])
def test_w4_plain_kernel_matches_oracle(tg, oracle_lib, dtype, M, N, K, G):
    used, _ = w4_case(tg, oracle_lib, M, N, K, G, dtype=dtype, bias=True,
                      forced=tg.TG_PATH_NAIVE, seed=3)
    assert used == "naive"


@pytest.mark.parametrize("M,N,K,G,pad,expect", [
    (16, 512, 1024, 128, (8, 16, 3, 4), "w4"),       # padded, still aligned
    (16, 512, 1024, 128, (1, 0, 0, 0), "naive"),     # lda odd
    (16, 512, 1024, 128, (0, 8, 0, 0), "naive"),     # ldw not a multiple of 16
    (16, 130, 1024, 128, (0, 0, 0, 0), "naive"),     # N % 4 != 0
    (16, 512, 960, 96, (0, 0, 0, 0), "w4"),          # groups of 96 span 256-k steps
    (16, 512, 960, 80, (0, 0, 0, 0), "naive"),       # group size not a multiple of 32
])
def test_w4_layouts(tg, oracle_lib, M, N, K, G, pad, expect):
    used, _ = w4_case(tg, oracle_lib, M, N, K, G, bias=True, pad=pad, seed=5)
    assert used == expect


def test_w4_deterministic_and_matches_dense_path(tg, oracle_lib):
    # power-of-two scales make every dequantized weight an exact fp16 value:
    # the int4 kernel and the dense (N,K) kernel then compute the same exact
    # products; both must pass the gates against the same oracle output
    M, N, K, G = 16, 2048, 2048, 128
    rng = np.random.default_rng(8)
    q = rng.integers(-8, 8, (N, K))
    u = (q & 15).astype(np.uint8)
    wq = (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)
    sv = 2.0 ** rng.integers(-10, -6, (N, K // G)).astype(np.float64)
    s = wl.to_f16_bits(sv)
    wdeq = wl.to_f16_bits(np.repeat(sv, G, axis=1) * q)     # exact: power-of-two scales
    a, _ = wl.generate_dense(M, 8, K, "uniform", 8)
    ref, _, Sa = oracle_lib.gemm_w4(a, wq, s, M, N, K, G, want_sums=True)
    dense_ref = oracle_lib.gemm_ex(a, wdeq, M, N, K, b_layout="nk")
    assert np.array_equal(ref, dense_ref)
    a_d, w_d, s_d, wd_d = dev(a), dev(wq, np.uint8), dev(s), dev(wdeq)
    outs = []
    st_ = torch.cuda.current_stream().cuda_stream
    say("w4 determinism / dense comparison")
    for _ in range(2):
        c = dev(np.zeros(M * N, np.uint16))
        assert tg.tg_gemm_w4(0, 1, a_d.data_ptr(), w_d.data_ptr(), s_d.data_ptr(), c.data_ptr(),
                             0, M, N, K, G, K, K // 2, K // G, N, st_) == tg.TG_OK
        torch.cuda.synchronize()
        outs.append(host(c))
    assert np.array_equal(outs[0], outs[1])
    c = dev(np.zeros(M * N, np.uint16))
    assert tg.tg_gemm_ex(0, tg.TG_B_NK, 1, a_d.data_ptr(), wd_d.data_ptr(), c.data_ptr(), 0, M, N,
                         K, K, K, N, 0, 0, 0, 1, st_) == tg.TG_OK
    torch.cuda.synchronize()
    for o in (outs[0], host(c)):
        rep = gate(o, ref, K, Sa.reshape(-1))
        assert rep.ok, str(rep)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_w4_decode_workload_full_size(tg, oracle_lib, dtype):
    # the decode shape of the benchmark: 16 x 16384 x 8192, groups of 128
    w4_case(tg, oracle_lib, 16, 16384, 8192, 128, dtype=dtype, act="none", bias=True, seed=3,
            dist="uniform_invsqrtk")


def test_w4_k_zero_writes_activation_of_bias(tg, oracle_lib):
    M, N = 3, 64
    b = wl.generate_bias(N, 1)
    b_d = dev(b)
    c = dev(np.full(M * N, 0x7E00, np.uint16))
    dummy = dev(np.zeros(16, np.uint16))
    say("w4 K=0")
    st = tg.tg_gemm_w4(0, 0, dummy.data_ptr(), dummy.data_ptr(), dummy.data_ptr(), c.data_ptr(),
                       b_d.data_ptr(), M, N, 0, 32, 1, 1, 1, N,
                       torch.cuda.current_stream().cuda_stream)
    assert st == tg.TG_OK
    torch.cuda.synchronize()
    want = b.copy()
    want[want == 0x8000] = 0
    assert np.array_equal(host(c).reshape(M, N), np.tile(want, (M, 1)))
