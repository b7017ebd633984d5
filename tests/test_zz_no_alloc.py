"""The allocation-free split-K entry point against the workspace one.

tg_gemm_relu_f16_splitk_noalloc runs the same kernels as
tg_gemm_relu_f16_splitk with the partial sums in the library's own per-device
scratch array; both are called through the C ABI (ctypes on libtg.so) on the
same inputs and must agree bit for bit, and both must pass the oracle gates.
Two calls in a row, the second with a smaller input, check that what the
first call left in the scratch array does not leak into the second.  Sizes
beyond the scratch array are refused on the host, before any GPU work.
"""

import ctypes
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
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiled_dense_gemm_05_amd as tg
    cl = ctypes.CDLL(tg.LIB_PATH)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    cl.tg_gemm_relu_f16_splitk_noalloc.argtypes = [vp] * 3 + [i64] * 7 + [vp]
    cl.tg_gemm_relu_f16_splitk_noalloc.restype = ctypes.c_int
    cl.tg_gemm_relu_f16_splitk.argtypes = [vp] * 3 + [i64] * 7 + [vp, i64, vp]
    cl.tg_gemm_relu_f16_splitk.restype = ctypes.c_int
    return cl, tg


def dev(bits):
    return torch.from_numpy(np.asarray(bits, np.uint16).view(np.int16).copy()).to("cuda")


def both(lib, M, N, K, splits, seed):
    cl, tg = lib
    a, b = wl.generate_dense(M, N, K, "uniform_invsqrtk", seed)
    a_d, b_d = dev(a), dev(b)
    c_ws = torch.zeros(M * N, dtype=torch.int16, device="cuda")
    c_na = torch.full((M * N,), 0x7E00, dtype=torch.int16, device="cuda")
    need = tg.tg_gemm_splitk_workspace_bytes(M, N, splits)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    say(f"noalloc M={M} N={N} K={K} splits={splits} seed={seed}")
    st = cl.tg_gemm_relu_f16_splitk(a_d.data_ptr(), b_d.data_ptr(), c_ws.data_ptr(), M, N, K, K,
                                    N, N, splits, ws.data_ptr(), need, s)
    assert st == tg.TG_OK, tg.tg_status_string(st)
    st = cl.tg_gemm_relu_f16_splitk_noalloc(a_d.data_ptr(), b_d.data_ptr(), c_na.data_ptr(), M,
                                            N, K, K, N, N, splits, s)
    assert st == tg.TG_OK, tg.tg_status_string(st)
    torch.cuda.synchronize()
    return a, b, c_ws.cpu().numpy().view(np.uint16), c_na.cpu().numpy().view(np.uint16)


def test_matches_workspace_entry_point_on_two_calls(lib, oracle_lib):
    # first call fills most of the scratch array, the second is smaller
    for (M, N, K, splits, seed) in [(16, 16384, 8192, 8, 61), (5, 264, 1000, 3, 62)]:
        a, b, c_ws, c_na = both(lib, M, N, K, splits, seed)
        assert np.array_equal(c_na, c_ws), f"differs in {int(np.sum(c_na != c_ws))} outputs"
        ref, _, sa = oracle_lib.gemm_relu(a, b, M, N, K, want_sums=True)
        rep = gate(c_na, ref, K, sa.reshape(-1))
        assert rep.ok, str(rep)


def test_largest_and_oversized_requests(lib):
    cl, tg = lib
    limit = tg.TG_SPLITK_NOALLOC_SCRATCH_BYTES
    # exactly the scratch size: 16 x 16384 x 4 bytes x 16 chunks
    a, b, c_ws, c_na = both(lib, 16, 16384, 4096, 16, 63)
    assert 16 * 16384 * 4 * 16 == limit
    assert np.array_equal(c_na, c_ws)
    # one chunk more is refused on the host before any GPU work (the CPU tests
    # check the same refusal without a device)
    s = torch.cuda.current_stream().cuda_stream
    a_d = torch.zeros(16 * 4096, dtype=torch.int16, device="cuda")
    b_d = torch.zeros(4096 * 16384, dtype=torch.int16, device="cuda")
    c_d = torch.zeros(16 * 16384, dtype=torch.int16, device="cuda")
    st = cl.tg_gemm_relu_f16_splitk_noalloc(a_d.data_ptr(), b_d.data_ptr(), c_d.data_ptr(), 16,
                                            16384, 4096, 4096, 16384, 16384, 17, s)
    assert st == tg.TG_ERR_INVALID_ARG
    # empty problems are no-ops
    assert cl.tg_gemm_relu_f16_splitk_noalloc(0, 0, 0, 0, 16, 64, 64, 16, 16, 1, s) == tg.TG_OK
