"""GPU parity of the ragged-layout kernel (an aligned A with a (K,N) B and a C
at any 2-byte alignment: odd leading dimensions, N not a multiple of 8, B and
C pointers at 2 mod 4 or 2 mod 16, an unaligned bias) against the oracle,
through the C ABI, for both of its tile configurations.

The kernel accumulates every output with the same 16-wide k steps, in the
same order and through the same matrix-core instruction as the any-layout
kernel, so besides the oracle gates its output must equal that kernel's bit
for bit.  Cells outside the M x N windows hold a sentinel that must survive.
"""

import sys

import numpy as np
import pytest

import workloads as wl
from parity import gate

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SENTINEL = 0x7E00
DTYPES = {"f16": 0, "bf16": 1}


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
def _reset(tg):
    yield
    tg.tg_set_path(tg.TG_PATH_AUTO)
    tg.tg_set_tile_variant(-1)


def dev(bits):
    return torch.from_numpy(np.asarray(bits, np.uint16).view(np.int16).copy()).to("cuda")


def ragged_case(tg, oracle_lib, M, N, K, ldb, ldc, offb=0, offc=0, batch=1, gap=0, act="relu",
                bias_off=None, dtype="f16", seed=0, variant=-1):
    """Runs forced-ragged and forced-generic on the same inputs; returns both
    outputs after gating the ragged one against the oracle (sentinels checked)."""
    lda = K
    sA, sB, sC = M * lda, K * ldb + gap, (M - 1) * ldc + N + gap
    a, b = wl.generate_dense(M, N, K, "uniform", seed, batch=batch, dtype=dtype)
    ab = wl.pad_rows(a, M, K, lda, batch)
    bb = np.full(batch * sB, SENTINEL, np.uint16)
    for t in range(batch):
        bb[t * sB:t * sB + K * ldb] = wl.pad_rows(b[t * K * N:(t + 1) * K * N], K, N, ldb)
    bias = wl.generate_bias(N, seed, dtype) if bias_off is not None else None
    csize = (batch - 1) * sC + (M - 1) * ldc + N
    ref = np.full(csize, SENTINEL, np.uint16)
    ref, S, Sa = oracle_lib.gemm_ex(ab, bb, M, N, K, lda, ldb, ldc, batch, sA, sB, sC, C=ref,
                                    bias=bias, act=act, dtype=dtype, want_sums=True)
    a_d = dev(ab)
    b_d = dev(np.concatenate([np.full(offb, SENTINEL, np.uint16), bb]))
    bias_d = (dev(np.concatenate([np.zeros(bias_off, np.uint16), bias]))
              if bias is not None else None)
    outs = {}
    for path in ("RAGGED", "GENERIC"):
        assert tg.tg_set_path(getattr(tg, "TG_PATH_" + path)) >= 0
        tg.tg_set_tile_variant(variant if path == "RAGGED" else -1)
        c_d = dev(np.full(offc + csize + 40, SENTINEL, np.uint16))
        say(f"ragged {path} {dtype} M={M} N={N} K={K} ldb={ldb} ldc={ldc} off=({offb},{offc}) "
            f"batch={batch} act={act} bias_off={bias_off} variant={variant}")
        st = tg.tg_gemm_ex(DTYPES[dtype], 0, 1 if act == "relu" else 0, a_d.data_ptr(),
                           b_d.data_ptr() + 2 * offb, c_d.data_ptr() + 2 * offc,
                           bias_d.data_ptr() + 2 * bias_off if bias is not None else 0,
                           M, N, K, lda, ldb, ldc, sA, sB, sC, batch,
                           torch.cuda.current_stream().cuda_stream)
        assert st == tg.TG_OK, tg.tg_status_string(st)
        torch.cuda.synchronize()
        used = tg.tg_path_name(tg.tg_last_path())
        assert used == path.lower()
        out = c_d.cpu().numpy().view(np.uint16)
        assert np.all(out[:offc] == SENTINEL) and np.all(out[offc + csize:] == SENTINEL)
        outs[path] = out[offc:offc + csize]
    got = outs["RAGGED"]
    assert np.array_equal(got == SENTINEL, ref == SENTINEL), "wrote outside the windows"
    win = ref != SENTINEL
    rep = gate(got[win], ref[win], K, Sa.reshape(-1), dtype=dtype, relu=(act == "relu"))
    assert rep.ok, str(rep)
    return outs["RAGGED"], outs["GENERIC"]


@pytest.mark.parametrize("variant", [0, 1, 2, 3])
@pytest.mark.parametrize("M,N,K,ldb,ldc,offb,offc", [
    (300, 500, 200, 500, 500, 0, 0),        # N % 8 != 0
    (301, 503, 136, 503, 503, 0, 0),        # odd N, odd ldb / ldc
    (257, 264, 72, 265, 267, 1, 3),         # aligned N, odd strides, pointers at 2 / 6 mod 16
    (520, 392, 1000, 397, 393, 1, 1),       # several K tiles, K tail of 40
    (129, 17, 64, 17, 19, 0, 5),            # one partial chunk column
    (600, 1000, 8, 1001, 1003, 3, 2),       # one 8-deep K tile
    (1, 300, 40, 301, 300, 1, 0),           # one row (forced; auto sends M <= 64 elsewhere)
])
def test_ragged_matches_oracle_and_generic(tg, oracle_lib, variant, M, N, K, ldb, ldc, offb, offc):
    r, g = ragged_case(tg, oracle_lib, M, N, K, ldb, ldc, offb, offc, seed=M + N, variant=variant)
    assert np.array_equal(r, g), f"{int(np.sum(r != g))} outputs differ from the generic kernel"


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("act", ["none", "relu"])
@pytest.mark.parametrize("bias_off", [None, 0, 1])
def test_ragged_modes_and_bias(tg, oracle_lib, dtype, act, bias_off):
    r, g = ragged_case(tg, oracle_lib, 333, 411, 264, 413, 415, 1, 3, act=act, bias_off=bias_off,
                       dtype=dtype, seed=7)
    assert np.array_equal(r, g)


@pytest.mark.parametrize("variant", [0, 1, 2, 3])
def test_ragged_batched_with_gaps(tg, oracle_lib, variant):
    r, g = ragged_case(tg, oracle_lib, 136, 203, 96, 205, 207, 1, 1, batch=3, gap=5,
                       seed=11, variant=variant)
    assert np.array_equal(r, g)


def test_ragged_is_auto_for_the_ragged_workload_shape(tg, oracle_lib):
    # odd ldb / ldc with an aligned A: the automatic choice is the ragged kernel
    M, N, K = 300, 501, 136
    a, b = wl.generate_dense(M, N, K, "uniform", 3)
    # keep the device copies referenced until the kernel has run
    a_d, b_d, c_d = dev(a), dev(b), dev(np.zeros(M * N, np.uint16))
    say("ragged auto")
    st = tg.tg_gemm_relu_f16(a_d.data_ptr(), b_d.data_ptr(), c_d.data_ptr(), M, N, K, K, N,
                             N, torch.cuda.current_stream().cuda_stream)
    assert st == tg.TG_OK
    torch.cuda.synchronize()
    assert tg.tg_path_name(tg.tg_last_path()) == "ragged"
    ref, _, Sa = oracle_lib.gemm_relu(a, b, M, N, K, want_sums=True)
    rep = gate(c_d.cpu().numpy().view(np.uint16), ref, K, Sa.reshape(-1))
    assert rep.ok, str(rep)


def _call(tg, A, B, M, N, K):
    """C = ReLU(A B) on the forced path, dense layouts; returns C's bits."""
    # keep the device copies referenced until the kernel has run
    a_d, b_d = dev(wl.to_f16_bits(A)), dev(wl.to_f16_bits(B))
    c_d = dev(np.zeros(M * N, np.uint16))
    st = tg.tg_gemm_relu_f16(a_d.data_ptr(), b_d.data_ptr(), c_d.data_ptr(), M, N, K, K, N, N,
                             torch.cuda.current_stream().cuda_stream)
    assert st == tg.TG_OK
    torch.cuda.synchronize()
    assert tg.tg_path_name(tg.tg_last_path()) == "ragged"
    return c_d.cpu().numpy().view(np.uint16)


def test_ones_and_probes_exact(tg):
    # closed forms on the ragged kernel: ones -> K, the RNE tie, subnormals
    tg.tg_set_path(tg.TG_PATH_RAGGED)
    say("ragged ones / tie / subnormal")
    M, N, K = 130, 131, 1000
    assert np.all(_call(tg, np.ones((M, K)), np.ones((K, N)), M, N, K) ==
                  np.float16(K).view(np.uint16))
    # tie: 1 + 3 * 2^-11 rounds to even 1 + 2^-9 (0x3c02); N = 9 keeps it ragged
    A = np.zeros((72, 8)); A[:, :3] = 1
    B = np.zeros((8, 9)); B[:3, :] = np.array([1, 2 ** -10, 2 ** -11])[:, None]
    assert np.all(_call(tg, A, B, 72, 9, 8) == 0x3C02)
    # subnormal output 2^-20 from subnormal inputs
    A = np.zeros((72, 16)); A[:16, :16] = np.eye(16) * 2.0 ** -20; A[16:, 0] = 2.0 ** -20
    B = np.ones((16, 9))
    assert np.all(_call(tg, A, B, 72, 9, 16) == 0x0010)
