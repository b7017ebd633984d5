"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every case prints its name, shape and path before touching the GPU so that a
failure names itself.  Inputs come from the seeded generator; expected values
come only from the oracle or from closed forms.
"""

import sys

import numpy as np
import pytest

import workloads as wl
from parity import f16_values, gate

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SENTINEL = 0x7E00   # quiet NaN: cells the kernel must not write


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


def dev(bits: np.ndarray, extra: int = 0) -> "torch.Tensor":
    """Device copy of a uint16 bit array (plus `extra` trailing sentinel cells)."""
    x = np.asarray(bits, dtype=np.uint16).reshape(-1)
    if extra:
        x = np.concatenate([x, np.full(extra, SENTINEL, np.uint16)])
    return torch.from_numpy(x.view(np.int16).copy()).to("cuda")


def host(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def run_gemm(tg, a_d, b_d, c_d, M, N, K, lda, ldb, ldc, offsets=(0, 0, 0)):
    s = torch.cuda.current_stream().cuda_stream
    st = tg.tg_gemm_relu_f16(a_d.data_ptr() + 2 * offsets[0], b_d.data_ptr() + 2 * offsets[1],
                             c_d.data_ptr() + 2 * offsets[2], M, N, K, lda, ldb, ldc, s)
    assert st == tg.TG_OK, tg.tg_status_string(st)
    torch.cuda.synchronize()
    return tg.tg_path_name(tg.tg_last_path())


def run_batched(tg, a_d, b_d, c_d, M, N, K, lda, ldb, ldc, sA, sB, sC, batch):
    s = torch.cuda.current_stream().cuda_stream
    st = tg.tg_gemm_relu_f16_strided_batched(a_d.data_ptr(), b_d.data_ptr(), c_d.data_ptr(), M,
                                             N, K, lda, ldb, ldc, sA, sB, sC, batch, s)
    assert st == tg.TG_OK, tg.tg_status_string(st)
    torch.cuda.synchronize()
    return tg.tg_path_name(tg.tg_last_path())


def full_case(tg, oracle_lib, M, N, K, dist="uniform", seed=0, lda=None, ldb=None, ldc=None,
              path=None, offsets=(0, 0, 0), guard=64):
    lda = K if lda is None else lda
    ldb = N if ldb is None else ldb
    ldc = N if ldc is None else ldc
    a, b = wl.generate_dense(M, N, K, dist, seed)
    a = wl.pad_rows(a, M, K, lda)
    b = wl.pad_rows(b, K, N, ldb)
    csize = (M - 1) * ldc + N
    ref = np.full(csize, SENTINEL, np.uint16)
    ref, S, Sa = oracle_lib.gemm_relu(a, b, M, N, K, lda, ldb, ldc, C=ref, want_sums=True)
    if path is not None:
        assert tg.tg_set_path(path) >= 0
    pre = [np.full(o, SENTINEL, np.uint16) for o in offsets]
    a_d = dev(np.concatenate([pre[0], a]))
    b_d = dev(np.concatenate([pre[1], b]))
    c_d = dev(np.full(offsets[2] + csize + guard, SENTINEL, np.uint16))
    say(f"M={M} N={N} K={K} ld=({lda},{ldb},{ldc}) off={offsets} forced={path}")
    used = run_gemm(tg, a_d, b_d, c_d, M, N, K, lda, ldb, ldc, offsets)
    out = host(c_d)
    assert np.all(out[:offsets[2]] == SENTINEL) and np.all(out[offsets[2] + csize:] == SENTINEL)
    out = out[offsets[2]:offsets[2] + csize]
    win = np.zeros(csize, bool)
    idx = (np.arange(M)[:, None] * ldc + np.arange(N)[None, :]).reshape(-1)
    win[idx] = True
    assert np.all(out[~win] == SENTINEL), "wrote outside the M x N window"
    rep = gate(out[win], ref[win], K, Sa.reshape(-1))
    assert rep.ok, f"{used}: {rep}"
    return used, rep, out[win]


# ------------------------------------------------------------------ parity cases

SHAPES = [
    # (M, N, K) spanning several tiles, with and without ragged tails
    (512, 512, 512),
    (384, 640, 256),
    (257, 264, 136),       # ragged M, N%8 == 0, K tail of 8 in a 32-wide K tile
    (300, 500, 200),       # N % 8 != 0 -> masked path
    (129, 131, 33),        # everything ragged, odd sizes
    (1, 1, 1),
    (7, 9, 5),
    (64, 4096, 1024),      # short and wide
    (2048, 64, 512),       # tall and narrow
]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_auto_path_matches_oracle(tg, oracle_lib, M, N, K):
    full_case(tg, oracle_lib, M, N, K, seed=M + N + K)


FORCED = ["naive", "generic", "tile128", "tile256", "skinny"]


@pytest.mark.parametrize("path", FORCED)
@pytest.mark.parametrize("M,N,K", [(512, 512, 512), (257, 264, 136), (300, 500, 200),
                                   (96, 1024, 64)])
def test_forced_paths_match_oracle(tg, oracle_lib, path, M, N, K):
    used, _, _ = full_case(tg, oracle_lib, M, N, K, seed=3, path=getattr(
        tg, "TG_PATH_" + path.upper()))
    if path == "skinny" and M > 64:
        assert used == ("tile128" if (N % 8 == 0 and K % 8 == 0) else "generic")
    elif (N % 8 == 0 and K % 8 == 0) or path in ("naive", "generic"):
        assert used == path


def test_padded_leading_dims_with_nan_pads(tg, oracle_lib):
    # NaN in the pad columns of A and B must not reach C; ldc padding untouched
    full_case(tg, oracle_lib, 200, 136, 96, lda=104, ldb=144, ldc=152)
    full_case(tg, oracle_lib, 200, 136, 96, lda=101, ldb=139, ldc=141)


def test_unaligned_pointers(tg, oracle_lib):
    used, _, _ = full_case(tg, oracle_lib, 160, 192, 128, offsets=(1, 3, 5))
    assert used == "generic"


@pytest.mark.parametrize("M,N,K", [(512, 512, 512), (3001 // 8, 5003 // 8, 1000 // 8)])
def test_deterministic(tg, oracle_lib, M, N, K):
    a, b = wl.generate_dense(M, N, K, "uniform", 77)
    a_d, b_d = dev(a), dev(b)
    c1 = dev(np.zeros(M * N, np.uint16))
    c2 = dev(np.zeros(M * N, np.uint16))
    say(f"determinism M={M} N={N} K={K}")
    run_gemm(tg, a_d, b_d, c1, M, N, K, K, N, N)
    run_gemm(tg, a_d, b_d, c2, M, N, K, K, N, N)
    assert torch.equal(c1, c2)


# ------------------------------------------------------------- closed forms (bit-exact)


def _bits(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("path", ["auto", "naive", "generic", "tile128", "tile256", "skinny"])
@pytest.mark.parametrize("K", [1000, 2048, 8192])
def test_ones_give_K_exactly(tg, path, K):
    M, N = (64, 256) if path == "skinny" else (256, 256)
    if path != "auto":
        tg.tg_set_path(getattr(tg, "TG_PATH_" + path.upper()))
    a_d = dev(np.full(M * K, 0x3C00, np.uint16))
    b_d = dev(np.full(K * N, 0x3C00, np.uint16))
    c_d = dev(np.zeros(M * N, np.uint16))
    say(f"ones K={K} path={path}")
    run_gemm(tg, a_d, b_d, c_d, M, N, K, K, N, N)
    assert np.all(host(c_d) == _bits(K))
    # and -A gives zero everywhere
    a_d = dev(np.full(M * K, 0xBC00, np.uint16))
    run_gemm(tg, a_d, b_d, c_d, M, N, K, K, N, N)
    assert np.all(host(c_d) == 0)


@pytest.mark.parametrize("path", ["auto", "generic", "tile128", "tile256"])
def test_identity_and_integer_matrices_exact(tg, path):
    if path != "auto":
        tg.tg_set_path(getattr(tg, "TG_PATH_" + path.upper()))
    rng = np.random.default_rng(5)
    n, N = 264, 392
    b = _bits(rng.uniform(-1, 1, (n, N)))
    eye = _bits(np.eye(n))
    c_d = dev(np.zeros(n * N, np.uint16))
    say(f"identity path={path}")
    run_gemm(tg, dev(eye), dev(b), c_d, n, N, n, n, N, N)
    bv = f16_values(b).reshape(-1)
    assert np.array_equal(host(c_d), np.where(bv > 0, b.reshape(-1), 0).astype(np.uint16))
    # integer entries in {-1, 0, 1}: every fp32 partial sum is exact
    M, N, K = 320, 264, 2048
    ai = rng.integers(-1, 2, (M, K))
    bi = rng.integers(-1, 2, (K, N))
    c_d = dev(np.zeros(M * N, np.uint16))
    say(f"integer path={path}")
    run_gemm(tg, dev(_bits(ai)), dev(_bits(bi)), c_d, M, N, K, K, N, N)
    ref = _bits(np.maximum(ai @ bi, 0)).reshape(-1)
    assert np.array_equal(host(c_d), ref)


def _probe(tg, M, N, K, A, B):
    c_d = dev(np.zeros(M * N, np.uint16))
    run_gemm(tg, dev(_bits(A)), dev(_bits(B)), c_d, M, N, K, K, N, N)
    return host(c_d)


@pytest.mark.parametrize("path", ["auto", "naive", "generic", "tile128", "tile256", "skinny"])
def test_rounding_and_subnormal_probes(tg, path):
    if path != "auto":
        tg.tg_set_path(getattr(tg, "TG_PATH_" + path.upper()))
    say(f"probes path={path}")
    # a tie: s = 1 + 3*2^-11 must round to even 1 + 2^-9 (0x3c02), not 0x3c01;
    # padded to K = 8 with zeros so aligned paths serve it
    A = np.zeros((8, 8)); A[:, :3] = 1
    B = np.zeros((8, 8)); B[:3, :] = np.array([1, 2 ** -10, 2 ** -11])[:, None]
    assert np.all(_probe(tg, 8, 8, 8, A, B) == 0x3C02)
    # subnormal inputs and outputs: A = 2^-20 I, B = ones -> C = 2^-20 (0x0010)
    A = np.eye(16) * 2.0 ** -20
    B = np.ones((16, 16))
    assert np.all(_probe(tg, 16, 16, 16, A, B) == 0x0010)
    # overflow to +inf, and the largest finite value
    A = np.zeros((8, 8)); A[:, :2] = [256, 256]
    B = np.zeros((8, 8)); B[:2, :] = np.array([256, 1])[:, None]
    assert np.all(_probe(tg, 8, 8, 8, A, B) == 0x7C00)
    A = np.zeros((8, 8)); A[:, :2] = [255, 1]
    B = np.zeros((8, 8)); B[:2, :] = np.array([256, 224])[:, None]
    assert np.all(_probe(tg, 8, 8, 8, A, B) == 0x7BFF)
    # a negative sum stores +0 (not -0)
    A = np.zeros((8, 8)); A[:, :2] = [1, -2]
    B = np.zeros((8, 8)); B[:2, :] = 1
    assert np.all(_probe(tg, 8, 8, 8, A, B) == 0x0000)


def test_k_zero_writes_zero_and_empty_is_noop(tg):
    c_d = dev(np.full(64 * 8, SENTINEL, np.uint16))
    say("K=0")
    s = torch.cuda.current_stream().cuda_stream
    assert tg.tg_gemm_relu_f16(0, 0, c_d.data_ptr(), 60, 8, 0, 1, 8, 8, s) == tg.TG_OK
    torch.cuda.synchronize()
    out = host(c_d)
    assert np.all(out[:480] == 0) and np.all(out[480:] == SENTINEL)
    assert tg.tg_gemm_relu_f16(0, 0, c_d.data_ptr(), 0, 8, 4, 4, 8, 8, s) == tg.TG_OK
    torch.cuda.synchronize()
    assert np.all(host(c_d)[:480] == 0)


# ------------------------------------------------------------------ batched


@pytest.mark.parametrize("path", ["auto", "generic", "tile128"])
def test_strided_batched_matches_oracle(tg, oracle_lib, path):
    if path != "auto":
        tg.tg_set_path(getattr(tg, "TG_PATH_" + path.upper()))
    M, N, K, bt = 136, 200, 72, 5
    a, b = wl.generate_dense(M, N, K, "uniform", 31, batch=bt)
    sA, sB, sC = M * K + 8, K * N + 16, M * N + 24
    ab = np.full(bt * sA, SENTINEL, np.uint16)
    bb = np.full(bt * sB, SENTINEL, np.uint16)
    for i in range(bt):
        ab[i * sA:i * sA + M * K] = a[i * M * K:(i + 1) * M * K]
        bb[i * sB:i * sB + K * N] = b[i * K * N:(i + 1) * K * N]
    ref = np.full(bt * sC, SENTINEL, np.uint16)
    ref, S, Sa = oracle_lib.gemm_relu(ab, bb, M, N, K, batch=bt, sA=sA, sB=sB, sC=sC, C=ref,
                                      want_sums=True)
    c_d = dev(np.full(bt * sC, SENTINEL, np.uint16))
    say(f"batched path={path}")
    run_batched(tg, dev(ab), dev(bb), c_d, M, N, K, K, N, N, sA, sB, sC, bt)
    out = host(c_d)
    assert np.array_equal(out == SENTINEL, ref == SENTINEL)
    win = ref != SENTINEL
    rep = gate(out[win], ref[win], K, Sa.reshape(-1))
    assert rep.ok, str(rep)


def test_strided_batched_broadcast_operand(tg, oracle_lib):
    M, N, K, bt = 64, 72, 48, 6
    a, b = wl.generate_dense(M, N, K, "uniform", 32, batch=bt)
    b1 = b[:K * N]
    ref, S, Sa = oracle_lib.gemm_relu(a, b1, M, N, K, batch=bt, sB=0, want_sums=True)
    c_d = dev(np.zeros(bt * M * N, np.uint16))
    say("batched broadcast B")
    run_batched(tg, dev(a), dev(b1), c_d, M, N, K, K, N, N, M * K, 0, M * N, bt)
    rep = gate(host(c_d), ref, K, Sa.reshape(-1))
    assert rep.ok, str(rep)


# ------------------------------------------- full-size workloads (every output)


def _workload_case(tg, oracle_lib, name, n_samples=None):
    w = wl.WORKLOADS[name]
    a, b = wl.generate(w)
    a_d, b_d = dev(a), dev(b)
    csize = (w.batch - 1) * w.sC + (w.M - 1) * w.ldc_ + w.N
    c_d = dev(np.full(csize + 64, SENTINEL, np.uint16))
    say(f"workload {name}")
    if w.batch == 1:
        used = run_gemm(tg, a_d, b_d, c_d, w.M, w.N, w.K, w.lda_, w.ldb_, w.ldc_)
    else:
        used = run_batched(tg, a_d, b_d, c_d, w.M, w.N, w.K, w.lda_, w.ldb_, w.ldc_, w.sA, w.sB,
                           w.sC, w.batch)
    out = host(c_d)
    assert np.all(out[csize:] == SENTINEL)
    out = out[:csize]
    if n_samples is None:
        ref, S, Sa = oracle_lib.gemm_relu(a, b, w.M, w.N, w.K, w.lda_, w.ldb_, w.ldc_, w.batch,
                                          w.sA, w.sB, w.sC, want_sums=True)
        rep = gate(out, ref, w.K, Sa.reshape(-1))
    else:
        idx = wl.sample_positions(w, n_samples)
        ref, s, sa = oracle_lib.gemm_relu_sampled(a, b, w.K, w.lda_, w.ldb_, idx, w.sA, w.sB)
        got = out[idx[:, 0] * w.sC + idx[:, 1] * w.ldc_ + idx[:, 2]]
        rep = gate(got, ref, w.K, sa)
        # properties that hold at any size, checked on every output
        assert not np.any(out & 0x8000), "negative output"
        assert not np.any((out & 0x7C00) == 0x7C00), "non-finite output"
    say(f"workload {name} path={used} {rep}")
    assert rep.ok, f"{used}: {rep}"


@pytest.mark.parametrize("name,n", [
    ("small_512", None),
    ("mid_2048", None),
    ("large_8192", None),
    ("skinny_16x16384x8192", None),
    ("ragged_3001x5003x1000", None),
    ("batched_1024x128x128x64", None),
])
def test_workloads_full_size(tg, oracle_lib, name, n):
    _workload_case(tg, oracle_lib, name, n)


# ------------------------------------------------------ every tile configuration

VARIANTS = list(range(43)) + [100, 101]


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("M,N,K", [(257, 264, 136), (520, 392, 1000), (64, 256, 8)])
def test_tile_variants_match_oracle(tg, oracle_lib, variant, M, N, K):
    assert tg.tg_set_tile_variant(variant) >= -1
    try:
        used, _, _ = full_case(tg, oracle_lib, M, N, K, seed=variant + 11,
                               path=tg.TG_PATH_TILE256)
        assert used == "tile256"
    finally:
        tg.tg_set_tile_variant(-1)


@pytest.mark.parametrize("path,M,N,K", [("TG_PATH_TILE256", 1000, 1032, 264),
                                         ("TG_PATH_TILE128", 1000, 1032, 264),
                                         ("TG_PATH_GENERIC", 1001, 1003, 263)])
def test_raster_orders_are_bitwise_identical(tg, oracle_lib, path, M, N, K):
    """Every tile order computes each tile the same way: the outputs of all
    raster settings agree bit for bit (and with the oracle)."""
    outs = []
    try:
        for g in (8, 0, 1, 3, 64):
            assert tg.tg_set_raster(g) >= 0
            used, _, out = full_case(tg, oracle_lib, M, N, K, seed=77,
                                     path=getattr(tg, path))
            outs.append(out)
    finally:
        tg.tg_set_raster(-1)
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


# ------------------------------------------------------------------ skinny M


@pytest.mark.parametrize("variant", [0, 1, 2, 3, 4, 5, 6, 7, 8, 9])
@pytest.mark.parametrize("M,N,K", [(16, 1024, 8192), (1, 264, 520), (7, 1000, 136),
                                   (17, 512, 1000), (33, 96, 64), (64, 520, 2056),
                                   (48, 8, 8)])
def test_skinny_variants_match_oracle(tg, oracle_lib, variant, M, N, K):
    assert tg.tg_set_skinny_variant(variant) >= -1
    try:
        used, _, _ = full_case(tg, oracle_lib, M, N, K, dist="uniform", seed=variant + M,
                               path=tg.TG_PATH_SKINNY)
        assert used == "skinny"
    finally:
        tg.tg_set_skinny_variant(-1)


def test_skinny_is_auto_for_small_m(tg, oracle_lib):
    used, _, _ = full_case(tg, oracle_lib, 16, 4096, 4096, seed=5)
    assert used == "skinny"
    used, _, _ = full_case(tg, oracle_lib, 65, 512, 256, seed=6)
    assert used != "skinny"


# ------------------------------------------------------------ random shapes


def _random_case(rng):
    """Random small strided-batched problem: sizes 1..300 with a bias towards
    tile edges, aligned or not, padded leading dimensions, a few batches."""
    def dim(hi):
        r = rng.random()
        if r < 0.3:
            return int(rng.integers(1, 17))
        if r < 0.6:
            base = int(rng.choice([32, 64, 128, 256]))
            return max(1, base + int(rng.integers(-2, 3)))
        return int(rng.integers(1, hi))
    M, N, K = dim(300), dim(300), dim(300)
    if rng.random() < 0.5:      # aligned layouts (fast paths)
        N = (N + 7) // 8 * 8
        K = (K + 7) // 8 * 8
        lda = K + 8 * int(rng.integers(0, 3))
        ldb = N + 8 * int(rng.integers(0, 3))
        ldc = N + 8 * int(rng.integers(0, 3))
    else:
        lda = K + int(rng.integers(0, 5))
        ldb = N + int(rng.integers(0, 5))
        ldc = N + int(rng.integers(0, 5))
    batch = int(rng.choice([1, 1, 2, 3]))
    return M, N, K, lda, ldb, ldc, batch


@pytest.mark.parametrize("seed", range(40))
def test_random_shapes_match_oracle(tg, oracle_lib, seed):
    rng = np.random.default_rng(9000 + seed)
    M, N, K, lda, ldb, ldc, batch = _random_case(rng)
    sA = M * lda + 8 * int(rng.integers(0, 2))
    sB = K * ldb + 8 * int(rng.integers(0, 2))
    sC = (M - 1) * ldc + N + 8 * int(rng.integers(0, 3))
    a, b = wl.generate_dense(M, N, K, "uniform", seed, batch=batch)
    ab = np.full(batch * sA, SENTINEL, np.uint16)
    bb = np.full(batch * sB, SENTINEL, np.uint16)
    for i in range(batch):
        ab[i * sA:i * sA + M * lda] = wl.pad_rows(a[i * M * K:(i + 1) * M * K], M, K, lda)
        bb[i * sB:i * sB + K * ldb] = wl.pad_rows(b[i * K * N:(i + 1) * K * N], K, N, ldb)
    csize = (batch - 1) * sC + (M - 1) * ldc + N
    ref = np.full(csize + 32, SENTINEL, np.uint16)
    ref, S, Sa = oracle_lib.gemm_relu(ab, bb, M, N, K, lda, ldb, ldc, batch, sA, sB, sC, C=ref,
                                      want_sums=True)
    c_d = dev(np.full(csize + 32, SENTINEL, np.uint16))
    say(f"random seed={seed} M={M} N={N} K={K} ld=({lda},{ldb},{ldc}) batch={batch} "
        f"strides=({sA},{sB},{sC})")
    used = run_batched(tg, dev(ab), dev(bb), c_d, M, N, K, lda, ldb, ldc, sA, sB, sC, batch)
    out = host(c_d)
    assert np.array_equal(out == SENTINEL, ref == SENTINEL), f"{used}: wrote outside the windows"
    win = ref != SENTINEL
    rep = gate(out[win], ref[win], K, Sa.reshape(-1))
    assert rep.ok, f"{used}: {rep}"
