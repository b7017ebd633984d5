"""Race check for the hand-scheduled pipelines: configurations that accumulate
every output in the same order must agree bit for bit.

The tile kernels place their own counter waits and barriers where a tile
compiler would infer them from the copy / GEMM dependencies ("TileLang paper
reading", section 3).  A stage read before its loads have landed, or
overwritten while a wave still reads it, changes some products; the oracle
gate, with its tolerance, can miss a slip confined to a few outputs.

Every configuration with one K group feeds each 32 x 32 output fragment the
same 16-wide k steps in ascending order through the same matrix-core
instruction with the same operand roles (C^T = B^T A^T), whatever its block
tile, K tile, stage count, swizzle, wave grid or whether loads go through
registers or straight to LDS; trailing zero steps add exact zeros.  So their
outputs must be bitwise identical, and the same holds inside each group of
two-K-group configurations that deal the same K tiles to each group.  The
configurations built on 16x16x32 products (32-wide k steps) are in the same
set: on this part a 32-wide product step gives the bits of its two 16-wide
halves taken in order, which this test checks along with the races.  The
comparison runs without the activation, so negative outputs are compared too.
One output of each set is gated against the oracle.
"""

import sys

import numpy as np
import pytest

import workloads as wl
from parity import gate

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DTYPES = {"f16": 0, "bf16": 1}
LAYOUTS = {"kn": 0, "nk": 1}

# one K group (any tile / stages / swizzle / waves / product shape), the
# register-staged kernels (and, below, the any-layout and ragged-layout kernels)
KG1 = [c for c in range(43) if c not in (14, 15, 16, 20)] + [100, 101]
# two K groups: K tiles of 64 (configs 14, 20) or of 32 (15, 16) dealt alternately
KG2_GROUPS = [[14, 20], [15, 16]]
# configurations that exist for bf16 elements and an (N,K) B
MODE_KG1 = [8, 29, 12, 32, 34, 36, 38, 39, 41]
# persistent configurations (a workgroup walks a list of tiles, its ring of K
# tiles running across tile boundaries) and one-tile-per-workgroup ones
STREAM = [35, 36, 37, 39]
ONE_SHOT = [12, 34, 38]


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


def dev(bits) -> "torch.Tensor":
    x = np.asarray(bits, dtype=np.uint16).reshape(-1)
    return torch.from_numpy(x.view(np.int16).copy()).to("cuda")


def run(tg, a_d, b_d, M, N, K, dtype, layout, path, variant):
    """One call of tg_gemm_ex without activation on a forced path/config."""
    assert tg.tg_set_path(path) >= 0
    assert tg.tg_set_tile_variant(variant) >= -1
    ldb = N if layout == "kn" else K
    c_d = torch.zeros(M * N, dtype=torch.int16, device="cuda")
    say(f"race {dtype}/{layout} M={M} N={N} K={K} path={path} variant={variant}")
    st = tg.tg_gemm_ex(DTYPES[dtype], LAYOUTS[layout], 0, a_d.data_ptr(), b_d.data_ptr(),
                       c_d.data_ptr(), 0, M, N, K, K, ldb, N, 0, 0, 0, 1,
                       torch.cuda.current_stream().cuda_stream)
    assert st == tg.TG_OK, tg.tg_status_string(st)
    torch.cuda.synchronize()
    return c_d.cpu().numpy().view(np.uint16), tg.tg_path_name(tg.tg_last_path())


def operands(M, N, K, seed, dtype, layout):
    a, b = wl.generate_dense(M, N, K, "uniform", seed, dtype=dtype)
    if layout == "nk":
        b = wl.transpose_bits(b, K, N)
    return a, b


def check_against_oracle(oracle_lib, out, a, b, M, N, K, dtype, layout):
    ref, S, Sa = oracle_lib.gemm_ex(a, b, M, N, K, dtype=dtype, b_layout=layout, act="none",
                                    want_sums=True)
    rep = gate(out, ref, K, Sa.reshape(-1), dtype=dtype, relu=False)
    assert rep.ok, str(rep)


def assert_same(outs, ref_key):
    ref = outs[ref_key]
    bad = {k: int(np.sum(v != ref)) for k, v in outs.items() if not np.array_equal(v, ref)}
    assert not bad, f"outputs differing from {ref_key} (count of differing elements): {bad}"


SHAPES = [(520, 392, 1000), (2048, 2048, 2048), (257, 264, 136), (384, 256, 40), (264, 392, 440)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_one_k_group_configs_bitwise_identical(tg, oracle_lib, M, N, K):
    a, b = operands(M, N, K, 101 + K, "f16", "kn")
    a_d, b_d = dev(a), dev(b)
    outs = {}
    for v in KG1:
        outs[v], used = run(tg, a_d, b_d, M, N, K, "f16", "kn", tg.TG_PATH_TILE256, v)
        assert used == "tile256"
    outs["generic"], used = run(tg, a_d, b_d, M, N, K, "f16", "kn", tg.TG_PATH_GENERIC, -1)
    assert used == "generic"
    for v in (0, 1, 2, 3):
        outs[f"ragged{v}"], used = run(tg, a_d, b_d, M, N, K, "f16", "kn", tg.TG_PATH_RAGGED, v)
        assert used == "ragged"
    check_against_oracle(oracle_lib, outs[8], a, b, M, N, K, "f16", "kn")
    assert_same(outs, 8)


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("group", KG2_GROUPS)
def test_two_k_group_configs_bitwise_identical(tg, oracle_lib, M, N, K, group):
    a, b = operands(M, N, K, 201 + K, "f16", "kn")
    a_d, b_d = dev(a), dev(b)
    outs = {}
    for v in group:
        outs[v], used = run(tg, a_d, b_d, M, N, K, "f16", "kn", tg.TG_PATH_TILE256, v)
        assert used == "tile256"
    check_against_oracle(oracle_lib, outs[group[0]], a, b, M, N, K, "f16", "kn")
    assert_same(outs, group[0])


@pytest.mark.parametrize("dtype,layout", [("bf16", "kn"), ("f16", "nk"), ("bf16", "nk")])
@pytest.mark.parametrize("M,N,K", [(520, 392, 1000), (257, 264, 136)])
def test_modes_bitwise_identical_across_configs(tg, oracle_lib, dtype, layout, M, N, K):
    a, b = operands(M, N, K, 301 + K, dtype, layout)
    a_d, b_d = dev(a), dev(b)
    outs = {}
    for v in MODE_KG1:
        outs[v], used = run(tg, a_d, b_d, M, N, K, dtype, layout, tg.TG_PATH_TILE256, v)
        assert used == "tile256"
    outs["generic"], used = run(tg, a_d, b_d, M, N, K, dtype, layout, tg.TG_PATH_GENERIC, -1)
    assert used == "generic"
    check_against_oracle(oracle_lib, outs[8], a, b, M, N, K, dtype, layout)
    assert_same(outs, 8)


def run_batched(tg, a_d, b_d, M, N, K, batch, sA, sB, dtype, layout, variant, bias_d=None,
                act=0):
    """One strided-batched call of tg_gemm_ex on the 128x128 tile path."""
    assert tg.tg_set_path(tg.TG_PATH_TILE128) >= 0
    assert tg.tg_set_tile_variant(variant) >= -1
    ldb = N if layout == "kn" else K
    c_d = torch.full((batch * M * N,), 0x7E00, dtype=torch.int16, device="cuda")
    say(f"stream race {dtype}/{layout} batch={batch} M={M} N={N} K={K} sB={sB} "
        f"variant={variant} bias={bias_d is not None} act={act}")
    st = tg.tg_gemm_ex(DTYPES[dtype], LAYOUTS[layout], act, a_d.data_ptr(), b_d.data_ptr(),
                       c_d.data_ptr(), bias_d.data_ptr() if bias_d is not None else 0, M, N, K,
                       K, ldb, N, sA, sB, M * N, batch, torch.cuda.current_stream().cuda_stream)
    assert st == tg.TG_OK, tg.tg_status_string(st)
    torch.cuda.synchronize()
    return c_d.cpu().numpy().view(np.uint16), tg.tg_path_name(tg.tg_last_path())


# batch, M, N, K, B shared by every entry: more tiles than workgroups (several
# per workgroup, items not a multiple of the grid), K tiles per item from 1 to
# 4 with a partial last one, ragged M and N edges
STREAM_SHAPES = [(1024, 128, 128, 64, False), (600, 130, 136, 200, False),
                 (9, 1000, 1000, 64, False), (300, 64, 256, 8, True), (1, 2056, 1032, 264, False)]


@pytest.mark.parametrize("batch,M,N,K,shared_b", STREAM_SHAPES)
def test_stream_configs_bitwise_identical(tg, oracle_lib, batch, M, N, K, shared_b):
    """The persistent configurations give the bits of the one-tile-per-workgroup
    ones for every tile of every batch entry (a stage reused too early, or a
    tile's epilogue given another tile's coordinates, would show here)."""
    a, b = wl.generate_dense(M, N, K, "uniform", 401 + K, batch=batch)
    if shared_b:
        b = b[:K * N]
    a_d, b_d = dev(a), dev(b)
    sB = 0 if shared_b else K * N
    outs = {}
    for v in ONE_SHOT + STREAM:
        outs[v], used = run_batched(tg, a_d, b_d, M, N, K, batch, M * K, sB, "f16", "kn", v)
        assert used == "tile128"
    for v in STREAM:
        assert not np.any(outs[v] == 0x7E00), f"configuration {v}: a cell of C was not written"
    for e in sorted({0, batch // 2, batch - 1}):
        out = outs[36].reshape(batch, M * N)[e]
        ref, S, Sa = oracle_lib.gemm_ex(a[e * M * K:(e + 1) * M * K],
                                        b[(e * K * N if not shared_b else 0):][:K * N], M, N, K,
                                        act="none", want_sums=True)
        rep = gate(out, ref, K, Sa.reshape(-1), relu=False)
        assert rep.ok, f"batch entry {e}: {rep}"
    assert_same(outs, 34)


@pytest.mark.parametrize("dtype,layout", [("f16", "kn"), ("bf16", "kn"), ("f16", "nk"),
                                          ("bf16", "nk")])
@pytest.mark.parametrize("act,with_bias", [(1, False), (1, True), (0, True)])
def test_stream_modes_and_epilogues_match_one_shot(tg, dtype, layout, act, with_bias):
    """Element types, B layouts, bias and activation on the persistent
    configuration: the same bits as the one-tile-per-workgroup one."""
    batch, M, N, K = 700, 72, 136, 96
    a, b = wl.generate_dense(M, N, K, "uniform", 7 + act, batch=batch, dtype=dtype)
    if layout == "nk":
        b = wl.transpose_bits(b, K, N, batch)
    a_d, b_d = dev(a), dev(b)
    bias_d = dev(wl.generate_bias(N, 9, dtype=dtype, scale=0.5)) if with_bias else None
    o34, u34 = run_batched(tg, a_d, b_d, M, N, K, batch, M * K, K * N, dtype, layout, 34,
                           bias_d, act)
    for v in (36, 39):
        o, u = run_batched(tg, a_d, b_d, M, N, K, batch, M * K, K * N, dtype, layout, v, bias_d,
                           act)
        assert u34 == u == "tile128"
        assert not np.any(o == 0x7E00), f"configuration {v}: a cell of C was not written"
        assert np.array_equal(o34, o), (v, int(np.sum(o34 != o)))
