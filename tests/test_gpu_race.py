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
KG1 = [c for c in range(35) if c not in (14, 15, 16, 20)] + [100, 101]
# two K groups: K tiles of 64 (configs 14, 20) or of 32 (15, 16) dealt alternately
KG2_GROUPS = [[14, 20], [15, 16]]
# configurations that exist for bf16 elements and an (N,K) B
MODE_KG1 = [8, 29, 12, 32, 34]


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


SHAPES = [(520, 392, 1000), (2048, 2048, 2048), (257, 264, 136), (384, 256, 40)]


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
