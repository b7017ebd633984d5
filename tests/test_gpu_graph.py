"""The entry points inside a captured HIP graph: they allocate nothing and only
enqueue kernels on the caller's stream, so a graph captured around them
replays the same work.  Each graph is replayed several times, with eager work
(clearing the outputs) and synchronisations between the replays, and every
replay must reproduce the eager result bit for bit."""

import math
import sys

import numpy as np
import pytest

import workloads as wl

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


def dev(bits) -> "torch.Tensor":
    x = np.asarray(bits, dtype=np.uint16).reshape(-1)
    return torch.from_numpy(x.view(np.int16).copy()).to("cuda")


def replay_matches(call, out, replays=3):
    """Runs call() eagerly, captures it, then replays it `replays` times."""
    call(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for r in range(replays):
        out.zero_()
        torch.cuda.synchronize()
        assert not torch.equal(out, eager) or not eager.any()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r} differs from the eager result"


@pytest.mark.parametrize("M,N,K", [(512, 512, 512), (16, 4096, 8192), (300, 500, 200)])
def test_gemm_relu_in_a_graph(tg, M, N, K):
    a, b = wl.generate_dense(M, N, K, "uniform", M + N)
    A, B = dev(a), dev(b)
    C = torch.empty(M * N, dtype=torch.int16, device="cuda")
    say(f"graph gemm {M}x{N}x{K}")

    def call(s):
        assert tg.tg_gemm_relu_f16(A.data_ptr(), B.data_ptr(), C.data_ptr(), M, N, K, K, N, N,
                                   s) == tg.TG_OK

    replay_matches(call, C)


def test_mla_decode_with_key_ranges_in_a_graph(tg):
    B, H, Sk = 2, 128, 3000
    rng = np.random.default_rng(80_000)
    q = np.asarray(rng.normal(0, 1, B * H * 576)).astype(np.float16).view(np.uint16)
    kv = np.asarray(rng.normal(0, 1, B * Sk * 576)).astype(np.float16).view(np.uint16)
    Q, KV = dev(q), dev(kv)
    O = torch.empty(B * H * 512, dtype=torch.int16, device="cuda")
    need = tg.tg_mla_decode_workspace_bytes(B, H, Sk)
    assert need > 0   # the two-kernel form with partials
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    lens = torch.tensor([3000, 1234], dtype=torch.int32, device="cuda")
    say("graph mla decode")

    def call(s):
        assert tg.tg_mla_decode_f16(Q.data_ptr(), KV.data_ptr(), O.data_ptr(), lens.data_ptr(), B,
                                    H, Sk, 1.0 / math.sqrt(192), ws.data_ptr(), need,
                                    s) == tg.TG_OK

    replay_matches(call, O)


def test_split_k_in_a_graph(tg):
    M, N, K, S = 16, 2048, 4096, 4
    a, b = wl.generate_dense(M, N, K, "uniform", 9)
    A, B = dev(a), dev(b)
    C = torch.empty(M * N, dtype=torch.int16, device="cuda")
    need = tg.tg_gemm_splitk_workspace_bytes(M, N, S)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    say("graph split-K")

    def call(s):
        assert tg.tg_gemm_relu_f16_splitk(A.data_ptr(), B.data_ptr(), C.data_ptr(), M, N, K, K, N,
                                          N, S, ws.data_ptr(), need, s) == tg.TG_OK

    replay_matches(call, C)
