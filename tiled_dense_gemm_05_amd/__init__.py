"""Python binding of the MI355X fused fp16 GEMM + ReLU library (``libtg.so``).

Argument marshalling only: every step of C = ReLU(A·B) runs in the HIP kernels
behind the C ABI declared in ``include/tg.h``.  The functions named like the
C entry points take raw device pointers and sizes; ``gemm_relu`` and
``gemm_relu_strided_batched`` accept torch tensors (torch provides device
memory and streams only).  There is no fallback: if the library is not built,
importing this package raises.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtg.so")

TG_OK = 0
TG_ERR_INVALID_ARG = 1
TG_ERR_NO_DEVICE = 2
TG_ERR_UNSUPPORTED_DEVICE = 3
TG_ERR_HIP = 4

TG_PATH_AUTO = 0
TG_PATH_NAIVE = 1
TG_PATH_GENERIC = 2
TG_PATH_TILE128 = 3
TG_PATH_TILE256 = 4
TG_PATH_SKINNY = 5
TG_PATH_W4 = 6
TG_PATH_ATTENTION = 7
TG_PATH_MLA = 8
TG_PATH_RAGGED = 9
TG_PATH_COUNT = 10

EXPORTED_SYMBOLS = (
    "tg_gemm_relu_f16",
    "tg_gemm_relu_f16_strided_batched",
    "tg_status_string",
    "tg_set_path",
    "tg_last_path",
    "tg_path_name",
    "tg_set_tile_variant",
    "tg_set_skinny_variant",
    "tg_set_raster",
    "tg_gemm_ex",
    "tg_gemm_w4",
    "tg_attention_fwd_f16",
    "tg_attention_fwd_f16_gqa",
    "tg_set_attention_variant",
    "tg_mla_decode_f16",
    "tg_mla_decode_workspace_bytes",
    "tg_set_mla_splits",
    "tg_gemm_relu_f16_splitk",
    "tg_gemm_splitk_workspace_bytes",
    "tg_gemm_relu_f16_splitk_noalloc",
)

TG_DTYPE_F16 = 0
TG_DTYPE_BF16 = 1
TG_B_KN = 0
TG_B_NK = 1
TG_ACT_NONE = 0
TG_ACT_RELU = 1


class TGError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(tg_status_string(status))


if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python tiled_dense_gemm_05_amd/build.py` "
        "(there is no CPU fallback)")

_lib = ctypes.CDLL(LIB_PATH)
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_lib.tg_gemm_relu_f16.argtypes = [_vp, _vp, _vp] + [_i64] * 6 + [_vp]
_lib.tg_gemm_relu_f16.restype = ctypes.c_int
_lib.tg_gemm_relu_f16_strided_batched.argtypes = [_vp, _vp, _vp] + [_i64] * 10 + [_vp]
_lib.tg_gemm_relu_f16_strided_batched.restype = ctypes.c_int
_lib.tg_gemm_ex.argtypes = [ctypes.c_int] * 3 + [_vp] * 4 + [_i64] * 10 + [_vp]
_lib.tg_gemm_ex.restype = ctypes.c_int
_lib.tg_gemm_w4.argtypes = [ctypes.c_int] * 2 + [_vp] * 5 + [_i64] * 8 + [_vp]
_lib.tg_gemm_w4.restype = ctypes.c_int
_lib.tg_attention_fwd_f16.argtypes = [_vp] * 4 + [_i64] * 5 + [ctypes.c_float, ctypes.c_int, _vp]
_lib.tg_attention_fwd_f16.restype = ctypes.c_int
_lib.tg_attention_fwd_f16_gqa.argtypes = [_vp] * 4 + [_i64] * 6 + [ctypes.c_float, ctypes.c_int,
                                                                 _vp]
_lib.tg_attention_fwd_f16_gqa.restype = ctypes.c_int
_lib.tg_set_attention_variant.argtypes = [ctypes.c_int]
_lib.tg_set_attention_variant.restype = ctypes.c_int
_lib.tg_mla_decode_f16.argtypes = [_vp] * 4 + [_i64] * 3 + [ctypes.c_float, _vp, _i64, _vp]
_lib.tg_mla_decode_f16.restype = ctypes.c_int
_lib.tg_mla_decode_workspace_bytes.argtypes = [_i64] * 3
_lib.tg_mla_decode_workspace_bytes.restype = ctypes.c_int64
_lib.tg_set_mla_splits.argtypes = [ctypes.c_int]
_lib.tg_set_mla_splits.restype = ctypes.c_int
_lib.tg_gemm_relu_f16_splitk.argtypes = [_vp] * 3 + [_i64] * 7 + [_vp, _i64, _vp]
_lib.tg_gemm_relu_f16_splitk.restype = ctypes.c_int
_lib.tg_gemm_splitk_workspace_bytes.argtypes = [_i64] * 3
_lib.tg_gemm_splitk_workspace_bytes.restype = ctypes.c_int64
_lib.tg_gemm_relu_f16_splitk_noalloc.argtypes = [_vp] * 3 + [_i64] * 7 + [_vp]
_lib.tg_gemm_relu_f16_splitk_noalloc.restype = ctypes.c_int

TG_SPLITK_NOALLOC_SCRATCH_BYTES = 16 << 20
_lib.tg_status_string.argtypes = [ctypes.c_int]
_lib.tg_status_string.restype = ctypes.c_char_p
_lib.tg_set_path.argtypes = [ctypes.c_int]
_lib.tg_set_path.restype = ctypes.c_int
_lib.tg_last_path.argtypes = []
_lib.tg_last_path.restype = ctypes.c_int
_lib.tg_set_tile_variant.argtypes = [ctypes.c_int]
_lib.tg_set_tile_variant.restype = ctypes.c_int
_lib.tg_set_skinny_variant.argtypes = [ctypes.c_int]
_lib.tg_set_skinny_variant.restype = ctypes.c_int
_lib.tg_set_raster.argtypes = [ctypes.c_int]
_lib.tg_set_raster.restype = ctypes.c_int
_lib.tg_path_name.argtypes = [ctypes.c_int]
_lib.tg_path_name.restype = ctypes.c_char_p


# ----------------------------------------------------------- C-ABI mirror


def tg_gemm_relu_f16(A: int, B: int, C: int, M: int, N: int, K: int, lda: int, ldb: int,
                     ldc: int, stream: int = 0) -> int:
    """Raw call: device pointers as ints, returns the tg_status code."""
    return _lib.tg_gemm_relu_f16(A, B, C, M, N, K, lda, ldb, ldc, stream)


def tg_gemm_relu_f16_strided_batched(A: int, B: int, C: int, M: int, N: int, K: int, lda: int,
                                     ldb: int, ldc: int, strideA: int, strideB: int,
                                     strideC: int, batch: int, stream: int = 0) -> int:
    """Raw strided-batched call, returns the tg_status code."""
    return _lib.tg_gemm_relu_f16_strided_batched(A, B, C, M, N, K, lda, ldb, ldc, strideA,
                                                 strideB, strideC, batch, stream)


def tg_gemm_ex(dtype: int, b_layout: int, activation: int, A: int, B: int, C: int, bias: int,
               M: int, N: int, K: int, lda: int, ldb: int, ldc: int, strideA: int, strideB: int,
               strideC: int, batch: int, stream: int = 0) -> int:
    """Raw extended call (bias may be 0 for none), returns the tg_status code."""
    return _lib.tg_gemm_ex(dtype, b_layout, activation, A, B, C, bias or None, M, N, K, lda, ldb,
                           ldc, strideA, strideB, strideC, batch, stream)


def tg_gemm_w4(dtype: int, activation: int, A: int, Wq: int, scales: int, C: int, bias: int,
               M: int, N: int, K: int, group_size: int, lda: int, ldw: int, lds: int, ldc: int,
               stream: int = 0) -> int:
    """Raw weight-only int4 call (bias may be 0 for none), returns the tg_status code."""
    return _lib.tg_gemm_w4(dtype, activation, A, Wq, scales, C, bias or None, M, N, K,
                           group_size, lda, ldw, lds, ldc, stream)


def tg_attention_fwd_f16(Q: int, K: int, V: int, O: int, batch: int, seq_q: int, seq_k: int,
                         heads: int, head_dim: int, scale: float, causal: int,
                         stream: int = 0) -> int:
    """Raw attention-forward call, returns the tg_status code."""
    return _lib.tg_attention_fwd_f16(Q, K, V, O, batch, seq_q, seq_k, heads, head_dim, scale,
                                     causal, stream)


def tg_attention_fwd_f16_gqa(Q: int, K: int, V: int, O: int, batch: int, seq_q: int, seq_k: int,
                             heads: int, kv_heads: int, head_dim: int, scale: float, causal: int,
                             stream: int = 0) -> int:
    """Raw grouped-query attention-forward call (K and V hold kv_heads heads), returns the
    tg_status code."""
    return _lib.tg_attention_fwd_f16_gqa(Q, K, V, O, batch, seq_q, seq_k, heads, kv_heads,
                                         head_dim, scale, causal, stream)


def tg_mla_decode_f16(Q: int, KV: int, O: int, seqlens: int, batch: int, heads: int,
                      seq_k: int, scale: float, workspace: int, workspace_bytes: int,
                      stream: int = 0) -> int:
    """Raw latent-attention decode call (seqlens and workspace may be 0 for none), returns the
    tg_status code."""
    return _lib.tg_mla_decode_f16(Q, KV, O, seqlens or None, batch, heads, seq_k, scale,
                                  workspace or None, workspace_bytes, stream)


def tg_mla_decode_workspace_bytes(batch: int, heads: int, seq_k: int) -> int:
    return _lib.tg_mla_decode_workspace_bytes(batch, heads, seq_k)


def tg_set_mla_splits(splits: int) -> int:
    return _lib.tg_set_mla_splits(splits)


def tg_gemm_relu_f16_splitk(A: int, B: int, C: int, M: int, N: int, K: int, lda: int, ldb: int,
                            ldc: int, splits: int, workspace: int, workspace_bytes: int,
                            stream: int = 0) -> int:
    """Raw split-K skinny call, returns the tg_status code."""
    return _lib.tg_gemm_relu_f16_splitk(A, B, C, M, N, K, lda, ldb, ldc, splits,
                                        workspace or None, workspace_bytes, stream)


def tg_gemm_splitk_workspace_bytes(M: int, N: int, splits: int) -> int:
    return _lib.tg_gemm_splitk_workspace_bytes(M, N, splits)


def tg_gemm_relu_f16_splitk_noalloc(A: int, B: int, C: int, M: int, N: int, K: int, lda: int,
                                    ldb: int, ldc: int, splits: int, stream: int = 0) -> int:
    """Raw allocation-free split-K call (library-owned scratch), returns the
    tg_status code."""
    return _lib.tg_gemm_relu_f16_splitk_noalloc(A, B, C, M, N, K, lda, ldb, ldc, splits,
                                                stream)


def tg_status_string(status: int) -> str:
    return _lib.tg_status_string(status).decode()


def tg_set_path(path: int) -> int:
    return _lib.tg_set_path(path)


def tg_last_path() -> int:
    return _lib.tg_last_path()


def tg_path_name(path: int) -> str:
    return _lib.tg_path_name(path).decode()


def tg_set_tile_variant(variant: int) -> int:
    return _lib.tg_set_tile_variant(variant)


def tg_set_skinny_variant(variant: int) -> int:
    return _lib.tg_set_skinny_variant(variant)


def tg_set_attention_variant(variant: int) -> int:
    return _lib.tg_set_attention_variant(variant)


def tg_set_raster(group_m: int) -> int:
    return _lib.tg_set_raster(group_m)


# ----------------------------------------------------------- torch helpers


def _check(status: int) -> None:
    if status != TG_OK:
        raise TGError(status)


def _stream_handle(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _row_major_2d(t, name):
    import torch
    if t.dtype != torch.float16:
        raise TypeError(f"{name} must be float16")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if t.stride(1) != 1 and t.size(1) > 1:
        raise ValueError(f"{name} must have unit column stride (row-major)")
    return max(t.stride(0), 1)


def gemm_relu(A, B, out=None, stream=None):
    """C = ReLU(A @ B) for 2-D fp16 device tensors with unit column stride.

    ``out`` (optional) is an (M, N) fp16 tensor with unit column stride; its
    leading dimension is taken from its row stride.  Enqueued on ``stream``
    (default: torch's current stream); returns ``out``.
    """
    import torch
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError(f"inner sizes differ: {tuple(A.shape)} @ {tuple(B.shape)}")
    lda = _row_major_2d(A, "A") if M and K else max(K, 1)
    ldb = _row_major_2d(B, "B") if K and N else max(N, 1)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=A.device)
    ldc = _row_major_2d(out, "out") if M and N else max(N, 1)
    if tuple(out.shape) != (M, N):
        raise ValueError("out has the wrong shape")
    _check(tg_gemm_relu_f16(A.data_ptr(), B.data_ptr(), out.data_ptr(), M, N, K,
                            max(lda, K, 1), max(ldb, N, 1), max(ldc, N, 1),
                            _stream_handle(stream)))
    return out


def gemm_relu_strided_batched(A, B, out=None, stream=None):
    """C[b] = ReLU(A[b] @ B[b]) for 3-D fp16 device tensors (batch, rows, cols)
    with unit column stride; batch strides come from the tensors' strides (a
    stride of 0, e.g. from ``expand``, shares one operand across the batch)."""
    import torch
    bt, M, K = A.shape
    bt2, K2, N = B.shape
    if bt2 != bt or K2 != K:
        raise ValueError(f"shapes do not match: {tuple(A.shape)} @ {tuple(B.shape)}")
    if out is None:
        out = torch.empty((bt, M, N), dtype=torch.float16, device=A.device)
    for t, name in ((A, "A"), (B, "B"), (out, "out")):
        if t.dtype != torch.float16:
            raise TypeError(f"{name} must be float16")
        if t.stride(2) != 1 and t.size(2) > 1:
            raise ValueError(f"{name} must have unit column stride")
    _check(tg_gemm_relu_f16_strided_batched(
        A.data_ptr(), B.data_ptr(), out.data_ptr(), M, N, K,
        max(A.stride(1), K, 1), max(B.stride(1), N, 1), max(out.stride(1), N, 1),
        A.stride(0), B.stride(0), out.stride(0), bt, _stream_handle(stream)))
    return out


def gemm_ex(A, B, bias=None, activation="relu", b_layout="kn", out=None, stream=None):
    """C = act(A @ B' + bias) through tg_gemm_ex for 2-D device tensors.

    A is (M, K); B is (K, N) for ``b_layout="kn"`` or (N, K) for "nk" (then
    B' = B^T, as a linear layer's weight); both float16 or both bfloat16 with
    unit column stride; ``bias`` (optional) is a contiguous 1-D tensor of N
    elements of the same type; ``activation`` is "relu" or "none".  ``out``
    (optional) is an (M, N) tensor of that type with unit column stride.
    Enqueued on ``stream`` (default: torch's current stream); returns ``out``.
    """
    import torch
    dtypes = {torch.float16: TG_DTYPE_F16, torch.bfloat16: TG_DTYPE_BF16}
    if A.dtype not in dtypes or B.dtype != A.dtype:
        raise TypeError("A and B must both be float16 or both bfloat16")
    if A.dim() != 2 or B.dim() != 2:
        raise ValueError("A and B must be 2-D")
    acts = {"relu": TG_ACT_RELU, "none": TG_ACT_NONE}
    layouts = {"kn": TG_B_KN, "nk": TG_B_NK}
    if activation not in acts or b_layout not in layouts:
        raise ValueError("activation is 'relu' or 'none'; b_layout is 'kn' or 'nk'")
    M, K = A.shape
    N, K2 = (B.shape[1], B.shape[0]) if b_layout == "kn" else (B.shape[0], B.shape[1])
    if K2 != K:
        raise ValueError(f"inner sizes differ: {tuple(A.shape)} and {tuple(B.shape)} ({b_layout})")
    for t, name in ((A, "A"), (B, "B")):
        if t.numel() and t.stride(1) != 1 and t.size(1) > 1:
            raise ValueError(f"{name} must have unit column stride (row-major)")
    if bias is not None:
        if bias.dtype != A.dtype or bias.dim() != 1 or bias.numel() != N or \
                (N > 1 and bias.stride(0) != 1):
            raise ValueError("bias must be a contiguous 1-D tensor of N elements of A's type")
    if out is None:
        out = torch.empty((M, N), dtype=A.dtype, device=A.device)
    if tuple(out.shape) != (M, N) or out.dtype != A.dtype:
        raise ValueError("out has the wrong shape or type")
    if out.numel() and out.stride(1) != 1 and out.size(1) > 1:
        raise ValueError("out must have unit column stride")
    inner = K if b_layout == "nk" else N
    _check(tg_gemm_ex(dtypes[A.dtype], layouts[b_layout], acts[activation], A.data_ptr(),
                      B.data_ptr(), out.data_ptr(), bias.data_ptr() if bias is not None else 0,
                      M, N, K, max(A.stride(0), K, 1), max(B.stride(0), inner, 1),
                      max(out.stride(0), N, 1), 0, 0, 0, 1, _stream_handle(stream)))
    return out


def linear(x, weight, bias=None, activation="none", out=None, stream=None):
    """A linear layer, x @ weight^T + bias, with an optional fused ReLU: x is
    (M, K), weight (N, K) (the (N,K) B layout), bias N elements."""
    return gemm_ex(x, weight, bias=bias, activation=activation, b_layout="nk", out=out,
                   stream=stream)


MLA_DL, MLA_DR = 512, 64


def mla_decode(q, kv, scale, seqlens=None, out=None, workspace=None, stream=None):
    """Latent-attention decode through tg_mla_decode_f16: q (B, H, 576) and the
    cache kv (B, Sk, 576) fp16 device tensors, contiguous; returns O (B, H, 512).
    seqlens: optional int32 device tensor of B visible lengths.  The workspace
    (a uint8 device tensor) is allocated here when not given."""
    import torch
    if q.dtype != torch.float16 or kv.dtype != torch.float16:
        raise TypeError("q and kv must be float16")
    if q.dim() != 3 or kv.dim() != 3 or q.shape[2] != MLA_DL + MLA_DR or \
            kv.shape[2] != MLA_DL + MLA_DR or kv.shape[0] != q.shape[0]:
        raise ValueError("q must be (B, H, 576) and kv (B, Sk, 576)")
    if not q.is_contiguous() or not kv.is_contiguous():
        raise ValueError("q and kv must be contiguous")
    B, H, Sk = q.shape[0], q.shape[1], kv.shape[1]
    sl = 0
    if seqlens is not None:
        if seqlens.dtype != torch.int32 or seqlens.numel() != B or not seqlens.is_contiguous():
            raise ValueError("seqlens must be a contiguous int32 tensor of B entries")
        sl = seqlens.data_ptr()
    if out is None:
        out = torch.empty((B, H, MLA_DL), dtype=torch.float16, device=q.device)
    if tuple(out.shape) != (B, H, MLA_DL) or out.dtype != torch.float16 or not out.is_contiguous():
        raise ValueError("out must be a contiguous (B, H, 512) float16 tensor")
    need = tg_mla_decode_workspace_bytes(B, H, Sk)
    if need < 0:
        raise ValueError("sizes out of range")
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws, wsb = (workspace.data_ptr(), workspace.numel()) if workspace is not None else (0, 0)
    _check(tg_mla_decode_f16(q.data_ptr(), kv.data_ptr(), out.data_ptr(), sl, B, H, Sk,
                             float(scale), ws, wsb, _stream_handle(stream)))
    return out
