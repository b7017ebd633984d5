"""CPU oracle for C = ReLU(A·B) with fp16 storage (binary64 accumulation),
and for its variants C = act(A·B + bias) with fp16 or bf16 storage and B
stored as (K,N) or (N,K).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It shares no code with the HIP
library under ``tiled_dense_gemm_05_amd`` and never imports it.

The arithmetic lives in ``gemm_relu_oracle.c`` and ``attention_oracle.c``
(attention, grouped-query attention and the latent-attention decode)
(plain C, compiled with gcc,
no BLAS, no SIMD intrinsics, no fast-math); this module only builds it, loads it
with ctypes and marshals numpy arrays.  What it computes, and the passages it
follows, are stated at the top of the C file: the matmul_relu tile program in
section 2 of the "TileLang paper reading" page (hotelren.com) and the serial,
fp32-or-wider K accumulation in section 3.2 of the "tilelang practitioner's
notes" page (dpshk.com).

Every fp16 / bf16 array here is passed as its raw bit patterns
(``numpy.uint16``).
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gemm_relu_oracle.c")
_SRC_ATTN = os.path.join(_HERE, "attention_oracle.c")
_LIB = os.path.join(_HERE, "_build", "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/_build/liboracle.so``."""
    if not force and os.path.exists(_LIB):
        return _LIB
    os.makedirs(os.path.dirname(_LIB), exist_ok=True)
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-std=c11",
           "-D_GNU_SOURCE", "-fPIC", "-shared", "-o", tmp, _SRC, _SRC_ATTN, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    i64 = ctypes.c_int64
    vp = ctypes.c_void_p
    lib.oracle_dec16_array.argtypes = [vp, vp, i64]
    lib.oracle_dec16_array.restype = None
    lib.oracle_enc16_array.argtypes = [vp, vp, i64]
    lib.oracle_enc16_array.restype = None
    lib.oracle_relu_store_array.argtypes = [vp, vp, i64]
    lib.oracle_relu_store_array.restype = None
    lib.oracle_gemm_relu_f16.argtypes = [vp, vp, vp] + [i64] * 10 + [vp, vp, ctypes.c_int]
    lib.oracle_gemm_relu_f16.restype = ctypes.c_int
    lib.oracle_gemm_relu_f16_sampled.argtypes = [vp, vp] + [i64] * 5 + [vp, i64, vp, vp, vp,
                                                                        ctypes.c_int]
    lib.oracle_gemm_relu_f16_sampled.restype = ctypes.c_int
    lib.oracle_decbf16_array.argtypes = [vp, vp, i64]
    lib.oracle_decbf16_array.restype = None
    lib.oracle_encbf16_array.argtypes = [vp, vp, i64]
    lib.oracle_encbf16_array.restype = None
    ci = ctypes.c_int
    lib.oracle_gemm_ex.argtypes = [ci, ci, ci, vp, vp, vp, vp] + [i64] * 10 + [vp, vp, ci]
    lib.oracle_gemm_ex.restype = ctypes.c_int
    lib.oracle_gemm_ex_sampled.argtypes = [ci, ci, ci, vp, vp, vp] + [i64] * 5 + [vp, i64, vp,
                                                                                  vp, vp, ci]
    lib.oracle_gemm_ex_sampled.restype = ctypes.c_int
    lib.oracle_s4_decode_array.argtypes = [vp, vp, vp, i64]
    lib.oracle_s4_decode_array.restype = None
    lib.oracle_gemm_w4.argtypes = [ci, ci, vp, vp, vp, vp, vp] + [i64] * 8 + [vp, vp, ci]
    lib.oracle_gemm_w4.restype = ctypes.c_int
    lib.oracle_attention_f16.argtypes = [vp] * 4 + [i64] * 5 + [ctypes.c_double, ci, vp, vp, ci]
    lib.oracle_attention_f16.restype = ctypes.c_int
    lib.oracle_attention_gqa_f16.argtypes = [vp] * 4 + [i64] * 6 + [ctypes.c_double, ci, vp, vp,
                                                                    ci]
    lib.oracle_attention_gqa_f16.restype = ctypes.c_int
    lib.oracle_mla_decode_f16.argtypes = [vp] * 4 + [i64] * 5 + [ctypes.c_double, vp, vp, ci]
    lib.oracle_mla_decode_f16.restype = ctypes.c_int
    _lib = lib
    return lib


def host_threads() -> int:
    """Threads the oracle uses by default: the CPUs this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError("fp16 operands are passed as uint16 bit patterns")
    return a


def dec16(bits) -> np.ndarray:
    """Exact binary16 -> binary64 decode of an array of bit patterns."""
    b = _u16(bits)
    out = np.empty(b.shape, dtype=np.float64)
    _load().oracle_dec16_array(_ptr(b), _ptr(out), b.size)
    return out


def enc16(x) -> np.ndarray:
    """binary64 -> binary16 bit patterns, round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_enc16_array(_ptr(x), _ptr(out), x.size)
    return out


def decbf16(bits) -> np.ndarray:
    """Exact bfloat16 -> binary64 decode of an array of bit patterns."""
    b = _u16(bits)
    out = np.empty(b.shape, dtype=np.float64)
    _load().oracle_decbf16_array(_ptr(b), _ptr(out), b.size)
    return out


def encbf16(x) -> np.ndarray:
    """binary64 -> bfloat16 bit patterns, round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_encbf16_array(_ptr(x), _ptr(out), x.size)
    return out


def relu_store(x) -> np.ndarray:
    """ReLU (s if s > 0 else +0) followed by the fp16 store, on binary64 sums."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_relu_store_array(_ptr(x), _ptr(out), x.size)
    return out


def _check_extent(buf: np.ndarray, rows: int, cols: int, ld: int, stride: int, batch: int,
                  name: str) -> None:
    if rows == 0 or cols == 0 or batch == 0:
        return
    need = (batch - 1) * stride + (rows - 1) * ld + cols
    if buf.size < need:
        raise ValueError(f"{name} holds {buf.size} elements, layout needs {need}")


def gemm_relu(A, B, M: int, N: int, K: int, lda: int | None = None, ldb: int | None = None,
              ldc: int | None = None, batch: int = 1, sA: int | None = None,
              sB: int | None = None, sC: int | None = None, C=None, want_sums: bool = False,
              threads: int | None = None):
    """Every output of C = ReLU(A·B), strided-batched.

    A, B: flat uint16 arrays (fp16 bits) in the row-major layouts given by
    lda / ldb and the batch strides sA / sB (elements).  C, if given, is a flat
    uint16 array updated in place inside the M×N windows only; otherwise a new
    one of (batch-1)*sC + (M-1)*ldc + N elements is returned.
    With ``want_sums`` also returns the binary64 sums s and Σ|A_ik·B_kj|, each
    shaped (batch, M, N).
    """
    lda = K if lda is None else lda
    ldb = N if ldb is None else ldb
    ldc = N if ldc is None else ldc
    sA = M * lda if sA is None else sA
    sB = K * ldb if sB is None else sB
    sC = M * ldc if sC is None else sC
    A = _u16(A).reshape(-1)
    B = _u16(B).reshape(-1)
    if M > 0 and N > 0:
        _check_extent(A, M, K, lda, sA, batch, "A")
        _check_extent(B, K, N, ldb, sB, batch, "B")
    if C is None:
        size = 0 if (M == 0 or N == 0 or batch == 0) else (batch - 1) * sC + (M - 1) * ldc + N
        C = np.zeros(size, dtype=np.uint16)
    else:
        if C.dtype != np.uint16 or not C.flags.c_contiguous:
            raise TypeError("C must be a contiguous uint16 array")
        C = C.reshape(-1)
    _check_extent(C, M, N, ldc, sC, batch, "C")
    S = Sa = None
    if want_sums:
        S = np.zeros((batch, M, N), dtype=np.float64)
        Sa = np.zeros((batch, M, N), dtype=np.float64)
    rc = _load().oracle_gemm_relu_f16(
        _ptr(A), _ptr(B), _ptr(C), M, N, K, lda, ldb, ldc, sA, sB, sC, batch,
        _ptr(S) if S is not None else None, _ptr(Sa) if Sa is not None else None,
        host_threads() if threads is None else threads)
    if rc != 0:
        raise MemoryError("oracle ran out of memory")
    if want_sums:
        return C, S, Sa
    return C


def gemm_relu_sampled(A, B, K: int, lda: int, ldb: int, idx, sA: int = 0, sB: int = 0,
                      threads: int | None = None):
    """Outputs at chosen positions: idx is an (n, 3) int array of (b, i, j).

    Returns (c_bits uint16[n], s float64[n], abs_sum float64[n]).  The caller
    guarantees the positions lie inside the operands' layouts.
    """
    A = _u16(A).reshape(-1)
    B = _u16(B).reshape(-1)
    idx = np.ascontiguousarray(np.asarray(idx, dtype=np.int64).reshape(-1, 3))
    n = idx.shape[0]
    if n:
        bmax, imax, jmax = idx.max(axis=0)
        if idx.min() < 0:
            raise ValueError("negative index")
        if K > 0:
            if bmax * sA + imax * lda + K > A.size:
                raise ValueError("sample outside A")
            if bmax * sB + (K - 1) * ldb + jmax >= B.size:
                raise ValueError("sample outside B")
    out = np.zeros(n, dtype=np.uint16)
    s = np.zeros(n, dtype=np.float64)
    sa = np.zeros(n, dtype=np.float64)
    _load().oracle_gemm_relu_f16_sampled(
        _ptr(A), _ptr(B), K, lda, ldb, sA, sB, _ptr(idx), n, _ptr(out), _ptr(s), _ptr(sa),
        host_threads() if threads is None else threads)
    return out, s, sa


DTYPES = {"f16": 0, "bf16": 1}
B_LAYOUTS = {"kn": 0, "nk": 1}
ACTS = {"none": 0, "relu": 1}


def gemm_ex(A, B, M: int, N: int, K: int, lda: int | None = None, ldb: int | None = None,
            ldc: int | None = None, batch: int = 1, sA: int | None = None,
            sB: int | None = None, sC: int | None = None, C=None, bias=None,
            dtype: str = "f16", b_layout: str = "kn", act: str = "relu",
            want_sums: bool = False, threads: int | None = None):
    """Every output of C = act(A·B + bias), strided-batched.

    As ``gemm_relu``, plus: ``dtype`` "f16" or "bf16" (the element type of A,
    B, bias and C, all passed as uint16 bit patterns); ``b_layout`` "kn" (B
    is (K,N) row-major, B(k,j) at k*ldb + j) or "nk" (B is (N,K) row-major,
    B(k,j) at j*ldb + k); ``act`` "none" or "relu"; ``bias`` None or N values
    added to every row before the activation.  The sums returned with
    ``want_sums`` include the bias.
    """
    layout = B_LAYOUTS[b_layout]
    lda = K if lda is None else lda
    ldb = (N if layout == 0 else K) if ldb is None else ldb
    ldc = N if ldc is None else ldc
    sA = M * lda if sA is None else sA
    sB = (K * ldb if layout == 0 else N * ldb) if sB is None else sB
    sC = M * ldc if sC is None else sC
    A = _u16(A).reshape(-1)
    B = _u16(B).reshape(-1)
    if M > 0 and N > 0:
        _check_extent(A, M, K, lda, sA, batch, "A")
        if layout == 0:
            _check_extent(B, K, N, ldb, sB, batch, "B")
        else:
            _check_extent(B, N, K, ldb, sB, batch, "B")
    if bias is not None:
        bias = _u16(bias).reshape(-1)
        if bias.size < N:
            raise ValueError(f"bias holds {bias.size} values, N = {N}")
    if C is None:
        size = 0 if (M == 0 or N == 0 or batch == 0) else (batch - 1) * sC + (M - 1) * ldc + N
        C = np.zeros(size, dtype=np.uint16)
    else:
        if C.dtype != np.uint16 or not C.flags.c_contiguous:
            raise TypeError("C must be a contiguous uint16 array")
        C = C.reshape(-1)
    _check_extent(C, M, N, ldc, sC, batch, "C")
    S = Sa = None
    if want_sums:
        S = np.zeros((batch, M, N), dtype=np.float64)
        Sa = np.zeros((batch, M, N), dtype=np.float64)
    rc = _load().oracle_gemm_ex(
        DTYPES[dtype], layout, ACTS[act], _ptr(A), _ptr(B), _ptr(C),
        _ptr(bias) if bias is not None else None, M, N, K, lda, ldb, ldc, sA, sB, sC, batch,
        _ptr(S) if S is not None else None, _ptr(Sa) if Sa is not None else None,
        host_threads() if threads is None else threads)
    if rc != 0:
        raise MemoryError("oracle ran out of memory") if rc == -1 else ValueError("bad mode")
    if want_sums:
        return C, S, Sa
    return C


def gemm_ex_sampled(A, B, K: int, lda: int, ldb: int, idx, sA: int = 0, sB: int = 0,
                    bias=None, dtype: str = "f16", b_layout: str = "kn", act: str = "relu",
                    threads: int | None = None):
    """``gemm_relu_sampled`` for the variants of ``gemm_ex``."""
    layout = B_LAYOUTS[b_layout]
    A = _u16(A).reshape(-1)
    B = _u16(B).reshape(-1)
    idx = np.ascontiguousarray(np.asarray(idx, dtype=np.int64).reshape(-1, 3))
    n = idx.shape[0]
    if n:
        bmax, imax, jmax = idx.max(axis=0)
        if idx.min() < 0:
            raise ValueError("negative index")
        if K > 0:
            if bmax * sA + imax * lda + K > A.size:
                raise ValueError("sample outside A")
            last = (K - 1) * ldb + jmax if layout == 0 else jmax * ldb + K - 1
            if bmax * sB + last >= B.size:
                raise ValueError("sample outside B")
        if bias is not None and jmax >= np.asarray(bias).size:
            raise ValueError("sample outside bias")
    if bias is not None:
        bias = _u16(bias).reshape(-1)
    out = np.zeros(n, dtype=np.uint16)
    s = np.zeros(n, dtype=np.float64)
    sa = np.zeros(n, dtype=np.float64)
    _load().oracle_gemm_ex_sampled(
        DTYPES[dtype], layout, ACTS[act], _ptr(A), _ptr(B),
        _ptr(bias) if bias is not None else None, K, lda, ldb, sA, sB, _ptr(idx), n, _ptr(out),
        _ptr(s), _ptr(sa), host_threads() if threads is None else threads)
    return out, s, sa


def s4_decode(packed) -> tuple[np.ndarray, np.ndarray]:
    """Signed values (-8..7) of the low and high nibbles of each byte."""
    b = np.ascontiguousarray(packed, dtype=np.uint8)
    lo = np.empty(b.shape, dtype=np.int8)
    hi = np.empty(b.shape, dtype=np.int8)
    _load().oracle_s4_decode_array(_ptr(b), _ptr(lo), _ptr(hi), b.size)
    return lo, hi


def gemm_w4(A, Wq, S, M: int, N: int, K: int, G: int, lda: int | None = None,
            ldw: int | None = None, lds: int | None = None, ldc: int | None = None, C=None,
            bias=None, dtype: str = "f16", act: str = "relu", want_sums: bool = False,
            threads: int | None = None):
    """C = act(A · W + bias) with W(k, n) = S[n*lds + k//G] * q(n, k), q the
    signed nibble k%2 of byte Wq[n*ldw + k//2] (see the C source).  A, S,
    bias, C are uint16 bit patterns of ``dtype``; Wq is uint8.  Sums come
    back shaped (M, N)."""
    lda = K if lda is None else lda
    ldw = (K + 1) // 2 if ldw is None else ldw
    lds = (K + G - 1) // G if lds is None else lds
    ldc = N if ldc is None else ldc
    A = _u16(A).reshape(-1)
    S = _u16(S).reshape(-1)
    Wq = np.ascontiguousarray(Wq, dtype=np.uint8).reshape(-1)
    if M > 0 and N > 0:
        _check_extent(A, M, K, lda, 0, 1, "A")
        if K > 0:
            if Wq.size < (N - 1) * ldw + (K + 1) // 2:
                raise ValueError("Wq too small")
            if S.size < (N - 1) * lds + (K - 1) // G + 1:
                raise ValueError("S too small")
    if bias is not None:
        bias = _u16(bias).reshape(-1)
        if bias.size < N:
            raise ValueError("bias too small")
    if C is None:
        C = np.zeros(0 if (M == 0 or N == 0) else (M - 1) * ldc + N, dtype=np.uint16)
    C = C.reshape(-1)
    _check_extent(C, M, N, ldc, 0, 1, "C")
    Sm = Sa = None
    if want_sums:
        Sm = np.zeros((M, N), dtype=np.float64)
        Sa = np.zeros((M, N), dtype=np.float64)
    rc = _load().oracle_gemm_w4(
        DTYPES[dtype], ACTS[act], _ptr(A), _ptr(Wq), _ptr(S), _ptr(C),
        _ptr(bias) if bias is not None else None, M, N, K, G, lda, ldw, lds, ldc,
        _ptr(Sm) if Sm is not None else None, _ptr(Sa) if Sa is not None else None,
        host_threads() if threads is None else threads)
    if rc != 0:
        raise MemoryError("oracle ran out of memory") if rc == -1 else ValueError("bad mode")
    if want_sums:
        return C, Sm, Sa
    return C


def attention(Q, K, V, B: int, Sq: int, Sk: int, H: int, D: int, scale: float,
              causal: bool = False, want_stats: bool = False, threads: int | None = None,
              kv_heads: int | None = None):
    """softmax(scale * Q K^T) V per (batch, head), fp16 bits; Q and O laid out
    (batch, seq, heads, head_dim), K and V (batch, seq, kv_heads, head_dim)
    with query head h reading key/value head h // (heads // kv_heads)
    (kv_heads defaults to heads); with ``causal`` key j is visible to query i
    when j <= i + (Sk - Sq).  Returns O (uint16, B*Sq*H*D) and, with
    ``want_stats``, each query's row maximum and sum of exponentials, shaped
    (B, H, Sq)."""
    Hkv = H if kv_heads is None else kv_heads
    Q = _u16(Q).reshape(-1)
    K = _u16(K).reshape(-1)
    V = _u16(V).reshape(-1)
    for name, t, n in (("Q", Q, B * Sq * H * D), ("K", K, B * Sk * Hkv * D),
                       ("V", V, B * Sk * Hkv * D)):
        if t.size < n:
            raise ValueError(f"{name} holds {t.size} elements, needs {n}")
    O = np.zeros(B * Sq * H * D, dtype=np.uint16)
    mx = sm = None
    if want_stats:
        mx = np.zeros((B, H, Sq), dtype=np.float64)
        sm = np.zeros((B, H, Sq), dtype=np.float64)
    rc = _load().oracle_attention_gqa_f16(
        _ptr(Q), _ptr(K), _ptr(V), _ptr(O), B, Sq, Sk, H, Hkv, D, float(scale), int(causal),
        _ptr(mx) if mx is not None else None, _ptr(sm) if sm is not None else None,
        host_threads() if threads is None else threads)
    if rc != 0:
        raise ValueError("bad attention sizes")
    if want_stats:
        return O, mx, sm
    return O


def mla_decode(Q, KV, B: int, H: int, Sk: int, scale: float, seqlens=None, Dl: int = 512,
               Dr: int = 64, want_stats: bool = False, threads: int | None = None):
    """Latent-attention decode, fp16 bits: Q (B, H, Dl + Dr), the cache KV
    (B, Sk, Dl + Dr) whose first Dl values per token are both key and value,
    O (B, H, Dl) = softmax over the first seqlens[b] tokens (all Sk when
    seqlens is None) of scale * q . c_j, applied to the latent parts c_j[:Dl].
    Returns O (uint16, B*H*Dl) and, with ``want_stats``, each (b, h)'s score
    maximum and sum of exponentials, shaped (B, H)."""
    Dq = Dl + Dr
    Q = _u16(Q).reshape(-1)
    KV = _u16(KV).reshape(-1)
    if Q.size < B * H * Dq or KV.size < B * Sk * Dq:
        raise ValueError("Q or KV too small")
    sl = None
    if seqlens is not None:
        sl = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int32).reshape(-1))
        if sl.size < B:
            raise ValueError("seqlens needs one entry per sequence")
    O = np.zeros(B * H * Dl, dtype=np.uint16)
    mx = sm = None
    if want_stats:
        mx = np.zeros((B, H), dtype=np.float64)
        sm = np.zeros((B, H), dtype=np.float64)
    rc = _load().oracle_mla_decode_f16(
        _ptr(Q), _ptr(KV), _ptr(O), _ptr(sl) if sl is not None else None, B, H, Sk, Dl, Dr,
        float(scale), _ptr(mx) if mx is not None else None,
        _ptr(sm) if sm is not None else None, host_threads() if threads is None else threads)
    if rc != 0:
        raise ValueError("bad latent-attention sizes")
    if want_stats:
        return O, mx, sm
    return O
