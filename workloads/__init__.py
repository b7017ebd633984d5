"""Seeded synthetic inputs for C = ReLU(A·B): shapes, layouts and value recipes.

This module is shared by the HIP path's tests/benchmark and by the oracle's
tests.  It holds no arithmetic of the method (no products, sums, ReLU or
rounding of results): it only draws operands and describes their layouts.

Recipe, the same for every workload:
  * one ``numpy.random.default_rng(seed)`` (PCG64) per workload;
  * values drawn in binary64: A first (every batch, row-major, M·K per batch),
    then B (every batch, row-major, K·N per batch);
  * the distribution scaled as named, then cast to fp16 with numpy's
    ``astype(float16)`` (round to nearest even);
  * operands are handed over as their raw bit patterns (uint16), in the dense
    row-major layouts lda = K, ldb = N, ldc = N and batch strides M·K, K·N, M·N,
    unless a workload names other leading dimensions.

The shapes are the fp16 GEMM+ReLU workloads this library is measured on:
  small  512^3, uniform(-1,1)                         (oracle finishes in seconds)
  mid    2048^3, uniform(-1,1)                        (128x128x32, 3 stages)
  large  8192^3, normal(0, 1/sqrt(K))                 (compute-bound headline)
  skinny M=16, N=16384, K=8192, uniform(-1,1)/sqrt(K) (HBM-bound decode shape)
  ragged 3001 x 5003 x 1000, uniform(-1,1)            (no dimension tile-aligned)
  batched 1024 x (128x128x64), uniform(-1,1)          (contiguous batch stride)
The pages measure their GEMMs on no public dataset or suite; these synthetic
operands are the whole workload.
"""

from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    dist: str            # "uniform", "normal_invsqrtk", "uniform_invsqrtk"
    seed: int
    batch: int = 1
    lda: int | None = None
    ldb: int | None = None
    ldc: int | None = None
    note: str = field(default="", compare=False)

    @property
    def lda_(self) -> int:
        return self.K if self.lda is None else self.lda

    @property
    def ldb_(self) -> int:
        return self.N if self.ldb is None else self.ldb

    @property
    def ldc_(self) -> int:
        return self.N if self.ldc is None else self.ldc

    @property
    def sA(self) -> int:
        return self.M * self.lda_

    @property
    def sB(self) -> int:
        return self.K * self.ldb_

    @property
    def sC(self) -> int:
        return self.M * self.ldc_

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K * self.batch

    @property
    def compulsory_bytes(self) -> int:
        """Each operand read once and C written once, fp16 elements."""
        return 2 * (self.M * self.K + self.K * self.N + self.M * self.N) * self.batch


WORKLOADS: dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("small_512", 512, 512, 512, "uniform", 0),
        Workload("mid_2048", 2048, 2048, 2048, "uniform", 1),
        Workload("large_8192", 8192, 8192, 8192, "normal_invsqrtk", 2),
        Workload("skinny_16x16384x8192", 16, 16384, 8192, "uniform_invsqrtk", 3),
        Workload("ragged_3001x5003x1000", 3001, 5003, 1000, "uniform", 4),
        Workload("batched_1024x128x128x64", 128, 128, 64, "uniform", 5, batch=1024),
    ]
}


def _draw(rng: np.random.Generator, dist: str, K: int, n: int) -> np.ndarray:
    if dist == "uniform":
        x = rng.uniform(-1.0, 1.0, n)
    elif dist == "normal_invsqrtk":
        x = rng.normal(0.0, 1.0 / np.sqrt(K), n)
    elif dist == "uniform_invsqrtk":
        x = rng.uniform(-1.0, 1.0, n) / np.sqrt(K)
    elif dist == "int3":
        # integers in {-1, 0, 1}: exact fp16 values whose sums are exact in fp32
        x = rng.integers(-1, 2, n).astype(np.float64)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return x


def to_f16_bits(x: np.ndarray) -> np.ndarray:
    """binary64 values -> fp16 bit patterns (numpy's round-to-nearest-even cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """binary64 values -> bfloat16 bit patterns (rounded to binary32 by numpy,
    then to bfloat16 by torch's round-to-nearest-even cast)."""
    import torch
    x32 = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    t = torch.from_numpy(x32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def to_bits(x: np.ndarray, dtype: str = "f16") -> np.ndarray:
    if dtype == "f16":
        return to_f16_bits(x)
    if dtype == "bf16":
        return to_bf16_bits(x)
    raise ValueError(f"unknown element type {dtype!r}")


def generate_dense(M: int, N: int, K: int, dist: str, seed: int, batch: int = 1,
                   dtype: str = "f16"):
    """(A_bits, B_bits): dense row-major operands, A drawn before B, as fp16
    (default) or bf16 bit patterns.  B is (K,N) row-major; its (N,K) form is
    the transpose of the same values."""
    rng = np.random.default_rng(seed)
    a = to_bits(_draw(rng, dist, K, batch * M * K), dtype)
    b = to_bits(_draw(rng, dist, K, batch * K * N), dtype)
    return a, b


def generate_bias(N: int, seed: int, dtype: str = "f16", scale: float = 1.0) -> np.ndarray:
    """N bias values, uniform(-scale, scale), from their own seeded stream."""
    rng = np.random.default_rng(10_000 + seed)
    return to_bits(rng.uniform(-scale, scale, N), dtype)


def transpose_bits(b: np.ndarray, K: int, N: int, batch: int = 1) -> np.ndarray:
    """(K,N) row-major slices -> (N,K) row-major slices (a copy)."""
    return np.ascontiguousarray(
        np.asarray(b).reshape(batch, K, N).transpose(0, 2, 1)).reshape(-1)


def pad_rows(x: np.ndarray, rows: int, cols: int, ld: int, batch: int = 1,
             fill: int = 0x7E00) -> np.ndarray:
    """Copy a dense (batch, rows, cols) bit array into a layout with leading
    dimension ``ld`` >= cols; the pad columns hold ``fill`` (a quiet NaN by
    default, so that reading them shows up in results)."""
    if ld == cols:
        return np.ascontiguousarray(x).reshape(-1)
    out = np.full((batch, rows, ld), fill, dtype=np.uint16)
    out[:, :, :cols] = np.asarray(x).reshape(batch, rows, cols)
    return out.reshape(-1)


def generate(w: Workload | str):
    """(A_bits, B_bits) for a named workload in its own layout (lda, ldb)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    a, b = generate_dense(w.M, w.N, w.K, w.dist, w.seed, w.batch)
    a = pad_rows(a, w.M, w.K, w.lda_, w.batch)
    b = pad_rows(b, w.K, w.N, w.ldb_, w.batch)
    return a, b


def sha256_of(*arrays: np.ndarray) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def sample_positions(w: Workload, n: int, seed: int = 1234) -> np.ndarray:
    """(n, 3) int64 array of (b, i, j) output positions to check at full size:
    the four corners of every batch's window, the last row and column, and
    uniformly drawn interior points (seeded)."""
    rng = np.random.default_rng(seed)
    M, N, B = w.M, w.N, w.batch
    pts = []
    for b in sorted({0, B - 1}):
        for i in sorted({0, M - 1}):
            for j in sorted({0, N - 1}):
                pts.append((b, i, j))
    extra = max(n - len(pts), 0)
    bb = rng.integers(0, B, extra)
    ii = rng.integers(0, M, extra)
    jj = rng.integers(0, N, extra)
    # a quarter of the random points on the last tile row / column, where
    # ragged edges live
    q = extra // 4
    ii[:q] = M - 1 - rng.integers(0, min(M, 128), q)
    jj[q:2 * q] = N - 1 - rng.integers(0, min(N, 128), q)
    pts.extend(zip(bb.tolist(), ii.tolist(), jj.tolist()))
    return np.asarray(pts, dtype=np.int64)


def generate_w4(N: int, K: int, G: int, seed: int, dtype: str = "f16"):
    """A packed int4 weight and its group scales for an (N,K) weight: q
    uniform on -8..7, two per byte along k (even k in the low nibble), and one
    scale per group of G k per row, uniform in [0.5, 1.5] / (8 sqrt(K)) (so
    the dequantized weights have the magnitude of uniform(-1,1)/sqrt(K)).
    Returns (Wq uint8 (N, K/2) flattened, S bits (N, K/G) flattened)."""
    rng = np.random.default_rng(20_000 + seed)
    q = rng.integers(-8, 8, (N, K))
    u = (q & 15).astype(np.uint8)
    wq = (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)
    s = rng.uniform(0.5, 1.5, (N, K // G)) / (8.0 * np.sqrt(K))
    return wq.reshape(-1), to_bits(s.reshape(-1), dtype)


# Latent-attention decode workload: 64 sequences of 8192 cached tokens, 128
# query heads, rows of 512 + 64 values (the pages plot batch 64 and 128 at fp16
# for this kernel; 8192 tokens is the cache length used here).
MLA_WORKLOAD = {"name": "mla_decode_64x128x8192", "B": 64, "H": 128, "Sk": 8192, "seed": 6}
MLA_ROW = 576


def generate_mla(B: int, H: int, Sk: int, seed: int):
    """Q (B, H, 576) and the cache KV (B, Sk, 576) as fp16 bits, each value
    normal(0, 1) drawn in binary32 from one default_rng(60_000 + seed), Q first,
    rounded to nearest even.  Returns (Q, KV) flattened."""
    rng = np.random.default_rng(60_000 + seed)
    q = rng.standard_normal(B * H * MLA_ROW, dtype=np.float32).astype(np.float16)
    kv = np.empty(B * Sk * MLA_ROW, dtype=np.float16)
    step = 1 << 24
    for i in range(0, kv.size, step):
        n = min(step, kv.size - i)
        kv[i:i + n] = rng.standard_normal(n, dtype=np.float32).astype(np.float16)
    return q.view(np.uint16), kv.view(np.uint16)
