"""The seeded input generator: reproducible bytes, layouts and distributions."""

import json
import os

import numpy as np
import pytest

import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("name", ["small_512", "mid_2048", "skinny_16x16384x8192",
                                  "ragged_3001x5003x1000", "batched_1024x128x128x64"])
def test_input_bytes_are_pinned(name):
    with open(os.path.join(GOLDEN, "inputs_sha256.json")) as f:
        want = json.load(f)[name]
    a, b = wl.generate(name)
    assert wl.sha256_of(a) == want["A"]
    assert wl.sha256_of(b) == want["B"]


def test_same_seed_same_bytes():
    a1, b1 = wl.generate_dense(17, 23, 31, "normal_invsqrtk", 99)
    a2, b2 = wl.generate_dense(17, 23, 31, "normal_invsqrtk", 99)
    assert np.array_equal(a1, a2) and np.array_equal(b1, b2)
    a3, _ = wl.generate_dense(17, 23, 31, "normal_invsqrtk", 100)
    assert not np.array_equal(a1, a3)


@pytest.mark.parametrize("dist,lo,hi,std", [
    ("uniform", -1, 1, 1 / np.sqrt(3)),
    ("normal_invsqrtk", None, None, 1 / np.sqrt(4096)),
    ("uniform_invsqrtk", -1 / 64, 1 / 64, 1 / np.sqrt(3) / 64),
])
def test_distribution_moments(dist, lo, hi, std):
    a, b = wl.generate_dense(256, 256, 4096, dist, 3)
    x = a.view(np.float16).astype(np.float64)
    assert abs(x.mean()) < 5 * std / np.sqrt(x.size)
    assert abs(x.std() / std - 1) < 0.01
    if lo is not None:
        assert x.min() >= lo and x.max() <= hi


def test_workload_shapes_and_layouts():
    w = wl.WORKLOADS["ragged_3001x5003x1000"]
    assert (w.M, w.N, w.K, w.lda_, w.ldb_, w.ldc_) == (3001, 5003, 1000, 1000, 5003, 5003)
    w = wl.WORKLOADS["batched_1024x128x128x64"]
    assert (w.batch, w.sA, w.sB, w.sC) == (1024, 128 * 64, 64 * 128, 128 * 128)
    assert wl.WORKLOADS["large_8192"].flops == 2 * 8192 ** 3


def test_pad_rows_layout():
    x = np.arange(6, dtype=np.uint16)
    p = wl.pad_rows(x, 2, 3, 5)
    assert list(p) == [0, 1, 2, 0x7E00, 0x7E00, 3, 4, 5, 0x7E00, 0x7E00]


def test_sample_positions_in_range():
    w = wl.WORKLOADS["ragged_3001x5003x1000"]
    idx = wl.sample_positions(w, 500)
    assert idx.shape == (500, 3)
    assert idx[:, 1].max() < w.M and idx[:, 2].max() < w.N and idx.min() >= 0
    assert (w.M - 1) in idx[:, 1] and (w.N - 1) in idx[:, 2]
