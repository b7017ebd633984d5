"""bench.py: host logic on the CPU, and the JSON line of a short run on the GPU."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_only_while_sources_unchanged(tmp_path, monkeypatch):
    f = tmp_path / "traffic.txt"
    h = bench.kernel_source_hash("large_8192")
    f.write_text("# comment\n"
                 f"large_8192 {h} 1.5e9 1.25e8\n"
                 "skinny_16x16384x8192 0000000000000000 2.7e8 5.2e5\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("large_8192") == pytest.approx(1.625e9)
    assert bench.measured_traffic("skinny_16x16384x8192") is None     # stale hash
    assert bench.measured_traffic("batched_1024x128x128x64") is None  # no entry


def test_source_hash_follows_the_workloads_kernel():
    # the skinny workload hashes its own kernel file; the ragged kernel lives
    # in the same file as the aligned tile kernels
    assert bench.kernel_source_hash("skinny_16x16384x8192") != bench.kernel_source_hash("large_8192")
    assert bench.kernel_source_hash("ragged_3001x5003x1000") == bench.kernel_source_hash("large_8192")
    assert bench.kernel_source_hash("mid_2048") == bench.kernel_source_hash("large_8192")


@pytest.mark.gpu
def test_json_line_contract():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("[case] bench.py --steps 2 --warmup 1", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "2",
                        "--warmup", "1"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["value"] > 0 and d["unit"] == "TFLOP/s" and d["higher_is_better"] is True
    assert d["dtype"] == "f16" and d["vs_baseline"] is None
    assert d["config"]["workload"] == "large_8192"
    # value is the 8192^3 flop over the measured time per step
    assert d["value"] == pytest.approx(2 * 8192 ** 3 / (d["ms_per_step"] * 1e-3) / 1e12, rel=1e-6)
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 2516.6
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"])
    assert rf["traffic"] is None or rf["traffic"] > 0
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0 and cb["sample"]
    # the trials protocol: >= 10 trials of >= 20 ms, median <= max, min <= median
    t = d["timing"]
    assert t["trials"] >= 10 and t["trial_ms_min"] >= 20.0 * 0.9
    assert t["min_ms_per_call"] <= t["median_ms_per_call"] <= t["max_ms_per_call"]
    assert t["rate_at_min"] >= t["rate_at_median"] > 0
    sc = d["sclk_mhz"]
    assert sc is None or (100 < sc["min"] <= sc["median"] <= sc["max"] < 5000)
    # the other workloads of the hot-path table ride along, each on its own protocol run
    others = {o["workload"]: o for o in d["other_workloads"]}
    assert set(others) == {"mid_2048", "batched_1024x128x128x64", "ragged_3001x5003x1000",
                           "small_512"}
    for o in list(others.values()) + [d["secondary"]]:
        assert o["value"] > 0 and o["ms_per_step"] > 0 and o["steps"] == 20
        orf = o["roofline"]
        assert orf["bound"] in ("mfma", "hbm") and orf["frac"] == pytest.approx(orf["achieved"] / orf["peak"])
        assert o["timing"]["trials"] >= 10
    assert others["mid_2048"]["unit"] == "TFLOP/s" and others["batched_1024x128x128x64"]["unit"] == "GB/s"
    # and the measured NEXT rows, each the object its own mode prints
    nxt = [o["config"]["workload"] for o in d["next_rows"]]
    assert nxt == ["attention_4x4096x32x128_full", "attention_4x4096x32x128_causal",
                   "mla_decode_64x128x8192", "w4_16x16384x8192_g128"]
    for o in d["next_rows"]:
        assert o["value"] > 0 and o["steps"] == 20 and o["timing"]["trials"] >= 10


@pytest.mark.gpu
def test_capi_bench_runs_through_the_c_abi():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    exe = os.path.join(ROOT, "tiled_dense_gemm_05_amd", "tg_capi_bench")
    if not os.path.exists(exe):
        pytest.fail("tg_capi_bench is not built")
    print("[case] tg_capi_bench 512 512 512 5 2", flush=True)
    r = subprocess.run([exe, "512", "512", "512", "5", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads(r.stdout.strip().splitlines()[-1])
    assert d["M"] == 512 and d["iters"] == 5 and d["copies"] == 2
    assert d["us_per_call"] > 0 and d["path"] == "tile128"
    assert d["tflops"] == pytest.approx(2 * 512 ** 3 / (d["us_per_call"] * 1e-6) / 1e12, rel=1e-2)
