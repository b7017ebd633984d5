"""Throughput of C = ReLU(A·B) (fp16 in, fp32 accumulate, fp16 out) on one MI355X.

A step is one call of the library on one synthetic workload already resident
in HBM.  The headline workload is the 8192^3 GEMM with normal(0, 1/sqrt(K))
operands (compute-bound, measured in TFLOP/s against the dense fp16 MFMA
peak); the M=16 decode-shaped workload (HBM-bound, GB/s against the HBM peak)
is reported alongside as a secondary figure, and with the headline workload the
other workloads (2048^3, the strided batch, the ragged shape, 512^3) follow in
`other_workloads`, each timed the same way, and the measured NEXT rows (attention
forward, the latent-attention decode, int4 weights) in `next_rows`, each the object
its own --attention / --mla / --w4 mode prints.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--no-secondary]
                    [--tile-variant V] [--skinny-variant V] [--raster G]
                    [--act relu|none] [--bias] [--dtype f16|bf16] [--layout kn|nk]

--tile-variant, --skinny-variant and --raster select non-default kernel
configurations and tile orders for ablations; --act, --bias, --dtype and
--layout measure the extended entry point tg_gemm_ex.  A line measured with any of them carries them
in `config` and no `traffic` figure (the counters are taken at the defaults).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

METRIC = "TFLOP/s fp16 GEMM+ReLU at 8192^3 (% of FP16 MFMA peak); GB/s at M=16"
PEAK_F16_TFLOPS = 2516.6     # 256 CU x 4096 flop/clk x 2.4 GHz, dense
PEAK_HBM_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "traffic.txt")
COPY_BYTES = 1 << 30          # the calibration copy: 1 GiB read + 1 GiB written
CSRC = os.path.join(ROOT, "tiled_dense_gemm_05_amd", "csrc")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# The sources that decide the kernel a workload's launch runs: the dispatcher,
# the shared internal header and the kernel's own file.
KERNEL_SOURCES = {
    "skinny_16x16384x8192": ("api.cpp", "tg_internal.h", "tg_lds_dma.h", "gemm_skinny.hip"),
}
DEFAULT_SOURCES = ("api.cpp", "tg_internal.h", "tg_lds_dma.h", "gemm_dma.hip")


def kernel_source_hash(workload: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES.get(workload, DEFAULT_SOURCES):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def read_traffic_file() -> dict:
    """profiles/traffic.txt: one line per workload,
    `workload source_hash fetch_bytes write_bytes` (per launch, calibrated)."""
    out = {}
    try:
        with open(TRAFFIC_FILE) as f:
            for line in f:
                parts = line.split()
                if len(parts) == 4 and not line.startswith("#"):
                    out[parts[0]] = (parts[1], float(parts[2]), float(parts[3]))
    except OSError:
        pass
    return out


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed counter runs, only while the
    kernel sources are unchanged since those counters were taken."""
    e = read_traffic_file().get(workload)
    if not e or e[0] != kernel_source_hash(workload):
        return None
    return e[1] + e[2]


TRIALS = 10            # timed trials per workload (median and min reported)
TRIAL_MS = 20.0        # each trial at least this long


class ClockSampler:
    """Measures the shader clock while a timed region runs: a one-wave spin
    kernel (torch.cuda._sleep, which spins until clock64() has advanced by n
    shader-clock cycles) runs on a second stream of default priority, next
    to the workload, bracketed by HIP events on that stream; n / elapsed time
    is the clock it saw.  The spinning wave needs no LDS and a few
    registers, so it shares a compute unit with the workload's workgroups
    instead of displacing one.  `idle` is the same measurement with nothing
    else running (the boost clock)."""

    SOURCE = ("torch.cuda._sleep(n) on a second stream during the trials: n shader-clock "
              "cycles / elapsed time between HIP events")

    def __init__(self, torch, cycles: int = 30_000_000, spins: int = 6):
        self.torch = torch
        self.cycles = cycles
        self.spins = spins
        self.stream = torch.cuda.Stream()
        self.samples = []
        self.idle = self._measure(1)[0]
        self._pending = []

    def _enqueue(self, n):
        t = self.torch
        evs = []
        with t.cuda.stream(self.stream):
            for _ in range(n):
                a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
                a.record(self.stream)
                t.cuda._sleep(self.cycles)
                b.record(self.stream)
                evs.append((a, b))
        return evs

    def _collect(self, evs):
        self.stream.synchronize()
        return [self.cycles / (a.elapsed_time(b) * 1e3) for a, b in evs]   # MHz

    def _measure(self, n):
        return self._collect(self._enqueue(n))

    def __enter__(self):
        # the current stream's work so far must not be overlapped by the spins
        self.stream.wait_stream(self.torch.cuda.current_stream())
        self._pending = self._enqueue(self.spins)
        return self

    def __exit__(self, *exc):
        self.samples.extend(self._collect(self._pending))
        self._pending = []
        return False

    def reset(self):
        self.samples = []

    def summary(self):
        if not self.samples:
            return None
        x = sorted(self.samples)
        return {"median": x[len(x) // 2], "min": x[0], "max": x[-1], "samples": len(x),
                "idle": self.idle, "source": self.SOURCE}


def time_calls(torch, call, steps: int, warmup: int, clock: ClockSampler | None = None,
               trials: int = TRIALS, graph_call=None):
    """The timing protocol of every workload line.

    1. `warmup` untimed calls.
    2. `trials` trials of n back-to-back calls each, n chosen so a trial lasts
       at least TRIAL_MS; one pair of HIP events per trial on the launch
       stream; the shader clock is sampled meanwhile.  Median and min of the
       per-call time over the trials are reported.
    3. The contract window: exactly `steps` calls (or one replay of
       `graph_call`, a graph of `steps` calls), synchronized on both sides
       and bracketed by events on the launch stream, behind one untimed
       primer call; ms_per_step comes from it.  It runs last, when the card
       has been busy for the trials, so it measures the sustained
       (power-limited) rate.
    call(i) enqueues call i on torch's current stream."""
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    out = {"trials": trials}
    if trials > 0:
        # a short probe sizes the trials
        t0, t1 = ev(), ev()
        t0.record(stream)
        for i in range(3):
            call(i)
        t1.record(stream)
        torch.cuda.synchronize()
        per = max(t0.elapsed_time(t1) / 3, 1e-4)
        n = max(1, int(np.ceil(1.25 * TRIAL_MS / per)))
        per_call = []
        with (clock if clock is not None else _Null()):
            for t in range(trials):
                a, b = ev(), ev()
                a.record(stream)
                for i in range(n):
                    call(i)
                b.record(stream)
                b.synchronize()
                per_call.append(a.elapsed_time(b) / n)
        x = sorted(per_call)
        out.update({"calls_per_trial": n, "trial_ms_min": x[0] * n,
                    "median_ms_per_call": x[len(x) // 2], "min_ms_per_call": x[0],
                    "max_ms_per_call": x[-1]})
    torch.cuda.synchronize()
    t0, t1 = ev(), ev()
    # one untimed call ahead of the start event: the window then starts when
    # the GPU reaches it, with the next calls already queued behind it, so it
    # holds the GPU time of exactly `steps` back-to-back calls and not the
    # latency of getting the first launch from an idle queue onto the GPU
    call(0)
    t0.record(stream)
    if graph_call is not None:
        graph_call()
    else:
        for i in range(steps):
            call(i)
    t1.record(stream)
    torch.cuda.synchronize()
    out["ms_per_step"] = t0.elapsed_time(t1) / steps
    return out


class _Null:
    def __enter__(self):
        return self

    def __exit__(self, *exc):
        return False


def timing_fields(timing: dict, clock: ClockSampler | None, work: float, scale: float):
    """The `timing` and `sclk_mhz` objects of a JSON line: work per call
    (flop or bytes) / per-call time, in the line's unit (work / s / scale)."""
    t = {"protocol": (f"{timing['trials']} trials of calls_per_trial back-to-back calls "
                      f"(each trial >= {TRIAL_MS:.0f} ms, one pair of HIP events on the launch "
                      f"stream), then the contract window of exactly `steps` calls that "
                      f"ms_per_step comes from")}
    t.update({k: v for k, v in timing.items() if k != "ms_per_step"})
    if "median_ms_per_call" in timing:
        t["rate_at_median"] = work / (timing["median_ms_per_call"] * 1e-3) / scale
        t["rate_at_min"] = work / (timing["min_ms_per_call"] * 1e-3) / scale
    sclk = clock.summary() if clock is not None else None
    return t, sclk


def calibration_copy(torch):
    """A plain 1 GiB device-to-device copy, twice, for counter calibration."""
    src = torch.ones(COPY_BYTES // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def run_workload(tg, torch, w: wl.Workload, steps: int, warmup: int, epilogue=None,
                 dtype: str = "f16", layout: str = "kn", graph: bool = False,
                 clock: ClockSampler | None = None, trials: int = TRIALS):
    """Times `steps` calls after `warmup`.  epilogue = (activation, with_bias)
    routes the calls through tg_gemm_ex, as do a bf16 element type and an
    (N,K) B; otherwise the GEMM+ReLU entry points are timed.  With `graph`
    the `steps` calls of the contract window are captured into one HIP graph
    and one replay is timed (no host launch cost between the kernels); the
    trials always launch directly.  Returns (timing dict of time_calls, path,
    input copies)."""
    a, b = wl.generate_dense(w.M, w.N, w.K, w.dist, w.seed, batch=w.batch, dtype=dtype)
    ex = epilogue is not None or dtype != "f16" or layout != "kn"
    if epilogue is None:
        epilogue = (tg.TG_ACT_RELU, False)
    ldb = w.ldb_
    if layout == "nk":
        # the workloads are dense (lda = K, ldb = N); the (N,K) form is the
        # transposed B with ldb = K
        b = wl.transpose_bits(b, w.K, w.N, w.batch)
        ldb = w.K
    dev = torch.device("cuda:0")
    nbuf = 1
    # skinny and batched workloads are HBM-bound: rotate input copies so a
    # rerun is not served from the 256 MB last-level cache
    if w.compulsory_bytes < 600e6 and w.flops / w.compulsory_bytes < 100:
        nbuf = max(2, int(np.ceil(600e6 / w.compulsory_bytes)))
    A = [torch.from_numpy(a.view(np.int16)).to(dev) for _ in range(nbuf)]
    B = [torch.from_numpy(b.view(np.int16)).to(dev) for _ in range(nbuf)]
    csize = (w.batch - 1) * w.sC + (w.M - 1) * w.ldc_ + w.N
    C = [torch.empty(csize, dtype=torch.int16, device=dev) for _ in range(nbuf)]
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    bias = None
    if epilogue[1]:
        bias = torch.from_numpy(
            wl.generate_bias(w.N, w.seed, dtype=dtype, scale=0.05).view(np.int16)).to(dev)
    dt = tg.TG_DTYPE_BF16 if dtype == "bf16" else tg.TG_DTYPE_F16
    lay = tg.TG_B_NK if layout == "nk" else tg.TG_B_KN

    def call(i, sh=sh):
        j = i % nbuf
        if ex:
            st = tg.tg_gemm_ex(dt, lay, epilogue[0], A[j].data_ptr(), B[j].data_ptr(),
                               C[j].data_ptr(), bias.data_ptr() if bias is not None else 0, w.M,
                               w.N, w.K, w.lda_, ldb, w.ldc_, w.sA, w.sB, w.sC, w.batch, sh)
        elif w.batch == 1:
            st = tg.tg_gemm_relu_f16(A[j].data_ptr(), B[j].data_ptr(), C[j].data_ptr(), w.M, w.N,
                                     w.K, w.lda_, w.ldb_, w.ldc_, sh)
        else:
            st = tg.tg_gemm_relu_f16_strided_batched(
                A[j].data_ptr(), B[j].data_ptr(), C[j].data_ptr(), w.M, w.N, w.K, w.lda_, w.ldb_,
                w.ldc_, w.sA, w.sB, w.sC, w.batch, sh)
        if st != tg.TG_OK:
            raise RuntimeError(tg.tg_status_string(st))

    graph_call = None
    if graph:
        for i in range(warmup):
            call(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cs = torch.cuda.current_stream().cuda_stream
            for i in range(steps):
                call(i, cs)
        g.replay()
        torch.cuda.synchronize()
        graph_call = g.replay
    timing = time_calls(torch, call, steps, warmup, clock, trials, graph_call)
    path = tg.tg_path_name(tg.tg_last_path())
    return timing, path, nbuf


def run_vendor(torch, w: wl.Workload, steps: int, warmup: int, dtype: str, layout: str,
               trials: int = TRIALS):
    """Times torch.matmul (hipBLASLt on ROCm) on the workload's operands, as
    context for the library's own rate: the same product without the ReLU,
    into a preallocated output.  Dense layouts only (the named workloads with
    lda = K, ldb = N); a batch goes through torch.bmm with contiguous
    operands."""
    a, b = wl.generate_dense(w.M, w.N, w.K, w.dist, w.seed, batch=w.batch, dtype=dtype)
    td = torch.bfloat16 if dtype == "bf16" else torch.float16
    dev = torch.device("cuda:0")
    A = torch.from_numpy(a.view(np.int16)).to(dev).view(td).reshape(w.batch, w.M, w.K)
    B = torch.from_numpy(b.view(np.int16)).to(dev).view(td).reshape(w.batch, w.K, w.N)
    if layout == "nk":
        # an (N,K) weight: the product reads it through a transposed view
        Bt = B.transpose(1, 2).contiguous()
        B = Bt.transpose(1, 2)
    C = torch.empty(w.batch, w.M, w.N, dtype=td, device=dev)
    if w.batch == 1:
        A2, B2, C2 = A[0], B[0], C[0]
        call = lambda: torch.matmul(A2, B2, out=C2)
    else:
        B = B.contiguous()
        call = lambda: torch.bmm(A, B, out=C)
    return time_calls(torch, lambda i: call(), steps, warmup, trials=trials)


def run_w4(tg, torch, M: int, N: int, K: int, G: int, steps: int, warmup: int, dtype: str,
           trials: int = TRIALS):
    """Times the weight-only int4 GEMM (tg_gemm_w4) on an (N,K) int4 weight with
    group scales; several weight copies rotate so reruns come from HBM."""
    a, _ = wl.generate_dense(M, 8, K, "uniform_invsqrtk", 3, dtype=dtype)
    wq, s = wl.generate_w4(N, K, G, 3, dtype=dtype)
    wbytes = wq.size + 2 * s.size
    nbuf = max(2, int(np.ceil(600e6 / wbytes)))
    dev = torch.device("cuda:0")
    A = torch.from_numpy(a.view(np.int16)).to(dev)
    W = [torch.from_numpy(wq).to(dev) for _ in range(nbuf)]
    S = [torch.from_numpy(s.view(np.int16)).to(dev) for _ in range(nbuf)]
    C = torch.empty(M * N, dtype=torch.int16, device=dev)
    stream = torch.cuda.current_stream()
    dt = tg.TG_DTYPE_BF16 if dtype == "bf16" else tg.TG_DTYPE_F16

    def call(i):
        j = i % nbuf
        st = tg.tg_gemm_w4(dt, tg.TG_ACT_RELU, A.data_ptr(), W[j].data_ptr(), S[j].data_ptr(),
                           C.data_ptr(), 0, M, N, K, G, K, K // 2, K // G, N, stream.cuda_stream)
        if st != tg.TG_OK:
            raise RuntimeError(tg.tg_status_string(st))

    timing = time_calls(torch, call, steps, warmup, trials=trials)
    return timing, tg.tg_path_name(tg.tg_last_path()), nbuf, wbytes + 2 * (M * K + M * N)


def run_attention(tg, torch, B: int, S: int, H: int, Hkv: int, D: int, causal: bool,
                  steps: int, warmup: int, trials: int = TRIALS):
    """Times the fused attention forward on (B, S, H, D) queries and (B, S, Hkv, D)
    keys and values (tg_attention_fwd_f16 when Hkv = H, else
    tg_attention_fwd_f16_gqa), normal(0,1) Q and K, uniform(-1,1) V."""
    rng = np.random.default_rng(11)
    dev = torch.device("cuda:0")
    n = B * S * H * D
    nkv = B * S * Hkv * D
    Q, K, V = (torch.from_numpy(wl.to_f16_bits(rng.normal(0, 1, m) if i < 2 else
                                               rng.uniform(-1, 1, m)).view(np.int16)).to(dev)
               for i, m in enumerate((n, nkv, nkv)))
    O = torch.empty(n, dtype=torch.int16, device=dev)
    stream = torch.cuda.current_stream()
    scale = 1.0 / float(np.sqrt(D))

    def call():
        if Hkv == H:
            st = tg.tg_attention_fwd_f16(Q.data_ptr(), K.data_ptr(), V.data_ptr(), O.data_ptr(),
                                         B, S, S, H, D, scale, int(causal), stream.cuda_stream)
        else:
            st = tg.tg_attention_fwd_f16_gqa(Q.data_ptr(), K.data_ptr(), V.data_ptr(),
                                             O.data_ptr(), B, S, S, H, Hkv, D, scale,
                                             int(causal), stream.cuda_stream)
        if st != tg.TG_OK:
            raise RuntimeError(tg.tg_status_string(st))

    return time_calls(torch, lambda i: call(), steps, warmup, trials=trials)


def run_mla(tg, torch, steps: int, warmup: int, trials: int = TRIALS):
    """Times the latent-attention decode (tg_mla_decode_f16) on the 64 x 8192-token,
    128-head workload; returns (ms per call, path, workspace bytes)."""
    w = wl.MLA_WORKLOAD
    B, H, Sk = w["B"], w["H"], w["Sk"]
    q, kv = wl.generate_mla(B, H, Sk, w["seed"])
    dev = torch.device("cuda:0")
    Q = torch.from_numpy(q.view(np.int16)).to(dev)
    KV = torch.from_numpy(kv.view(np.int16)).to(dev)
    del q, kv
    O = torch.empty(B * H * 512, dtype=torch.int16, device=dev)
    need = tg.tg_mla_decode_workspace_bytes(B, H, Sk)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    scale = 1.0 / float(np.sqrt(192.0))

    def call():
        st = tg.tg_mla_decode_f16(Q.data_ptr(), KV.data_ptr(), O.data_ptr(), 0, B, H, Sk,
                                  scale, ws.data_ptr(), need, stream.cuda_stream)
        if st != tg.TG_OK:
            raise RuntimeError(tg.tg_status_string(st))

    timing = time_calls(torch, lambda i: call(), steps, warmup, trials=trials)
    return timing, tg.tg_path_name(tg.tg_last_path()), need


def run_splitk(tg, torch, splits: int, steps: int, warmup: int, trials: int = TRIALS):
    """Times the split-K form of the skinny GEMM+ReLU (tg_gemm_relu_f16_splitk) on the
    16 x 16384 x 8192 workload, input copies rotated as for the single-pass path;
    returns (ms per call, copies, workspace bytes)."""
    w = wl.WORKLOADS["skinny_16x16384x8192"]
    a, b = wl.generate(w)
    dev = torch.device("cuda:0")
    nbuf = max(2, int(np.ceil(600e6 / w.compulsory_bytes)))
    A = [torch.from_numpy(a.view(np.int16)).to(dev) for _ in range(nbuf)]
    B = [torch.from_numpy(b.view(np.int16)).to(dev) for _ in range(nbuf)]
    C = [torch.empty(w.M * w.N, dtype=torch.int16, device=dev) for _ in range(nbuf)]
    need = tg.tg_gemm_splitk_workspace_bytes(w.M, w.N, splits)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def call(j):
        st = tg.tg_gemm_relu_f16_splitk(A[j].data_ptr(), B[j].data_ptr(), C[j].data_ptr(), w.M,
                                        w.N, w.K, w.K, w.N, w.N, splits, ws.data_ptr(), need,
                                        stream.cuda_stream)
        if st != tg.TG_OK:
            raise RuntimeError(tg.tg_status_string(st))

    timing = time_calls(torch, lambda i: call(i % nbuf), steps, warmup, trials=trials)
    return timing, nbuf, need


def cpu_baseline(w: wl.Workload, target_s: float = 16.0):
    """The oracle, as it stands, on the host cores: rows 0..r-1 of the
    workload's C (all N columns, full K), r sized for about target_s seconds."""
    import oracle
    oracle.build(force=False)
    threads = oracle.host_threads()
    a, b = wl.generate(w)
    K, N = w.K, w.N

    def timed(r):
        t = time.perf_counter()
        oracle.gemm_relu(a[: r * w.lda_], b, r, N, K, w.lda_, w.ldb_, w.ldc_, threads=threads)
        return time.perf_counter() - t

    r2, dt2 = max(threads, 16), 0.0
    for _ in range(4):
        dt2 = timed(r2)
        if dt2 >= 0.7 * target_s or r2 >= w.M:   # a sample of 11-30 s
            break
        r2 = int(min(w.M, r2 * target_s / max(dt2, 1e-3)))
        r2 = max(threads, (r2 // threads) * threads)
    tflops = 2.0 * r2 * N * K / dt2 / 1e12
    return {
        "value": tflops,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"rows 0..{r2 - 1} of the {w.M}x{w.N}x{w.K} workload's C ({r2}x{N}x{K} "
                   f"multiply-adds, binary64 C oracle, {threads} threads), {dt2:.1f} s, "
                   f"rate scaled to the whole workload"),
    }


def _csv_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _find(d, suffix):
    for root, _, files in os.walk(d):
        for fn in files:
            if fn.endswith(suffix):
                return os.path.join(root, fn)
    raise FileNotFoundError(f"no *{suffix} under {d}")


def summarize(workload: str, stats_dir: str, fetch_dir: str, write_dir: str, commands: list[str]):
    """Writes profiles/<kernel-workload>.md from rocprofv3 output directories
    (kernel-trace --stats run, then one --pmc FETCH_SIZE and one --pmc
    WRITE_SIZE run of `bench.py --calibrate-copy`), and records the
    calibrated HBM bytes per launch in profiles/traffic.txt."""
    import collections
    stats = _csv_rows(_find(stats_dir, "kernel_stats.csv"))
    stats.sort(key=lambda r: -float(r["TotalDurationNs"]))
    top = stats[0]

    def per_kernel(d, counter):
        acc = collections.defaultdict(list)
        per_dispatch = collections.defaultdict(float)
        names = {}
        for r in _csv_rows(_find(d, "counter_collection.csv")):
            if r["Counter_Name"] != counter:
                continue
            per_dispatch[r["Dispatch_Id"]] += float(r["Counter_Value"])
            names[r["Dispatch_Id"]] = r["Kernel_Name"]
        for k, v in per_dispatch.items():
            acc[names[k]].append(v)
        return acc

    fetch = per_kernel(fetch_dir, "FETCH_SIZE")
    write = per_kernel(write_dir, "WRITE_SIZE")
    copy_name = next(n for n in fetch if "copyBuffer" in n or "copy" in n.lower())
    gemm_name = max(fetch, key=lambda n: sum(fetch[n]) if "tg::" in n else -1)
    kib = 1024.0
    copy_fetch = sum(fetch[copy_name]) / len(fetch[copy_name]) * kib
    copy_write = sum(write[copy_name]) / len(write[copy_name]) * kib
    f_fetch = COPY_BYTES / copy_fetch
    f_write = COPY_BYTES / copy_write
    g_fetch = sum(fetch[gemm_name]) / len(fetch[gemm_name]) * kib * f_fetch
    g_write = sum(write[gemm_name]) / len(write[gemm_name]) * kib * f_write
    w = wl.WORKLOADS[workload]
    family = ("gemm_relu_dma_stream_kernel" if "dma_stream_kernel" in top["Name"] else
              "gemm_relu_dma_kernel" if "dma_kernel" in top["Name"] else
              "gemm_relu_skinny_kernel" if "skinny_kernel" in top["Name"] else
              "gemm_relu_tile_kernel" if "tile_kernel" in top["Name"] else "kernel")
    md = os.path.join(PROFILES, f"{family}-{workload}.md")
    with open(md, "w") as f:
        f.write(f"# {top['Name'].replace('tg::(anonymous namespace)::', '')} on {workload}\n\n")
        f.write("Commands (from the repository root on the GPU box):\n\n")
        for c in commands:
            f.write(f"    {c}\n")
        f.write("\nKernel trace (rocprofv3 --kernel-trace --stats), top kernels:\n\n")
        f.write("| kernel | calls | average ns | min ns | max ns |\n|---|---|---|---|---|\n")
        for r in stats[:4]:
            name = r["Name"].replace("tg::(anonymous namespace)::", "")
            f.write(f"| {name[:120]} | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                    f"{float(r['MinNs']):.0f} | {float(r['MaxNs']):.0f} |\n")
        f.write(f"\nAlgorithmic work per launch: {w.flops:.4e} flop, "
                f"{w.compulsory_bytes:.4e} compulsory HBM bytes.\n")
        f.write(f"\nCounters (rocprofv3 --pmc, one counter set per run), per launch:\n\n")
        f.write(f"* calibration copy of {COPY_BYTES} bytes: FETCH_SIZE {copy_fetch:.4e} B, "
                f"WRITE_SIZE {copy_write:.4e} B -> factors {f_fetch:.3f} (fetch), "
                f"{f_write:.3f} (write)\n")
        reads = 2 * (w.M * w.K + w.K * w.N) * w.batch
        writes = 2 * w.M * w.N * w.batch
        f.write(f"* GEMM: HBM read {g_fetch:.4e} B ({g_fetch / reads:.2f} x the {reads:.4e} B of A and B), "
                f"HBM write {g_write:.4e} B ({g_write / writes:.2f} x the {writes:.4e} B of C)\n")
        f.write(f"* kernel source hash {kernel_source_hash(workload)} "
                f"({', '.join(KERNEL_SOURCES.get(workload, DEFAULT_SOURCES))})\n")
    lines = {k: v for k, v in read_traffic_file().items()}
    lines[workload] = (kernel_source_hash(workload), g_fetch, g_write)
    with open(TRAFFIC_FILE, "w") as f:
        f.write("# workload source_hash hbm_read_bytes hbm_write_bytes (per launch, calibrated)\n")
        for k, (h, r_, w_) in sorted(lines.items()):
            f.write(f"{k} {h} {r_:.6e} {w_:.6e}\n")
    print(f"wrote {md} and {TRAFFIC_FILE}")


def _dispatch_counters(d):
    """Counter values per dispatch of the library's kernels under directory d:
    {dispatch id: {"name", "us", counter: value summed over its instances}}."""
    out = {}
    for r in _csv_rows(_find(d, "counter_collection.csv")):
        e = out.setdefault(r["Dispatch_Id"], {
            "name": r["Kernel_Name"],
            "us": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3})
        e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def summarize_ablation(out_md: str, root: str, title: str):
    """Writes a table of ablation runs.  root/labels.txt holds one line per
    run, `label<TAB>description`; root/<label>/bench.json is that run's bench
    line, root/<label>/pmc one counter run (SQ_CYCLES, SQ_VALU_MFMA_BUSY_CYCLES,
    SQ_LDS_BANK_CONFLICT, SQ_LDS_IDX_ACTIVE, TCC_HIT_sum, TCC_MISS_sum) and
    root/<label>/fetch one FETCH_SIZE run with the calibration copy;
    root/commands.txt the commands, copied into the summary."""
    with open(os.path.join(root, "labels.txt")) as f:
        labels = [ln.rstrip("\n").split("\t", 1) for ln in f if ln.strip()]
    with open(os.path.join(root, "commands.txt")) as f:
        commands = f.read().rstrip()
    rows = []
    for label, desc in labels:
        d = os.path.join(root, label)
        with open(os.path.join(d, "bench.json")) as f:
            b = json.loads(f.read().strip().splitlines()[-1])
        w = wl.WORKLOADS[b["config"]["workload"]]
        pmc = [v for v in _dispatch_counters(os.path.join(d, "pmc")).values() if "tg::" in v["name"]]
        n = len(pmc)
        avg = lambda key: sum(v[key] for v in pmc) / n
        clock = sum(v["SQ_CYCLES"] / 32 / v["us"] / 1e3 for v in pmc) / n
        mfma = sum(v["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * v["SQ_CYCLES"] / 32) for v in pmc) / n
        lds_conf = avg("SQ_LDS_BANK_CONFLICT") / max(avg("SQ_LDS_IDX_ACTIVE"), 1.0)
        l2_hit = avg("TCC_HIT_sum") / max(avg("TCC_HIT_sum") + avg("TCC_MISS_sum"), 1.0)
        fe = _dispatch_counters(os.path.join(d, "fetch"))
        copy = [v["FETCH_SIZE"] for v in fe.values() if "copy" in v["name"].lower()]
        gem = [v["FETCH_SIZE"] for v in fe.values() if "tg::" in v["name"]]
        factor = COPY_BYTES / (sum(copy) / len(copy) * 1024.0)
        read = sum(gem) / len(gem) * 1024.0 * factor
        ab = 2.0 * (w.M * w.K + w.K * w.N) * w.batch
        rows.append((label, desc, b["ms_per_step"] * 1e3, b["value"], b["unit"], clock, mfma,
                     lds_conf, l2_hit, read / ab, n))
    with open(out_md, "w") as f:
        f.write(f"# {title}\n\nCommands (from the repository root on the GPU box; "
                f"<label> and <args> per row):\n\n")
        for c in commands.splitlines():
            f.write(f"    {c}\n")
        f.write("\nRate and time from the bench line; clock, MFMA-busy fraction, LDS bank-conflict "
                "cycles per LDS-active cycle and L2 hit rate averaged over the profiled "
                "dispatches; HBM read = FETCH_SIZE x the factor a 1 GiB copy gives, per launch, "
                "over the bytes of A and B.\n\n")
        f.write("| run | setting | us / call | rate | clock GHz | MFMA busy | LDS conflict | "
                "L2 hit | HBM read / (A+B) |\n|---|---|---|---|---|---|---|---|---|\n")
        for (label, desc, us, val, unit, clock, mfma, lc, l2, rd, n) in rows:
            f.write(f"| {label} | {desc} | {us:.1f} | {val:.0f} {unit} | {clock:.2f} | "
                    f"{mfma:.1%} | {lc:.3f} | {l2:.1%} | {rd:.2f} |\n")
    print(f"wrote {out_md}")


PMC_SET = ("SQ_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_LDS_BANK_CONFLICT "
           "SQ_LDS_IDX_ACTIVE GRBM_GUI_ACTIVE TCC_HIT_sum TCC_MISS_sum")


def summarize_run(workload: str, root: str, commands: list[str]):
    """Writes profiles/<kernel family>-<workload>.md for the default kernel of a
    dense workload from one directory of runs:
      root/bench.json  the JSON line of a bench run made under
                       `rocprofv3 --kernel-trace --stats -d root/trace`
                       (the trace and the line come from the same invocation),
      root/pmc         one --pmc run of PMC_SET,
      root/fetch       one --pmc FETCH_SIZE run with --calibrate-copy,
      root/write       one --pmc WRITE_SIZE run with --calibrate-copy,
    and records the calibrated HBM bytes per launch in profiles/traffic.txt.
    The summary recomputes the roofline fraction from the trace's average
    kernel duration next to the bench line's own."""
    import collections
    with open(os.path.join(root, "bench.json")) as f:
        b = json.loads([ln for ln in f.read().splitlines() if ln.startswith("{")][-1])
    w = wl.WORKLOADS[workload]
    stats = _csv_rows(_find(os.path.join(root, "trace"), "kernel_stats.csv"))
    stats.sort(key=lambda r: -float(r["TotalDurationNs"]))
    top = stats[0]
    name = top["Name"]
    short = name.replace("tg::(anonymous namespace)::", "")
    pmc = [v for v in _dispatch_counters(os.path.join(root, "pmc")).values()
           if v["name"] == name]
    n = len(pmc)
    avg = lambda key: sum(v[key] for v in pmc) / n
    # SQ_CYCLES is summed over the 32 shader engines, GRBM_GUI_ACTIVE over the
    # 8 XCDs
    clock = sum(v["SQ_CYCLES"] / 32 / v["us"] / 1e3 for v in pmc) / n
    gui = sum(v["GRBM_GUI_ACTIVE"] / 8 / v["us"] / 1e3 for v in pmc) / n
    mfma = sum(v["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * v["SQ_CYCLES"] / 32) for v in pmc) / n
    lds_conf = avg("SQ_LDS_BANK_CONFLICT") / max(avg("SQ_LDS_IDX_ACTIVE"), 1.0)
    l2_hit = avg("TCC_HIT_sum") / max(avg("TCC_HIT_sum") + avg("TCC_MISS_sum"), 1.0)
    pmc_us = avg("us")

    def per_launch(sub, counter):
        d = _dispatch_counters(os.path.join(root, sub))
        copy = [v[counter] for v in d.values() if "copy" in v["name"].lower()]
        gem = [v[counter] for v in d.values() if v["name"] == name]
        factor = COPY_BYTES / (sum(copy) / len(copy) * 1024.0)
        return sum(gem) / len(gem) * 1024.0 * factor, factor, sum(copy) / len(copy) * 1024.0

    g_fetch, f_fetch, c_fetch = per_launch("fetch", "FETCH_SIZE")
    g_write, f_write, c_write = per_launch("write", "WRITE_SIZE")
    reads = 2 * (w.M * w.K + w.K * w.N) * w.batch
    writes = 2 * w.M * w.N * w.batch
    trace_ns = float(top["AverageNs"])
    compute = b["roofline"]["bound"] == "mfma"
    work = w.flops if compute else w.compulsory_bytes
    scale = 1e12 if compute else 1e9
    peak = PEAK_F16_TFLOPS if compute else PEAK_HBM_GBS
    unit = "TFLOP/s" if compute else "GB/s"
    rate_trace = work / (trace_ns * 1e-9) / scale
    family = ("gemm_relu_dma_stream_kernel" if "dma_stream_kernel" in name else
              "gemm_relu_dma_kernel" if "dma_kernel" in name else
              "gemm_relu_ragged_kernel" if "ragged_kernel" in name else
              "gemm_relu_skinny_kernel" if "skinny_kernel" in name else
              "gemm_relu_tile_kernel" if "tile_kernel" in name else "kernel")
    md = os.path.join(PROFILES, f"{family}-{workload}.md")
    t = b.get("timing", {})
    with open(md, "w") as f:
        f.write(f"# {short} on {workload}\n\n")
        f.write("Commands (from the repository root on the GPU box, R = that root):\n\n")
        for c in commands:
            f.write(f"    {c}\n")
        f.write(f"\n## Bench line of the traced run\n\n")
        f.write(f"* contract window: {b['steps']} calls after {b['warmup']} warm-ups, "
                f"{b['ms_per_step'] * 1e3:.1f} us per call, {b['value']:.1f} {b['unit']}, "
                f"frac {b['roofline']['frac']:.3f} of {b['roofline']['peak']} {unit}\n")
        if "median_ms_per_call" in t:
            f.write(f"* trials before it: {t['trials']} x {t['calls_per_trial']} calls, per call "
                    f"median {t['median_ms_per_call'] * 1e3:.1f} us, min "
                    f"{t['min_ms_per_call'] * 1e3:.1f} us, max {t['max_ms_per_call'] * 1e3:.1f} us "
                    f"({t['rate_at_median']:.1f} / {t['rate_at_min']:.1f} {unit} at median / min)\n")
        sc = b.get("sclk_mhz")
        if sc:
            f.write(f"* shader clock sampled during the trials ({sc['source']}): median "
                    f"{sc['median']:.0f} MHz, range {sc['min']:.0f}-{sc['max']:.0f} MHz, "
                    f"{sc['samples']} samples\n")
        f.write("\n## Kernel trace of the same invocation (rocprofv3 --kernel-trace --stats)\n\n")
        f.write("| kernel | calls | average ns | min ns | max ns |\n|---|---|---|---|---|\n")
        for r in stats[:4]:
            nm = r["Name"].replace("tg::(anonymous namespace)::", "")
            f.write(f"| {nm[:140]} | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                    f"{float(r['MinNs']):.0f} | {float(r['MaxNs']):.0f} |\n")
        f.write(f"\nAlgorithmic work per launch: {w.flops:.4e} flop, "
                f"{w.compulsory_bytes:.4e} compulsory HBM bytes.  From the trace's average "
                f"({trace_ns / 1e3:.1f} us over every call of the run: warm-ups, trials and the "
                f"window): {rate_trace:.1f} {unit} = {rate_trace / peak:.3f} of {peak} {unit}; "
                f"trace average / ms_per_step = {trace_ns / 1e6 / b['ms_per_step']:.3f}.\n")
        f.write(f"\n## Counters (rocprofv3 --pmc, one set per run), {n} dispatches\n\n")
        f.write(f"* shader clock {clock:.2f} GHz (SQ_CYCLES per shader engine / kernel time; "
                f"GRBM_GUI_ACTIVE per XCD gives {gui:.2f} GHz), kernel time under the counters "
                f"{pmc_us:.1f} us"
                + ("; for a launch this short the counters' window is longer than the kernel, "
                   "so this clock reads high and the busy fraction below is relative to it"
                   if pmc_us < 100 else "") + "\n")
        f.write(f"* matrix cores busy {mfma:.1%} of the SIMD cycles "
                f"(SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x SQ_CYCLES per engine)); "
                f"at that clock the busy fraction corresponds to "
                f"{mfma * clock / 2.4 * PEAK_F16_TFLOPS:.0f} TFLOP/s of issued matrix work\n")
        f.write(f"* LDS bank-conflict cycles per LDS-active cycle {lds_conf:.4f} "
                f"(SQ_LDS_BANK_CONFLICT {avg('SQ_LDS_BANK_CONFLICT'):.4e}, "
                f"SQ_LDS_IDX_ACTIVE {avg('SQ_LDS_IDX_ACTIVE'):.4e})\n")
        f.write(f"* L2 hit rate {l2_hit:.1%} (TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum))\n")
        f.write(f"* calibration copy of {COPY_BYTES} bytes: FETCH_SIZE {c_fetch:.4e} B, "
                f"WRITE_SIZE {c_write:.4e} B -> factors {f_fetch:.3f} (fetch), "
                f"{f_write:.3f} (write)\n")
        f.write(f"* HBM read {g_fetch:.4e} B per launch ({g_fetch / reads:.2f} x the "
                f"{reads:.4e} B of A and B), HBM write {g_write:.4e} B ({g_write / writes:.2f} "
                f"x the {writes:.4e} B of C)\n")
        f.write(f"* kernel source hash {kernel_source_hash(workload)} "
                f"({', '.join(KERNEL_SOURCES.get(workload, DEFAULT_SOURCES))})\n")
    lines = {k: v for k, v in read_traffic_file().items()}
    lines[workload] = (kernel_source_hash(workload), g_fetch, g_write)
    with open(TRAFFIC_FILE, "w") as f:
        f.write("# workload source_hash hbm_read_bytes hbm_write_bytes (per launch, calibrated)\n")
        for k, (h, r_, w_) in sorted(lines.items()):
            f.write(f"{k} {h} {r_:.6e} {w_:.6e}\n")
    print(f"wrote {md} and {TRAFFIC_FILE}")


def summarize_stats(out_md: str, title: str, stats_dir: str, commands: list[str]):
    """Writes a kernel-trace summary (top kernels by total time) for runs that
    are not one of the dense workloads (the int4 and attention benches)."""
    stats = _csv_rows(_find(stats_dir, "kernel_stats.csv"))
    stats.sort(key=lambda r: -float(r["TotalDurationNs"]))
    with open(out_md, "w") as f:
        f.write(f"# {title}\n\nCommands (from the repository root on the GPU box):\n\n")
        for c in commands:
            f.write(f"    {c}\n")
        f.write("\nKernel trace (rocprofv3 --kernel-trace --stats), top kernels:\n\n")
        f.write("| kernel | calls | average ns | min ns | max ns |\n|---|---|---|---|---|\n")
        for r in stats[:4]:
            name = r["Name"].replace("tg::(anonymous namespace)::", "")
            f.write(f"| {name[:120]} | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                    f"{float(r['MinNs']):.0f} | {float(r['MaxNs']):.0f} |\n")
    print(f"wrote {out_md}")


def attention_line(tg, torch, causal: bool, kv_heads: int, steps: int, warmup: int,
                   trials: int) -> dict:
    """One line for the fused attention forward, 4 x 4096 x 32 heads x 128."""
    B, S, H, D = 4, 4096, 32, 128
    timing = run_attention(tg, torch, B, S, H, kv_heads, D, causal, steps, warmup, trials)
    ms = timing["ms_per_step"]
    # two products of 2*S*S*D flop per (batch, head); half the pairs when causal
    flops = 4.0 * B * H * S * S * D * (0.5 if causal else 1.0)
    tflops = flops / (ms * 1e-3) / 1e12
    name = f"attention_{B}x{S}x{H}x{D}" + (f"_kv{kv_heads}" if kv_heads != H else "")
    mode = "causal" if causal else "full"
    log(f"{name} {mode}: {ms * 1e3:.1f} us/call, {tflops:.1f} TFLOP/s")
    return {
        "metric": "TFLOP/s fused attention forward", "value": tflops, "unit": "TFLOP/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"{name}_{mode}", "batch": B, "seq": S, "heads": H,
                   "kv_heads": kv_heads, "head_dim": D, "causal": causal,
                   "path": tg.tg_path_name(tg.tg_last_path())},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": PEAK_F16_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / PEAK_F16_TFLOPS, "traffic": None},
        "timing": timing_fields(timing, None, flops, 1e12)[0]}


def mla_line(tg, torch, steps: int, warmup: int, trials: int) -> dict:
    """One line for the latent-attention decode, 64 x 8192 x 128 heads."""
    w = wl.MLA_WORKLOAD
    B, H, Sk = w["B"], w["H"], w["Sk"]
    timing, path, need = run_mla(tg, torch, steps, warmup, trials)
    ms = timing["ms_per_step"]
    # score product over 576 values and value product over 512, per (sequence, head, token)
    flops = 2.0 * B * H * Sk * (576 + 512)
    nbytes = 2.0 * (B * Sk * 576 + B * H * 576 + B * H * 512)
    tflops = flops / (ms * 1e-3) / 1e12
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"{w['name']}: {ms * 1e3:.1f} us/call, {tflops:.1f} TFLOP/s, {gbs:.0f} GB/s, "
        f"workspace {need} bytes")
    return {
        "metric": "GB/s latent-attention decode", "value": gbs, "unit": "GB/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w["name"], "batch": B, "heads": H, "seq_k": Sk,
                   "row": "512+64", "tflops": tflops, "path": path, "splits": -1,
                   "workspace_bytes": need},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs / PEAK_HBM_GBS, "traffic": None},
        "timing": timing_fields(timing, None, nbytes, 1e9)[0]}


def w4_line(tg, torch, dtype: str, steps: int, warmup: int, trials: int) -> dict:
    """One line for the weight-only int4 GEMM+ReLU at the decode shape."""
    M, N, K, G = 16, 16384, 8192, 128
    timing, path, nbuf, nbytes = run_w4(tg, torch, M, N, K, G, steps, warmup, dtype, trials)
    ms = timing["ms_per_step"]
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"w4 {M}x{N}x{K} g{G}: {ms * 1e3:.1f} us/call, {gbs:.0f} GB/s, path={path}")
    return {
        "metric": "GB/s weight-only int4 GEMM+ReLU (decode shape)", "value": gbs,
        "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype, "data": "synthetic",
        "config": {"workload": f"w4_{M}x{N}x{K}_g{G}", "M": M, "N": N, "K": K,
                   "group_size": G, "path": path, "weight_copies": nbuf},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs / PEAK_HBM_GBS, "traffic": None},
        "timing": timing_fields(timing, None, nbytes, 1e9)[0]}


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-run":
        # bench.py --summarize-run WORKLOAD ROOT_DIR "cmd1" ...
        summarize_run(sys.argv[2], sys.argv[3], sys.argv[4:])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-stats":
        # bench.py --summarize-stats OUT_MD TITLE STATS_DIR "cmd1" ...
        summarize_stats(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5:])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-ablation":
        # bench.py --summarize-ablation OUT_MD ROOT_DIR TITLE
        summarize_ablation(sys.argv[2], sys.argv[3], sys.argv[4])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize":
        # bench.py --summarize WORKLOAD STATS_DIR FETCH_DIR WRITE_DIR "cmd1" "cmd2" ...
        summarize(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], sys.argv[6:])
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="large_8192", choices=sorted(wl.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a 1 GiB copy first (counter calibration runs only)")
    ap.add_argument("--tile-variant", type=int, default=-1,
                    help="tile-kernel configuration (tg_set_tile_variant), -1 = default")
    ap.add_argument("--skinny-variant", type=int, default=-1,
                    help="skinny-kernel configuration (tg_set_skinny_variant), -1 = default")
    ap.add_argument("--raster", type=int, default=-1,
                    help="tile order (tg_set_raster): panel height, 0 = row-major, -1 = default")
    ap.add_argument("--act", choices=["relu", "none"], default="relu",
                    help="epilogue activation (none: through tg_gemm_ex)")
    ap.add_argument("--bias", action="store_true",
                    help="add a per-column bias in the epilogue (through tg_gemm_ex)")
    ap.add_argument("--dtype", choices=["f16", "bf16"], default="f16",
                    help="element type (bf16: through tg_gemm_ex)")
    ap.add_argument("--layout", choices=["kn", "nk"], default="kn",
                    help="B stored (K,N) or (N,K) (nk: through tg_gemm_ex)")
    ap.add_argument("--attention", choices=["full", "causal"], default=None,
                    help="time the fused attention forward on 4 x 4096 x 32 heads x 128 "
                         "(tg_attention_fwd_f16) and exit")
    ap.add_argument("--kv-heads", type=int, default=32,
                    help="key/value heads of the attention bench (32: multi-head; a divisor "
                         "of 32: grouped-query, tg_attention_fwd_f16_gqa)")
    ap.add_argument("--attention-variant", type=int, default=-1,
                    help="attention workgroup shape (tg_set_attention_variant)")
    ap.add_argument("--mla", action="store_true",
                    help="time the latent-attention decode on 64 sequences x 8192 cached "
                         "tokens x 128 heads, rows of 512 + 64 (tg_mla_decode_f16) and exit")
    ap.add_argument("--mla-splits", type=int, default=-1,
                    help="key ranges per sequence of the decode bench (tg_set_mla_splits)")
    ap.add_argument("--skinny-splitk", type=int, default=0, metavar="S",
                    help="ablation: time the split-K form (S chunks of K, fp32 partials in a "
                         "workspace, tg_gemm_relu_f16_splitk) on the skinny workload and exit")
    ap.add_argument("--trials", type=int, default=TRIALS,
                    help=f"timed trials of >= {TRIAL_MS:.0f} ms before the contract window "
                         "(median and min reported; 0 skips them)")
    ap.add_argument("--graph", action="store_true",
                    help="capture the timed calls into one HIP graph and time its replay")
    ap.add_argument("--w4", action="store_true",
                    help="time the weight-only int4 GEMM on the decode shape "
                         "16 x 16384 x 8192, groups of 128 (tg_gemm_w4) and exit")
    ap.add_argument("--vendor", action="store_true",
                    help="context only: time the vendor GEMM (torch.matmul, i.e. hipBLASLt) "
                         "on the same operands, without the ReLU, and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this library runs the GEMM on a single "
              f"device and has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import tiled_dense_gemm_05_amd as tg

    knobs = {}
    for name, value, setter in (("tile_variant", args.tile_variant, tg.tg_set_tile_variant),
                                ("skinny_variant", args.skinny_variant, tg.tg_set_skinny_variant),
                                ("raster", args.raster, tg.tg_set_raster)):
        if value != -1:
            if setter(value) < -1:
                print(f"invalid --{name.replace('_', '-')} {value}", file=sys.stderr)
                sys.exit(2)
            knobs[name] = value
    epilogue = None
    if args.bias or args.act != "relu":
        epilogue = (tg.TG_ACT_RELU if args.act == "relu" else tg.TG_ACT_NONE, args.bias)
        knobs["epilogue"] = ("bias+" if args.bias else "") + args.act
    if args.layout != "kn":
        knobs["b_layout"] = args.layout
    if args.graph:
        knobs["graph"] = True
    if args.calibrate_copy:
        calibration_copy(torch)
    if args.vendor:
        w = wl.WORKLOADS[args.workload]
        timing = run_vendor(torch, w, args.steps, args.warmup, args.dtype, args.layout,
                            args.trials)
        ms = timing["ms_per_step"]
        rate = w.flops / (ms * 1e-3) / 1e12
        log(f"vendor {args.workload} {args.dtype} {args.layout}: {ms * 1e3:.1f} us/call, "
            f"{rate:.1f} TFLOP/s")
        print(json.dumps({
            "metric": "TFLOP/s vendor fp16 GEMM (context, no ReLU)", "value": rate,
            "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": args.dtype, "data": "synthetic",
            "config": {"workload": args.workload, "M": w.M, "N": w.N, "K": w.K,
                       "batch": w.batch, "b_layout": args.layout,
                       "library": "torch.matmul (hipBLASLt)"},
            "timing": timing_fields(timing, None, w.flops, 1e12)[0]}), flush=True)
        return
    if args.attention:
        if args.attention_variant != -1:
            tg.tg_set_attention_variant(args.attention_variant)
        if args.kv_heads <= 0 or 32 % args.kv_heads:
            sys.exit("--kv-heads must divide 32")
        print(json.dumps(attention_line(tg, torch, args.attention == "causal", args.kv_heads,
                                        args.steps, args.warmup, args.trials)), flush=True)
        return
    if args.skinny_splitk:
        w = wl.WORKLOADS["skinny_16x16384x8192"]
        S = args.skinny_splitk
        timing, nbuf, need = run_splitk(tg, torch, S, args.steps, args.warmup, args.trials)
        ms = timing["ms_per_step"]
        gbs = w.compulsory_bytes / (ms * 1e-3) / 1e9
        log(f"skinny split-K S={S}: {ms * 1e3:.1f} us/call, {gbs:.0f} GB/s, workspace {need} bytes")
        print(json.dumps({
            "metric": "GB/s fp16 GEMM+ReLU at M=16, split-K form (ablation)", "value": gbs,
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "f16", "data": "synthetic",
            "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "splits": S,
                       "input_copies": nbuf, "workspace_bytes": need},
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS, "traffic": None},
            "timing": timing_fields(timing, None, w.compulsory_bytes, 1e9)[0]}), flush=True)
        return
    if args.mla:
        if args.mla_splits != -1:
            tg.tg_set_mla_splits(args.mla_splits)
        line = mla_line(tg, torch, args.steps, args.warmup, args.trials)
        line["config"]["splits"] = args.mla_splits
        print(json.dumps(line), flush=True)
        return
    if args.w4:
        print(json.dumps(w4_line(tg, torch, args.dtype, args.steps, args.warmup, args.trials)),
              flush=True)
        return
    w = wl.WORKLOADS[args.workload]
    log(f"workload {w.name}: M={w.M} N={w.N} K={w.K} batch={w.batch}")
    clock = ClockSampler(torch) if args.trials > 0 else None
    timing, path, nbuf = run_workload(tg, torch, w, args.steps, args.warmup, epilogue,
                                      args.dtype, args.layout, graph=args.graph, clock=clock,
                                      trials=args.trials)
    ms = timing["ms_per_step"]
    tflops = w.flops / (ms * 1e-3) / 1e12
    gbs = w.compulsory_bytes / (ms * 1e-3) / 1e9
    compute_bound = w.flops / w.compulsory_bytes > PEAK_F16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    log(f"{w.name}: {ms * 1e3:.1f} us/call, {tflops:.1f} TFLOP/s, {gbs:.0f} GB/s, path={path}")

    if compute_bound:
        value, unit = tflops, "TFLOP/s"
        roof = {"bound": "mfma", "achieved": tflops, "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                "frac": tflops / PEAK_F16_TFLOPS}
        tfields, sclk = timing_fields(timing, clock, w.flops, 1e12)
    else:
        value, unit = gbs, "GB/s"
        roof = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": gbs / PEAK_HBM_GBS}
        tfields, sclk = timing_fields(timing, clock, w.compulsory_bytes, 1e9)
    if "median_ms_per_call" in timing:
        log(f"{w.name}: trials median {timing['median_ms_per_call'] * 1e3:.1f} us, min "
            f"{timing['min_ms_per_call'] * 1e3:.1f} us ({timing['calls_per_trial']} calls each); "
            f"sclk {sclk}")
    if args.dtype != "f16":
        knobs["element"] = args.dtype
    roof["traffic"] = None if knobs else measured_traffic(w.name)

    out = {
        "metric": METRIC,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "batch": w.batch,
                   "inputs": f"{w.dist}, seed {w.seed}", "accumulate": "fp32", "path": path,
                   "input_copies": nbuf, **knobs},
        "roofline": roof,
        "timing": tfields,
        "sclk_mhz": sclk,
    }

    def side_line(s, steps):
        """The same protocol on another workload: one object for the JSON line."""
        if clock is not None:
            clock.reset()
        stiming, spath, snbuf = run_workload(tg, torch, s, steps, args.warmup, epilogue,
                                             args.dtype, args.layout, graph=args.graph,
                                             clock=clock, trials=args.trials)
        sms = stiming["ms_per_step"]
        stf_flops = s.flops / (sms * 1e-3) / 1e12
        sgbs = s.compulsory_bytes / (sms * 1e-3) / 1e9
        log(f"{s.name}: {sms * 1e3:.1f} us/call, {stf_flops:.1f} TFLOP/s, {sgbs:.0f} GB/s, "
            f"path={spath}")
        if s.flops / s.compulsory_bytes > PEAK_F16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
            sval, sunit = stf_flops, "TFLOP/s"
            sroof = {"bound": "mfma", "achieved": stf_flops, "peak": PEAK_F16_TFLOPS,
                     "unit": "TFLOP/s", "frac": stf_flops / PEAK_F16_TFLOPS}
            stf, ssclk = timing_fields(stiming, clock, s.flops, 1e12)
        else:
            sval, sunit = sgbs, "GB/s"
            sroof = {"bound": "hbm", "achieved": sgbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": sgbs / PEAK_HBM_GBS}
            stf, ssclk = timing_fields(stiming, clock, s.compulsory_bytes, 1e9)
        sroof["traffic"] = None if knobs else measured_traffic(s.name)
        return {"workload": s.name, "value": sval, "unit": sunit, "ms_per_step": sms,
                "path": spath, "steps": steps, "input_copies": snbuf, "roofline": sroof,
                "timing": stf, "sclk_mhz": ssclk}

    if not args.no_secondary and w.name != "skinny_16x16384x8192":
        out["secondary"] = side_line(wl.WORKLOADS["skinny_16x16384x8192"], max(args.steps, 20))
    if not args.no_secondary and w.name == "large_8192":
        # the other workloads of the hot-path table, each on its own protocol
        # run (inputs resident in HBM, trials, then a window of its own steps)
        out["other_workloads"] = [
            side_line(wl.WORKLOADS[name], max(args.steps, 20))
            for name in ("mid_2048", "batched_1024x128x128x64", "ragged_3001x5003x1000",
                         "small_512")]
        # the measured NEXT rows (attention forward full and causal, the
        # latent-attention decode, int4 weights), their own lines as objects
        st = max(args.steps, 20)
        out["next_rows"] = [attention_line(tg, torch, False, 32, st, args.warmup, args.trials),
                            attention_line(tg, torch, True, 32, st, args.warmup, args.trials),
                            mla_line(tg, torch, st, args.warmup, args.trials),
                            w4_line(tg, torch, "f16", st, args.warmup, args.trials)]

    if not args.no_cpu_baseline:
        log("timing the oracle on the host cores ...")
        out["cpu_baseline"] = cpu_baseline(w)
        log(f"oracle: {out['cpu_baseline']['value'] * 1e3:.2f} GFLOP/s "
            f"({out['cpu_baseline']['cores']} threads)")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
