// Times tg_gemm_relu_f16 through the C ABI from C++ alone (no Python, no
// torch): the cross-check of the Python benchmark's timings.
//
//   tg_capi_bench [M N K [iters [copies]]]      (default 8192 8192 8192 50 1)
//
// Operands are row-major fp16 with entries normal(0, 1/sqrt(K)) from a
// seeded generator; `copies` independent operand sets are used in turn so
// that HBM-bound shapes are not served from the last-level cache.  Prints one
// JSON line: microseconds per call (HIP events on the launch stream around
// `iters` back-to-back calls after 10 warm-ups), TFLOP/s, GB/s of compulsory
// traffic and the kernel path.
#include "tg.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

namespace {

bool ok(hipError_t e, const char *what)
{
    if (e == hipSuccess)
        return true;
    std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return false;
}

uint16_t f16_bits(float x)
{
    const _Float16 h = (_Float16)x;   // round to nearest even
    uint16_t u;
    std::memcpy(&u, &h, sizeof(u));
    return u;
}

}  // namespace

int main(int argc, char **argv)
{
    const int64_t M = argc > 1 ? std::atoll(argv[1]) : 8192;
    const int64_t N = argc > 2 ? std::atoll(argv[2]) : 8192;
    const int64_t K = argc > 3 ? std::atoll(argv[3]) : 8192;
    const int iters = argc > 4 ? std::atoi(argv[4]) : 50;
    const int copies = argc > 5 ? std::atoi(argv[5]) : 1;
    if (M <= 0 || N <= 0 || K <= 0 || iters <= 0 || copies <= 0) {
        std::fprintf(stderr, "usage: %s [M N K [iters [copies]]]\n", argv[0]);
        return 2;
    }
    std::mt19937_64 rng(2);
    std::normal_distribution<float> nd(0.0f, 1.0f / std::sqrt((float)K));
    std::vector<uint16_t> a((size_t)(M * K)), b((size_t)(K * N));
    for (auto &v : a)
        v = f16_bits(nd(rng));
    for (auto &v : b)
        v = f16_bits(nd(rng));

    std::vector<void *> dA(copies), dB(copies), dC(copies);
    for (int c = 0; c < copies; ++c) {
        if (!ok(hipMalloc(&dA[c], a.size() * 2), "hipMalloc A") ||
            !ok(hipMalloc(&dB[c], b.size() * 2), "hipMalloc B") ||
            !ok(hipMalloc(&dC[c], (size_t)(M * N) * 2), "hipMalloc C") ||
            !ok(hipMemcpy(dA[c], a.data(), a.size() * 2, hipMemcpyHostToDevice), "copy A") ||
            !ok(hipMemcpy(dB[c], b.data(), b.size() * 2, hipMemcpyHostToDevice), "copy B"))
            return 1;
    }
    hipStream_t s;
    hipEvent_t e0, e1;
    if (!ok(hipStreamCreate(&s), "stream") || !ok(hipEventCreate(&e0), "event") ||
        !ok(hipEventCreate(&e1), "event"))
        return 1;
    auto call = [&](int i) {
        const int c = i % copies;
        return tg_gemm_relu_f16(dA[c], dB[c], dC[c], M, N, K, K, N, N, s);
    };
    for (int i = 0; i < 10; ++i) {
        const int st = call(i);
        if (st != TG_OK) {
            std::fprintf(stderr, "tg_gemm_relu_f16: %s\n", tg_status_string(st));
            return 1;
        }
    }
    if (!ok(hipStreamSynchronize(s), "sync") || !ok(hipEventRecord(e0, s), "record"))
        return 1;
    for (int i = 0; i < iters; ++i)
        call(i);
    float ms = 0.0f;
    if (!ok(hipEventRecord(e1, s), "record") || !ok(hipEventSynchronize(e1), "sync") ||
        !ok(hipEventElapsedTime(&ms, e0, e1), "elapsed"))
        return 1;
    const double us = 1e3 * ms / iters;
    const double tflops = 2.0 * M * N * K / (us * 1e-6) / 1e12;
    const double gbs = 2.0 * (M * K + K * N + M * N) / (us * 1e-6) / 1e9;
    std::printf("{\"M\": %lld, \"N\": %lld, \"K\": %lld, \"iters\": %d, \"copies\": %d, "
                "\"us_per_call\": %.2f, \"tflops\": %.1f, \"gbs\": %.0f, \"path\": \"%s\"}\n",
                (long long)M, (long long)N, (long long)K, iters, copies, us, tflops, gbs,
                tg_path_name(tg_last_path()));
    for (int c = 0; c < copies; ++c) {
        (void)hipFree(dA[c]);
        (void)hipFree(dB[c]);
        (void)hipFree(dC[c]);
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    (void)hipStreamDestroy(s);
    return 0;
}
