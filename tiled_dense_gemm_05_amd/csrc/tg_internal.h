// Internal interface between the host dispatcher (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tg {

// One strided-batched problem, sizes and strides in elements.  The host has
// validated it; every kernel masks its own edges, so any M, N, K >= 0 is safe
// for the layouts the ABI documents.
struct GemmArgs {
    const uint16_t *A;
    const uint16_t *B;
    uint16_t *C;
    int64_t M, N, K;
    int64_t lda, ldb, ldc;
    int64_t sA, sB, sC;
    int64_t batch;
};

// Every launcher enqueues on `stream` and returns hipGetLastError().
hipError_t launch_naive(const GemmArgs &p, hipStream_t stream);
hipError_t launch_generic(const GemmArgs &p, hipStream_t stream);
hipError_t launch_tile128(const GemmArgs &p, hipStream_t stream);
hipError_t launch_tile256(const GemmArgs &p, hipStream_t stream);

// Direct-to-LDS pipelined kernels (aligned layouts only).  `cfg` selects the
// block tile / K tile / stage count; see gemm_dma.hip.
constexpr int kDmaConfigs = 22;
hipError_t launch_dma_config(int cfg, const GemmArgs &p, hipStream_t stream, int groupM);
// Skinny-M kernels (M <= 64, aligned layouts); `cfg` selects slice width,
// waves and stages; see gemm_skinny.hip.
constexpr int kSkinnyConfigs = 10;
hipError_t launch_skinny_config(int cfg, const GemmArgs &p, hipStream_t stream);
bool skinny_layout_ok(const GemmArgs &p);
// Whether the leading dimensions fit the kernels' 32-bit buffer offsets.
bool dma_layout_ok(const GemmArgs &p);

}  // namespace tg
