// Internal interface of the split-K skinny path: entry point (splitk_api.cpp)
// to kernels (gemm_skinny.hip).
#pragma once

#include "tg_internal.h"

namespace tg {

// C = ReLU(A B) for an aligned skinny problem (the skinny kernel's layout
// rules, M <= 64, batch 1) as `splits` K chunks of whole 32-k steps: each
// chunk's fp32 sums go to part[chunk] ((M, N) row-major, M * N floats each),
// then a second kernel adds the chunks in order, applies the ReLU and rounds
// to fp16.  splits <= 65535.
hipError_t launch_skinny_splitk(const GemmArgs &p, int64_t splits, float *part,
                                hipStream_t stream);

}  // namespace tg
