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

// Argument checks shared by the split-K entry points (everything but the
// workspace): TG_OK with p filled in for the launch, or an error status.
// M == 0 or N == 0 returns TG_OK with p untouched (a no-op call).
int splitk_check(const void *A, const void *B, const void *C, int64_t M, int64_t N, int64_t K,
                 int64_t lda, int64_t ldb, int64_t ldc, int64_t splits, GemmArgs &p);

}  // namespace tg
