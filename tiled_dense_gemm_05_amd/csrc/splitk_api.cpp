// C ABI of the split-K skinny GEMM+ReLU: argument validation and launch.
// Declarations and the contract are in include/tg.h.
#include "tg.h"

#include <cstdint>

#include "tg_splitk.h"

namespace {

constexpr int64_t kMaxDim = 0x7fffffff;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

bool sizes_ok(int64_t M, int64_t N, int64_t splits)
{
    return M >= 0 && M <= 64 && N >= 0 && N <= kMaxDim && splits >= 1 && splits <= 65535;
}

}  // namespace

namespace tg {

int splitk_check(const void *A, const void *B, const void *C, int64_t M, int64_t N, int64_t K,
                 int64_t lda, int64_t ldb, int64_t ldc, int64_t splits, GemmArgs &p)
{
    if (!sizes_ok(M, N, splits) || K < 0 || K > kMaxDim)
        return TG_ERR_INVALID_ARG;
    if (lda < (K > 1 ? K : 1) || ldb < (N > 1 ? N : 1) || ldc < (N > 1 ? N : 1))
        return TG_ERR_INVALID_ARG;
    // the skinny kernel's layout: whole 16-byte chunks everywhere
    if (N % 8 != 0 || K % 8 != 0 || lda % 8 != 0 || ldb % 8 != 0 || ldc % 8 != 0)
        return TG_ERR_INVALID_ARG;
    if (M == 0 || N == 0)
        return TG_OK;
    if (C == nullptr || (K > 0 && (A == nullptr || B == nullptr)))
        return TG_ERR_INVALID_ARG;
    if (!aligned16(C) || (K > 0 && (!aligned16(A) || !aligned16(B))))
        return TG_ERR_INVALID_ARG;
    if (splits > (K + 31) / 32 && splits > 1)   // every chunk holds a 32-k step
        return TG_ERR_INVALID_ARG;
    p = GemmArgs{};
    p.A = static_cast<const uint16_t *>(A);
    p.B = static_cast<const uint16_t *>(B);
    p.C = static_cast<uint16_t *>(const_cast<void *>(C));
    p.M = M; p.N = N; p.K = K;
    p.lda = lda; p.ldb = ldb; p.ldc = ldc;
    p.batch = 1;
    p.relu = 1;
    if (!skinny_layout_ok(p))
        return TG_ERR_INVALID_ARG;
    return TG_OK;
}

}  // namespace tg

extern "C" {

int64_t tg_gemm_splitk_workspace_bytes(int64_t M, int64_t N, int64_t splits)
{
    if (!sizes_ok(M, N, splits))
        return -1;
    return splits * M * N * (int64_t)sizeof(float);
}

int tg_gemm_relu_f16_splitk(const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K,
                            int64_t lda, int64_t ldb, int64_t ldc, int64_t splits,
                            void *workspace, int64_t workspace_bytes, hipStream_t stream)
{
    tg::GemmArgs p{};
    int st = tg::splitk_check(A, B, C, M, N, K, lda, ldb, ldc, splits, p);
    if (st != TG_OK || M == 0 || N == 0)
        return st;
    if (workspace == nullptr || !aligned16(workspace) ||
        workspace_bytes < splits * M * N * (int64_t)sizeof(float))
        return TG_ERR_INVALID_ARG;
    st = tg::host_check_device();
    if (st != TG_OK)
        return st;
    if (tg::launch_skinny_splitk(p, splits, static_cast<float *>(workspace), stream) != hipSuccess)
        return TG_ERR_HIP;
    tg::host_set_last_path(TG_PATH_SKINNY);
    return TG_OK;
}

}  // extern "C"
