// The plain kernel: one thread per output element, fp32 fused multiply-add
// over k in ascending order, bias, ReLU, round-to-nearest-even store; element
// type (fp16 or bf16) and B layout ((K,N) or (N,K)) are read at run time.
// It is the literal reading of the GEMM+ReLU program of the "TileLang paper
// reading" page, section 2, without tiles; it serves as a slow cross-check
// path.
#include "tg_internal.h"

namespace tg {
namespace {

__global__ void __launch_bounds__(256) gemm_relu_naive_kernel(GemmArgs p)
{
    const int64_t per_batch = p.M * p.N;
    const int64_t total = per_batch * p.batch;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t b = e / per_batch;
        const int64_t r = e - b * per_batch;
        const int64_t i = r / p.N;
        const int64_t j = r - i * p.N;
        const uint16_t *a = p.A + b * p.sA + i * p.lda;
        // B(k, j) at bc[k * kstride]
        const uint16_t *bc = p.B + b * p.sB + (p.b_nk ? j * p.ldb : j);
        const int64_t kstride = p.b_nk ? 1 : p.ldb;
        const bool bf = p.bf16 != 0;
        auto val = [bf](uint16_t h) { return bf ? bits_to_float<true>(h) : bits_to_float<false>(h); };
        float s = 0.0f;
        for (int64_t k = 0; k < p.K; ++k)
            s = __builtin_fmaf(val(a[k]), val(bc[k * kstride]), s);
        if (p.bias != nullptr)
            s += val(p.bias[j]);
        const float r0 = (p.relu == 0 || s > 0.0f) ? s : 0.0f;
        p.C[b * p.sC + i * p.ldc + j] = bf ? __builtin_bit_cast(uint16_t, (__bf16)r0)
                                           : __builtin_bit_cast(uint16_t, (_Float16)r0);
    }
}

}  // namespace

hipError_t launch_naive(const GemmArgs &p, hipStream_t stream)
{
    const int64_t total = p.M * p.N * p.batch;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536)
        blocks = 65536;
    hipLaunchKernelGGL(gemm_relu_naive_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace tg
