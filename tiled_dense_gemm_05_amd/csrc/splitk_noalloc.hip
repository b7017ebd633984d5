// Allocation-free form of the split-K skinny GEMM+ReLU: the same kernels as
// tg_gemm_relu_f16_splitk, with the fp32 partial sums of the K chunks in a
// scratch array the library owns on each device instead of a workspace from
// the caller.  Declaration and contract in include/tg.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <mutex>

#include "tg.h"
#include "tg_splitk.h"

namespace {

constexpr int64_t kScratchBytes = TG_SPLITK_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

// The scratch array, one copy per device that runs this entry point.  In host
// code `scratch` names a host-side stand-in, not device memory: kernels and
// copies only ever receive the device address looked up below.
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::atomic<float *> g_scratch_ptr[kMaxDevices];
std::mutex g_init_mutex;

// The device address of this device's copy of `scratch`, looked up once per
// device with that device current (the caller's current device); nullptr if
// the lookup fails.
float *scratch_on_current_device(int &status)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        status = TG_ERR_NO_DEVICE;
        return nullptr;
    }
    if (dev >= kMaxDevices) {
        status = TG_ERR_UNSUPPORTED_DEVICE;
        return nullptr;
    }
    float *ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (ptr != nullptr)
        return ptr;
    std::lock_guard<std::mutex> lock(g_init_mutex);
    ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (ptr == nullptr) {
        void *addr = nullptr;
        if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr) {
            (void)hipGetLastError();
            status = TG_ERR_HIP;
            return nullptr;
        }
        ptr = static_cast<float *>(addr);
        g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
    return ptr;
}

}  // namespace

extern "C" {

int tg_gemm_relu_f16_splitk_noalloc(const void *A, const void *B, void *C, int64_t M, int64_t N,
                                    int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                                    int64_t splits, hipStream_t stream)
{
    tg::GemmArgs p{};
    int st = tg::splitk_check(A, B, C, M, N, K, lda, ldb, ldc, splits, p);
    if (st != TG_OK || M == 0 || N == 0)
        return st;
    // splits, M, N are bounded by splitk_check, so the product cannot overflow
    if (splits * M * N * (int64_t)sizeof(float) > kScratchBytes)
        return TG_ERR_INVALID_ARG;
    st = tg::host_check_device();
    if (st != TG_OK)
        return st;
    float *part = scratch_on_current_device(st);
    if (part == nullptr)
        return st;
    // every chunk writes all M x N of its partial sums before the reduction
    // reads them, so the previous call's contents need no clearing
    if (tg::launch_skinny_splitk(p, splits, part, stream) != hipSuccess)
        return TG_ERR_HIP;
    tg::host_set_last_path(TG_PATH_SKINNY);
    return TG_OK;
}

}  // extern "C"
