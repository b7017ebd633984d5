// Measured ceilings of the part the GEMM kernels run on, as one JSON line per
// figure: what the matrix cores sustain on their own, and how fast LDS
// delivers the two fragment read forms the tile kernels use.  These are the
// practical bounds the kernels' roofline fractions are read against (the
// spec peak assumes the 2.4 GHz clock, which the matrix cores do not hold
// under load).
//
//   mfma_f16_32x32x16  Every wave runs a loop of independent
//                      v_mfma_f32_32x32x16_f16 on register operands drawn
//                      from normal(0, 1/sqrt(8192)) (the 8192^3 workload's
//                      distribution: the matrix cores' power, and so the
//                      clock, depends on the data), 8 waves per CU, no memory
//                      traffic in the loop.  Reports TFLOP/s and the shader
//                      clock it ran at (clock64 / wall clock inside the kernel).
//   mfma_f16_16x16x32  The same flops as v_mfma_f32_16x16x32_f16 products
//                      (twice as many instructions on 16 accumulators).
//   lds_read_b128      ds_read_b128 (A fragments and (N,K) B fragments):
//                      bytes per shader clock per CU, 8 waves per CU,
//                      conflict-free addresses.
//   lds_read_tr_b64    ds_read_b64_tr_b16 (transpose reads of a row-major
//                      (K,N) B tile) in the tile kernels' XOR-swizzled layout.
//   hbm_read           A plain streaming read: 16 bytes per lane, grid-stride
//                      over 256 MiB, three buffers taken in turn so that no
//                      pass is served from the 256 MB last-level cache.
//   hbm_copy_batched   The traffic of the strided batch of 1024 128x128x64
//                      products without the arithmetic: 1024 workgroups, each
//                      reading 16 KiB from each of two buffers and writing
//                      32 KiB, 16 bytes per lane, non-temporal loads and
//                      stores, ten buffer sets taken in turn (64 MiB a pass,
//                      none of it left in the last-level cache).
//   l2_load_per_cu     What one CU's loads fetch from data the L2 holds: one
//                      8-wave workgroup per CU, each wave streaming 4 KiB
//                      blocks of a 2 MiB buffer (16 bytes per lane), bytes per
//                      shader clock per CU and GB/s per CU.
//
// Usage: tg_ceilings [seconds_per_figure]   (default 0.2)
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int kOperands = 65536;   // f16x8 operand vectors drawn on the host
constexpr int kChains = 8;         // independent accumulators per wave (128 registers)

#define CHECK(x)                                                                         \
    do {                                                                                 \
        hipError_t e_ = (x);                                                             \
        if (e_ != hipSuccess) {                                                          \
            std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));         \
            std::exit(1);                                                                \
        }                                                                                \
    } while (0)

// clock64 and the 100 MHz wall clock at the first and last instruction of
// wave 0 of each workgroup, for the clock the loop ran at.
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int MI>
__global__ void __launch_bounds__(512) mfma_loop(const f16x8 *in, float *out, long long *clk,
                                                 int iters)
{
    const int t = blockIdx.x * 512 + threadIdx.x;
    f16x8 a[4], b[2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        a[i] = in[(t * 6 + i) % kOperands];
#pragma unroll
    for (int i = 0; i < 2; ++i)
        b[i] = in[(t * 6 + 4 + i) % kOperands];
    // the same registers and flops either way: 8 accumulators of 16 or 16 of 4
    constexpr int NA = MI == 32 ? kChains : 2 * kChains, NE = MI == 32 ? 16 : 4;
    typedef float accv __attribute__((ext_vector_type(NE)));
    accv acc[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i)
        acc[i] = accv{};
    const long long c0 = clock64(), w0 = wall_clock64();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            if constexpr (MI == 32)
                acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i & 3], b[i >> 2], acc[i], 0, 0, 0);
            else
                acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i & 3], b[(i >> 2) & 1], acc[i], 0, 0, 0);
        }
        // rotate the operands so consecutive products see different values
#pragma unroll
        for (int i = 0; i < 4; ++i)
            a[i] = __builtin_shufflevector(a[i], a[i], 1, 2, 3, 4, 5, 6, 7, 0);
    }
    const long long c1 = clock64(), w1 = wall_clock64();
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
        for (int j = 0; j < NE; ++j)
            s += acc[i][j];
    out[t] = s;
    if (threadIdx.x == 0) {
        clk[2 * blockIdx.x] = c1 - c0;
        clk[2 * blockIdx.x + 1] = w1 - w0;
    }
}

// LDS reads: KIND 0 ds_read_b128, KIND 1 ds_read_b64_tr_b16 in the tile
// kernels' B layout (512-byte rows, 16-byte chunk c of row k stored at chunk
// c ^ ((k & 3) << 2)).  Every address stays inside the 64 KiB array.
template <int KIND>
__global__ void __launch_bounds__(512) lds_loop(uint32_t *out, long long *clk, int iters)
{
    __shared__ __attribute__((aligned(1024))) uint16_t smem[32768];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < 32768; i += 512)
        smem[i] = (uint16_t)i;
    __syncthreads();
    const lds_u8 *base = (const lds_u8 *)smem;
    u32x4 acc = {0, 0, 0, 0};
    const long long c0 = clock64();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            if constexpr (KIND == 0) {
                const int off = ((wave * 8 + r) * 1024 + lane * 16 + it * 64) & 65535 & ~15;
                acc += *(const lds_u32x4 *)(base + off);
            } else {
                const int k = 8 * (lane >> 5) + ((lane & 15) >> 2) + 16 * ((wave * 8 + r + it) & 3);
                const int n = 16 * ((lane >> 4) & 1) + 4 * (lane & 3) + 32 * ((wave + it) & 7);
                const int off = (k * 512 + (((n >> 3) ^ ((k & 3) << 2)) * 16) + (n & 7) * 2) & 65535;
                const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(base + off));
                acc.x += (uint32_t)(uint16_t)v.x;
                acc.y += (uint32_t)(uint16_t)v.w;
            }
        }
    }
    const long long c1 = clock64();
    out[blockIdx.x * 512 + tid] = acc.x + acc.y + acc.z + acc.w;
    if (tid == 0)
        clk[blockIdx.x] = c1 - c0;
}

// Reads n16 16-byte vectors, each lane striding by the grid; one sum per
// workgroup keeps the loads alive.
__global__ void __launch_bounds__(512) hbm_read(const u32x4 *p, int64_t n16, uint32_t *out)
{
    u32x4 acc = {0, 0, 0, 0};
    const int64_t stride = (int64_t)gridDim.x * 512;
    for (int64_t i = (int64_t)blockIdx.x * 512 + threadIdx.x; i < n16; i += stride)
        acc ^= __builtin_nontemporal_load(p + i);
    const uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (v == 0x9e3779b9u)   // practically never: keeps the reads without a store per lane
        out[blockIdx.x] = v;
}

// Workgroup g reads a[g] and b[g] (16 KiB each) and writes c[g] (32 KiB).
__global__ void __launch_bounds__(256) copy_batched(const u32x4 *a, const u32x4 *b, u32x4 *c)
{
    const int t = threadIdx.x;
    const size_t g = blockIdx.x;
    const u32x4 *ag = a + g * 1024, *bg = b + g * 1024;
    u32x4 *cg = c + g * 2048;
    u32x4 ra[4], rb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ra[i] = __builtin_nontemporal_load(ag + i * 256 + t);
        rb[i] = __builtin_nontemporal_load(bg + i * 256 + t);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        __builtin_nontemporal_store(ra[i], cg + i * 256 + t);
        __builtin_nontemporal_store(rb[i], cg + (i + 4) * 256 + t);
    }
}

// Each wave streams 4 KiB blocks (four 16-byte loads per lane) of an
// L2-resident buffer of `blocks4k` blocks, starting at its own block and
// stepping 37 blocks at a time; clock64 around wave 0's loop.
__global__ void __launch_bounds__(512) l2_load(const u32x4 *p, int blocks4k, int iters, uint32_t *out,
                                               long long *clk)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int blk = (blockIdx.x * 8 + w) % blocks4k;
    __syncthreads();
    const long long c0 = clock64();
    u32x4 acc = {0, 0, 0, 0};
    for (int it = 0; it < iters; ++it) {
        const u32x4 *q = p + (size_t)blk * 256;
        u32x4 v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            v[j] = q[j * 64 + lane];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc ^= v[j];
        blk = (blk + 37) % blocks4k;
    }
    const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (x == 0x9e3779b9u)   // practically never: keeps the loads without a store per lane
        out[blockIdx.x] = x;
    __syncthreads();
    const long long c1 = clock64();
    if (threadIdx.x == 0)
        clk[blockIdx.x] = c1 - c0;
}

}  // namespace

int main(int argc, char **argv)
{
    const double target_s = argc > 1 ? std::atof(argv[1]) : 0.2;
    int dev = 0, cus = 0, wall_khz = 0;
    CHECK(hipGetDevice(&dev));
    CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    CHECK(hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, dev));

    std::vector<_Float16> h((size_t)kOperands * 8);
    std::mt19937 gen(2);
    std::normal_distribution<double> nd(0.0, 1.0 / std::sqrt(8192.0));
    for (auto &x : h)
        x = (_Float16)nd(gen);
    f16x8 *d_in;
    float *d_out;
    long long *d_clk;
    const int blocks = cus;   // one 8-wave workgroup per CU
    CHECK(hipMalloc(&d_in, h.size() * sizeof(_Float16)));
    CHECK(hipMemcpy(d_in, h.data(), h.size() * sizeof(_Float16), hipMemcpyHostToDevice));
    CHECK(hipMalloc(&d_out, (size_t)blocks * 512 * sizeof(float)));
    CHECK(hipMalloc(&d_clk, (size_t)blocks * 2 * sizeof(long long)));
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    std::vector<long long> clk((size_t)blocks * 2);

    // matrix cores: size the loop for about target_s seconds from a short run
    for (int mi : {32, 16}) {
        int iters = 2000;
        for (int pass = 0; pass < 2; ++pass) {
            CHECK(hipEventRecord(e0, 0));
            if (mi == 32)
                hipLaunchKernelGGL(mfma_loop<32>, dim3(blocks), dim3(512), 0, 0, d_in, d_out, d_clk, iters);
            else
                hipLaunchKernelGGL(mfma_loop<16>, dim3(blocks), dim3(512), 0, 0, d_in, d_out, d_clk, iters);
            CHECK(hipGetLastError());
            CHECK(hipEventRecord(e1, 0));
            CHECK(hipEventSynchronize(e1));
            float ms = 0;
            CHECK(hipEventElapsedTime(&ms, e0, e1));
            if (pass == 0) {
                iters = (int)std::fmin(2.0e8, std::fmax(2000.0, iters * target_s * 1e3 / ms));
                continue;
            }
            CHECK(hipMemcpy(clk.data(), d_clk, clk.size() * sizeof(long long), hipMemcpyDeviceToHost));
            double c = 0, w = 0;
            for (int i = 0; i < blocks; ++i) {
                c += (double)clk[2 * i];
                w += (double)clk[2 * i + 1];
            }
            const double mhz = c / (w / (wall_khz * 1e3)) / 1e6;
            const double flop = (double)blocks * 8 /* waves */ * iters * kChains * 2.0 * 32 * 32 * 16;
            std::printf("{\"figure\": \"%s\", \"tflops\": %.1f, \"sclk_mhz\": %.0f, "
                        "\"ms\": %.3f, \"waves_per_cu\": 8, \"operands\": \"normal(0, 1/sqrt(8192))\"}\n",
                        mi == 32 ? "mfma_f16_32x32x16" : "mfma_f16_16x16x32",
                        flop / (ms * 1e-3) / 1e12, mhz, ms);
        }
    }
    // LDS read forms
    for (int kind = 0; kind < 2; ++kind) {
        const int iters = 20000;
        for (int pass = 0; pass < 2; ++pass) {
            if (kind == 0)
                hipLaunchKernelGGL(lds_loop<0>, dim3(blocks), dim3(512), 0, 0, (uint32_t *)d_out, d_clk, iters);
            else
                hipLaunchKernelGGL(lds_loop<1>, dim3(blocks), dim3(512), 0, 0, (uint32_t *)d_out, d_clk, iters);
            CHECK(hipGetLastError());
            CHECK(hipDeviceSynchronize());
        }
        CHECK(hipMemcpy(clk.data(), d_clk, (size_t)blocks * sizeof(long long), hipMemcpyDeviceToHost));
        double cyc = 0;
        for (int i = 0; i < blocks; ++i)
            cyc += (double)clk[i];
        cyc /= blocks;
        const double bytes = 8.0 * 64 * iters * 8 * (kind == 0 ? 16 : 8);   // per CU
        std::printf("{\"figure\": \"%s\", \"bytes_per_clock_per_cu\": %.1f, \"waves_per_cu\": 8}\n",
                    kind == 0 ? "lds_read_b128" : "lds_read_tr_b64", bytes / cyc);
    }
    // HBM streaming read
    {
        const int64_t bytes = 256ll << 20, n16 = bytes / 16;
        u32x4 *buf[3];
        for (auto &b : buf) {
            CHECK(hipMalloc(&b, bytes));
            CHECK(hipMemset(b, 1, bytes));
        }
        const int grid = cus * 4;
        for (int i = 0; i < 6; ++i)
            hipLaunchKernelGGL(hbm_read, dim3(grid), dim3(512), 0, 0, buf[i % 3], n16, (uint32_t *)d_out);
        CHECK(hipGetLastError());
        CHECK(hipDeviceSynchronize());
        const int reps = 30;
        CHECK(hipEventRecord(e0, 0));
        for (int i = 0; i < reps; ++i)
            hipLaunchKernelGGL(hbm_read, dim3(grid), dim3(512), 0, 0, buf[i % 3], n16, (uint32_t *)d_out);
        CHECK(hipGetLastError());
        CHECK(hipEventRecord(e1, 0));
        CHECK(hipEventSynchronize(e1));
        float ms = 0;
        CHECK(hipEventElapsedTime(&ms, e0, e1));
        std::printf("{\"figure\": \"hbm_read\", \"gbs\": %.0f, \"us_per_256MiB\": %.1f}\n",
                    (double)bytes * reps / (ms * 1e-3) / 1e9, ms * 1e3 / reps);
        for (auto &b : buf)
            CHECK(hipFree(b));
    }
    // the batched product's traffic, no arithmetic
    {
        constexpr int kSets = 10, kGroups = 1024;
        const size_t ab = (size_t)kGroups * 16384, cb = (size_t)kGroups * 32768;
        u32x4 *a[kSets], *b[kSets], *c[kSets];
        for (int i = 0; i < kSets; ++i) {
            CHECK(hipMalloc(&a[i], ab));
            CHECK(hipMalloc(&b[i], ab));
            CHECK(hipMalloc(&c[i], cb));
            CHECK(hipMemset(a[i], 1, ab));
            CHECK(hipMemset(b[i], 2, ab));
        }
        for (int i = 0; i < 2 * kSets; ++i)
            hipLaunchKernelGGL(copy_batched, dim3(kGroups), dim3(256), 0, 0, a[i % kSets], b[i % kSets],
                               c[i % kSets]);
        CHECK(hipGetLastError());
        CHECK(hipDeviceSynchronize());
        const int reps = 400;
        CHECK(hipEventRecord(e0, 0));
        for (int i = 0; i < reps; ++i)
            hipLaunchKernelGGL(copy_batched, dim3(kGroups), dim3(256), 0, 0, a[i % kSets], b[i % kSets],
                               c[i % kSets]);
        CHECK(hipGetLastError());
        CHECK(hipEventRecord(e1, 0));
        CHECK(hipEventSynchronize(e1));
        float ms = 0;
        CHECK(hipEventElapsedTime(&ms, e0, e1));
        const double us = ms * 1e3 / reps;
        std::printf("{\"figure\": \"hbm_copy_batched\", \"us_per_pass\": %.2f, \"gbs\": %.0f, "
                    "\"bytes_per_pass\": %zu}\n", us, (double)(2 * ab + cb) / (us * 1e-6) / 1e9, 2 * ab + cb);
        for (int i = 0; i < kSets; ++i) {
            CHECK(hipFree(a[i]));
            CHECK(hipFree(b[i]));
            CHECK(hipFree(c[i]));
        }
    }
    // one CU's loads from L2-resident data
    {
        const int blocks4k = 512;   // 2 MiB
        u32x4 *buf;
        CHECK(hipMalloc(&buf, (size_t)blocks4k * 4096));
        CHECK(hipMemset(buf, 3, (size_t)blocks4k * 4096));
        const int iters = 4096;
        for (int pass = 0; pass < 2; ++pass) {
            CHECK(hipEventRecord(e0, 0));
            hipLaunchKernelGGL(l2_load, dim3(blocks), dim3(512), 0, 0, buf, blocks4k, iters,
                               (uint32_t *)d_out, d_clk);
            CHECK(hipGetLastError());
            CHECK(hipEventRecord(e1, 0));
            CHECK(hipEventSynchronize(e1));
        }
        float ms = 0;
        CHECK(hipEventElapsedTime(&ms, e0, e1));
        CHECK(hipMemcpy(clk.data(), d_clk, (size_t)blocks * sizeof(long long), hipMemcpyDeviceToHost));
        double cyc = 0;
        for (int i = 0; i < blocks; ++i)
            cyc += (double)clk[i];
        cyc /= blocks;
        const double per_cu = 8.0 * iters * 4096;   // bytes one workgroup loads
        std::printf("{\"figure\": \"l2_load_per_cu\", \"bytes_per_clock_per_cu\": %.1f, "
                    "\"gbs_per_cu\": %.1f, \"waves_per_cu\": 8}\n",
                    per_cu / cyc, per_cu / (ms * 1e-3) / 1e9);
        CHECK(hipFree(buf));
    }
    CHECK(hipFree(d_in));
    CHECK(hipFree(d_out));
    CHECK(hipFree(d_clk));
    return 0;
}
