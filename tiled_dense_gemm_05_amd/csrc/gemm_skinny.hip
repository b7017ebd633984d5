// Skinny-M fp16 GEMM + ReLU (M <= 64) on gfx950: a memory-bound stream of B.
//
// Same operation as the GEMM+ReLU tile program of the "TileLang paper
// reading" page (hotelren.com), section 2, for the shape where A has a
// handful of rows (decode-like): each element of B is used by at most 64
// output rows, so the time is the time to stream B from HBM once.  The
// "tilelang practitioner's notes" page (dpshk.com), section 1.1, names such
// long, thin GEMMs as a case vendor libraries handle poorly; section 3.2 of
// that page fixes K as a serial accumulation, so a K split must be summed
// before the ReLU (done here in registers and LDS, in a fixed order).
//
// Design:
//  * One workgroup per NB-column slice of C (grid = ceil(N / NB)), NW waves.
//    The K steps are dealt to the waves in turn (wave w takes steps w,
//    w + NW, ...); each wave streams its steps of the B slice through a
//    private S-stage LDS ring with buffer_load_dwordx4 ... lds (one 1 KiB
//    block per instruction) and never waits for the other waves until the
//    end.  Dealing the steps (rather than giving each wave a quarter of K)
//    keeps every wave of every workgroup on neighbouring rows of B, a narrow
//    window of memory that HBM serves faster (at 16 x 16384 x 8192: 5.5
//    against 5.1 TB/s).  The A rows of the same K step ride along in the
//    same stage (A is small and stays in L2).
//  * Per 32-wide k step: v_mfma_f32_16x16x32_f16 with the operand roles
//    swapped as in the tile kernels (C^T = B^T A^T): B^T fragments come from
//    transpose reads (ds_read_b64_tr_b16) of the row-major B block, A^T
//    fragments from one 16-byte LDS read per lane; a lane ends up owning 4
//    consecutive columns of one C row.
//  * Out-of-range chunks (k >= K, columns >= N, rows >= M) get a buffer
//    offset at the descriptor's record count and read as zeros.
//  * At the end each wave's fp32 partial sums go to LDS; after one barrier
//    every output fragment is summed over the waves in wave order (the result
//    is deterministic), clamped at zero, rounded to fp16 (nearest even) and
//    stored.
//  * MODE bit 0: bf16 elements (v_mfma_f32_16x16x32_bf16, bf16 store); bit 1:
//    B stored (N,K): the slice is NB rows of B^T, staged like the A rows
//    (64-byte rows of 32 k) and read with one 16-byte read per fragment.
// Requirements (checked by the dispatcher): 16-byte aligned A, B, C; lda,
// ldb, ldc, N, K multiples of 8; M <= 16 * MB.
#include "tg_lds_dma.h"
#include "tg_splitk.h"

namespace tg {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) f16x8 lds_f16x8;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

using dma::dma16;
using dma::dma16_nt;
using dma::kOutOfRange;
using dma::make_rsrc;
using dma::wait_lgkm0;
using dma::wait_vmcnt;

template <int MB_, int NB_, int NW_, int S_, bool NTB_ = false, int MODE_ = 0>
struct Skinny {
    static constexpr bool NTB = NTB_;            // stream B with non-temporal loads
    static constexpr bool BF16 = (MODE_ & 1) != 0;
    static constexpr bool BT = (MODE_ & 2) != 0;  // B stored (N,K)
    // fp32 partial sums of one K chunk per grid.y entry (split-K): see
    // launch_skinny_partial
    static constexpr bool PARTIAL = (MODE_ & 4) != 0;
    static constexpr int MB = MB_;               // 16-row blocks of A / C
    static constexpr int NB = NB_;               // columns of C per workgroup
    static constexpr int NW = NW_;               // waves (K split)
    static constexpr int S = S_;                 // LDS stages per wave
    static constexpr int NT = 64 * NW;
    static constexpr int NF = NB / 16;           // 16-column fragments
    // k per step: 32 for a (K,N) B (32 rows of NB columns); 64 for an (N,K)
    // B, so that each B^T row contributes a whole 128-byte line per step
    static constexpr int KS = BT ? 64 : 32;
    static constexpr int CR = KS / 8;            // 16-byte chunks per A (and B^T) row
    static constexpr int RPB = 64 / CR;          // A (and B^T) rows per 1 KiB block
    static constexpr int A_BYTES = MB * 16 * KS * 2;      // A rows of one step
    static constexpr int B_BYTES = KS * NB * 2;           // B block of one step
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int A_LD = A_BYTES / 1024, B_LD = B_BYTES / 1024;
    static constexpr int LOADS = A_LD + B_LD;
    static constexpr int CB = NB / 8;            // 16-byte chunks per B row
    static constexpr int B_RPB = BT ? 16 : 64 / CB;   // B rows per 1 KiB block
    static constexpr int RING = NW * S * STAGE;
    static constexpr int RED = NW * MB * NF * 64 * 16;    // partial sums
    static constexpr int LDS = RING > RED ? RING : RED;
    static_assert(NB == 32 || NB == 64 || NB == 128, "slice width");
    static_assert(LOADS * (S - 1) <= 63, "vmcnt range");
    static_assert(LDS <= 160 * 1024, "LDS size");
};

// A block (MB*16 rows x KS k): a 16-byte read of 16 rows at the same chunk
// is spread over the bank line by XOR-ing the chunk with the row's position
// in it (64-byte rows: row / 4; 128-byte rows: row / 2).
template <int CR>
__device__ __forceinline__ int swz_a(int row, int c)
{
    if constexpr (CR == 4)
        return c ^ ((row >> 2) & 3);
    else
        return c ^ ((row >> 1) & 7);
}

// B block (32 rows x NB columns): a transpose read touches rows
// {4h..4h+3} and {8+4h..8+4h+3} (32 bytes each) per half-wave; XOR the
// 32-byte window of the row so those eight rows hit distinct windows.
template <int CB>
__device__ __forceinline__ int swz_b(int k, int c)
{
    if constexpr (CB == 16)
        return c ^ (((k & 3) | (((k >> 3) & 1) << 2)) << 1);
    else if constexpr (CB == 8)
        return c ^ ((((k >> 1) & 1) | (((k >> 3) & 1) << 1)) << 1);
    else
        return c ^ (((k >> 3) & 1) << 1);
}

template <class T>
__global__ void __launch_bounds__(T::NT) gemm_relu_skinny_kernel(GemmArgs p, int steps_per_wave)
{
    __shared__ __attribute__((aligned(1024))) uint8_t smem[T::LDS];
    const lds_u16 *lds = (const lds_u16 *)smem;
    const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t bidx = blockIdx.y;
    // split-K: grid.y entry bidx covers k in [bidx * sA, bidx * sA + sA) of K
    int64_t K = p.K;
    if constexpr (T::PARTIAL) {
        const int64_t left = p.K - bidx * p.sA;
        K = left < 0 ? 0 : (left < p.sA ? left : p.sA);
    }
    const int64_t M = p.M, N = p.N;
    const int64_t n0 = (int64_t)blockIdx.x * T::NB;
    const uint16_t *Ab = p.A + bidx * p.sA;
    const uint16_t *Bb = p.B + bidx * p.sB + (T::BT ? n0 * p.ldb : n0);
    uint16_t *C = p.C + bidx * p.sC;
    const uint32_t ring = lds_base + (uint32_t)(wave * T::S * T::STAGE);

    // Load plan.  A block j (16 rows of 64 bytes): lane L -> row 16 j + L / 4,
    // physical chunk L % 4.  B block j: lane L -> row j * B_RPB + L / CB,
    // physical chunk L % CB.  The logical chunk is the swizzled one.
    uint32_t a_voff[T::A_LD];
    int a_col[T::A_LD];
#pragma unroll
    for (int j = 0; j < T::A_LD; ++j) {
        const int row = T::RPB * j + lane / T::CR;
        const int c = swz_a<T::CR>(row, lane % T::CR);
        a_col[j] = c * 8;
        a_voff[j] = row < M ? (uint32_t)((row * p.lda + c * 8) * 2) : kOutOfRange;
    }
    // (N,K) B: block j is rows 16 j .. 16 j + 15 of the B^T slice, laid out
    // like an A block; b_row then holds the chunk's k column.
    uint32_t b_voff[T::B_LD];
    int b_row[T::B_LD];
#pragma unroll
    for (int j = 0; j < T::B_LD; ++j) {
        if constexpr (T::BT) {
            const int row = T::RPB * j + lane / T::CR;
            const int c = swz_a<T::CR>(row, lane % T::CR);
            b_row[j] = c * 8;
            b_voff[j] = (n0 + row < N) ? (uint32_t)((row * p.ldb + c * 8) * 2) : kOutOfRange;
        } else {
            const int row = j * T::B_RPB + lane / T::CB;
            const int c = swz_b<T::CB>(row, lane % T::CB);
            b_row[j] = row;
            b_voff[j] = (n0 + c * 8 < N) ? (uint32_t)((row * p.ldb + c * 8) * 2) : kOutOfRange;
        }
    }

    auto issue = [&](int st) {
        const int64_t k0 = ((int64_t)st * T::NW + wave) * T::KS;   // the wave's st-th step
        const int64_t kleft = K - k0;                     // valid k from here
        const i32x4 ra = make_rsrc(Ab + k0);
        const i32x4 rb = make_rsrc(Bb + (T::BT ? k0 : k0 * p.ldb));
        const uint32_t base = ring + (uint32_t)((st % T::S) * T::STAGE);
#pragma unroll
        for (int j = 0; j < T::A_LD; ++j)
            dma16(ra, a_col[j] < kleft ? a_voff[j] : kOutOfRange, base + j * 1024);
#pragma unroll
        for (int j = 0; j < T::B_LD; ++j) {
            const uint32_t v = b_row[j] < kleft ? b_voff[j] : kOutOfRange;
            if constexpr (T::NTB)
                dma16_nt(rb, v, base + T::A_BYTES + j * 1024);
            else
                dma16(rb, v, base + T::A_BYTES + j * 1024);
        }
    };

    f32x4 acc[T::MB][T::NF];
#pragma unroll
    for (int mb = 0; mb < T::MB; ++mb)
#pragma unroll
        for (int f = 0; f < T::NF; ++f)
            acc[mb][f] = f32x4{};

    // Every wave runs the same number of steps; steps past the end of K load
    // zeros (no memory access) so the wait counts stay constant.
#pragma unroll
    for (int s = 0; s < T::S - 1; ++s)
        issue(s);
    for (int st = 0; st < steps_per_wave; ++st) {
        // Refill the stage read one step ago (its reads completed before that
        // step's MFMAs; the wait makes the order explicit), then wait until
        // step st has landed: the S-1 later steps may still be in flight.
        wait_lgkm0();
        issue(st + T::S - 1);
        wait_vmcnt<(T::S - 1) * T::LOADS>();
        const lds_u16 *As = lds + (wave * T::S + st % T::S) * (T::STAGE / 2);
        const lds_u16 *Bs = As + T::A_BYTES / 2;
#pragma unroll
        for (int ks = 0; ks < T::KS / 32; ++ks) {
            f16x8 af[T::MB], bf[T::NF];
#pragma unroll
            for (int mb = 0; mb < T::MB; ++mb) {
                const int row = mb * 16 + (lane & 15);
                const int c = ks * 4 + (lane >> 4);
                af[mb] = *reinterpret_cast<const lds_f16x8 *>(As + row * T::KS +
                                                              swz_a<T::CR>(row, c) * 8);
            }
#pragma unroll
            for (int f = 0; f < T::NF; ++f) {
                if constexpr (T::BT) {
                    const int row = f * 16 + (lane & 15);
                    const int c = ks * 4 + (lane >> 4);
                    bf[f] = *reinterpret_cast<const lds_f16x8 *>(Bs + row * T::KS +
                                                                 swz_a<T::CR>(row, c) * 8);
                    continue;
                }
                s16x4 h[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int k = 8 * (lane >> 4) + 4 * hh + ((lane & 15) >> 2);
                    const int n = f * 16 + 4 * (lane & 3);
                    const lds_u16 *src = Bs + k * T::NB + swz_b<T::CB>(k, n >> 3) * 8 + (n & 7);
                    h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)src);
                }
                bf[f] = __builtin_bit_cast(
                    f16x8, __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7));
            }
#pragma unroll
            for (int mb = 0; mb < T::MB; ++mb)
#pragma unroll
                for (int f = 0; f < T::NF; ++f)
                    if constexpr (T::BF16)
                        acc[mb][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, bf[f]), __builtin_bit_cast(bf16x8, af[mb]),
                            acc[mb][f], 0, 0, 0);
                    else
                        acc[mb][f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bf[f], af[mb],
                                                                            acc[mb][f], 0, 0, 0);
        }
    }
    wait_vmcnt<0>();
    __syncthreads();   // every wave is done with its ring before it is reused

    // Partial sums: [wave][mb][f][lane] of 4 floats.
    lds_f32x4 *part = (lds_f32x4 *)smem;
#pragma unroll
    for (int mb = 0; mb < T::MB; ++mb)
#pragma unroll
        for (int f = 0; f < T::NF; ++f)
            part[((wave * T::MB + mb) * T::NF + f) * 64 + lane] = acc[mb][f];
    __syncthreads();

    // Fragment q = (mb, f) is finished by wave q % NW: sum over the waves in
    // order, bias, ReLU, fp16, store.  Lane owns C[m][n .. n+3].
    const bool relu = p.relu != 0;
    for (int q = wave; q < T::MB * T::NF; q += T::NW) {
        f32x4 s = part[q * 64 + lane];
        for (int w = 1; w < T::NW; ++w)
            s += part[(w * T::MB * T::NF + q) * 64 + lane];
        const int mb = q / T::NF, f = q % T::NF;
        const int64_t m = mb * 16 + (lane & 15);
        const int64_t n = n0 + f * 16 + 4 * (lane >> 4);
        if constexpr (T::PARTIAL) {
            // the chunk's fp32 sums, (M, N) row-major at C + bidx * sC floats
            if (m < M && n < N)
                *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(p.C) + bidx * p.sC +
                                           m * N + n) = s;
            continue;
        }
        if (m < M && n < N) {
            float bv[4];
            load_bias4<T::BF16>(p.bias, n, N, bv);
            u32x2 w2;
            w2.x = epi_pack2<T::BF16>(s[0] + bv[0], s[1] + bv[1], relu);
            w2.y = epi_pack2<T::BF16>(s[2] + bv[2], s[3] + bv[3], relu);
            *reinterpret_cast<u32x2 *>(C + m * p.ldc + n) = w2;
        }
    }
}

template <class T>
hipError_t launch(const GemmArgs &p, hipStream_t stream)
{
    const int64_t slices = (p.N + T::NB - 1) / T::NB;
    const int64_t ksteps = (p.K + T::KS - 1) / T::KS;
    const int64_t per_wave = (ksteps + T::NW - 1) / T::NW;
    if (slices > 0x7fffffff || per_wave > 0x7fffffff)
        return hipErrorInvalidValue;
    GemmArgs q = p;
    for (int64_t b0 = 0; b0 < p.batch; b0 += 65535) {
        const int64_t nb = (p.batch - b0) < 65535 ? (p.batch - b0) : 65535;
        q.A = p.A + b0 * p.sA;
        q.B = p.B + b0 * p.sB;
        q.C = p.C + b0 * p.sC;
        q.batch = nb;
        hipLaunchKernelGGL((gemm_relu_skinny_kernel<T>), dim3((unsigned)slices, (unsigned)nb),
                           dim3(T::NT), 0, stream, q, (int)per_wave);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

// Split-K reduction: C[m][n] = fp16_rne(ReLU(sum_s part[s][m][n])), the
// chunks added in order; thread owns 4 consecutive columns of one row.
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float *part, uint16_t *C,
                                                             int64_t M, int64_t N, int64_t ldc,
                                                             int64_t splits)
{
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t per_row = N / 4;
    if (q >= M * per_row)
        return;
    const int64_t m = q / per_row, n = (q % per_row) * 4;
    f32x4 s = *reinterpret_cast<const f32x4 *>(part + m * N + n);
    for (int64_t c = 1; c < splits; ++c)
        s += *reinterpret_cast<const f32x4 *>(part + c * M * N + m * N + n);
    u32x2 w;
    w.x = epi_pack2<false>(s[0], s[1], true);
    w.y = epi_pack2<false>(s[2], s[3], true);
    *reinterpret_cast<u32x2 *>(C + m * ldc + n) = w;
}

}  // namespace

hipError_t launch_skinny_splitk(const GemmArgs &p, int64_t splits, float *part,
                                hipStream_t stream)
{
    // chunks of whole 32-k steps; each grid.y entry writes its (M, N) fp32 sums
    const int64_t steps = (p.K + 31) / 32;
    const int64_t kc = (steps + splits - 1) / splits * 32;
    GemmArgs q = p;
    q.C = reinterpret_cast<uint16_t *>(part);
    q.sA = kc;
    q.sB = kc * p.ldb;
    q.sC = p.M * p.N;
    q.batch = splits;
    q.bias = nullptr;
    q.relu = 0;
    q.bf16 = 0;
    q.b_nk = 0;
    q.K = p.K;
    using T = Skinny<1, 64, 8, 3, true, 4>;
    using T4 = Skinny<4, 64, 8, 2, true, 4>;
    const int64_t slices = (p.N + 63) / 64;
    const int64_t per_wave = (kc / 32 + 7) / 8;
    if (p.M <= 16)
        hipLaunchKernelGGL((gemm_relu_skinny_kernel<T>), dim3((unsigned)slices, (unsigned)splits),
                           dim3(T::NT), 0, stream, q, (int)per_wave);
    else
        hipLaunchKernelGGL((gemm_relu_skinny_kernel<T4>), dim3((unsigned)slices, (unsigned)splits),
                           dim3(T4::NT), 0, stream, q, (int)per_wave);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int64_t threads = p.M * (p.N / 4);
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       stream, part, p.C, p.M, p.N, p.ldc, splits);
    return hipGetLastError();
}

bool skinny_layout_ok(const GemmArgs &p)
{
    // M <= 64; 32-bit buffer offsets: 64 A rows and 32 (K,N) B rows, or 64
    // (N,K) B rows, per step (an (N,K) slice spans 64 rows of ldb)
    return p.M <= 64 && p.lda <= (1 << 24) && p.ldb <= (p.b_nk ? (1 << 22) : (1 << 24));
}

namespace {

// bf16 and (N,K)-B instances of configurations 0, 4 and 7 (the default).
// An (N,K) B stages 64 k per step, twice the bytes per stage, so its rings
// are shallower to fit the LDS (and configuration 7 keeps eight waves only
// for one 16-row block of A).
template <int MODE>
hipError_t launch_mode(int cfg, const GemmArgs &p, hipStream_t stream)
{
    constexpr bool bt = (MODE & 2) != 0;
    constexpr int s1 = bt ? 3 : 6, s2 = bt ? 3 : 5, s4 = bt ? 2 : 4;
    const int mb = (int)((p.M + 15) / 16);
    switch (cfg) {
    case 0:
        if (mb <= 1) return launch<Skinny<1, 64, 4, s1, false, MODE>>(p, stream);
        if (mb <= 2) return launch<Skinny<2, 64, 4, s2, false, MODE>>(p, stream);
        return launch<Skinny<4, 64, 4, s4, false, MODE>>(p, stream);
    case 4:
        if (mb <= 1) return launch<Skinny<1, 64, 4, s1, true, MODE>>(p, stream);
        if (mb <= 2) return launch<Skinny<2, 64, 4, s2, true, MODE>>(p, stream);
        return launch<Skinny<4, 64, 4, s4, true, MODE>>(p, stream);
    case 7:
        if constexpr (bt) {
            if (mb <= 1) return launch<Skinny<1, 64, 8, 2, true, MODE>>(p, stream);
            if (mb <= 2) return launch<Skinny<2, 64, 4, s2, true, MODE>>(p, stream);
            return launch<Skinny<4, 64, 4, s4, true, MODE>>(p, stream);
        } else {
            if (mb <= 1) return launch<Skinny<1, 64, 8, 3, true, MODE>>(p, stream);
            if (mb <= 2) return launch<Skinny<2, 64, 8, 3, true, MODE>>(p, stream);
            return launch<Skinny<4, 64, 8, 2, true, MODE>>(p, stream);
        }
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool skinny_config_has_mode(int cfg, int mode)
{
    return mode == 0 ? (cfg >= 0 && cfg < kSkinnyConfigs) : (cfg == 0 || cfg == 4 || cfg == 7);
}

hipError_t launch_skinny_config(int cfg, const GemmArgs &p, hipStream_t stream)
{
    switch ((p.bf16 ? 1 : 0) | (p.b_nk ? 2 : 0)) {
    case 1: return launch_mode<1>(cfg, p, stream);
    case 2: return launch_mode<2>(cfg, p, stream);
    case 3: return launch_mode<3>(cfg, p, stream);
    default: break;
    }
    const int mb = (int)((p.M + 15) / 16);
    switch (cfg) {
    case 0:   // 64-column slices, 4 waves, 6 stages
        if (mb <= 1) return launch<Skinny<1, 64, 4, 6>>(p, stream);
        if (mb <= 2) return launch<Skinny<2, 64, 4, 5>>(p, stream);
        return launch<Skinny<4, 64, 4, 4>>(p, stream);
    case 1:   // 32-column slices, 4 waves, 8 stages
        if (mb <= 1) return launch<Skinny<1, 32, 4, 8>>(p, stream);
        if (mb <= 2) return launch<Skinny<2, 32, 4, 6>>(p, stream);
        return launch<Skinny<4, 32, 4, 5>>(p, stream);
    case 2:   // 64-column slices, 8 waves, 3 stages
        if (mb <= 1) return launch<Skinny<1, 64, 8, 3>>(p, stream);
        if (mb <= 2) return launch<Skinny<2, 64, 8, 3>>(p, stream);
        return launch<Skinny<4, 64, 8, 2>>(p, stream);
    case 3:   // 32-column slices, 8 waves, 4 stages
        if (mb <= 1) return launch<Skinny<1, 32, 8, 4>>(p, stream);
        if (mb <= 2) return launch<Skinny<2, 32, 8, 4>>(p, stream);
        return launch<Skinny<4, 32, 8, 3>>(p, stream);
    case 4:   // 64-column slices, 4 waves, 6 stages, non-temporal B
        if (mb <= 1) return launch<Skinny<1, 64, 4, 6, true>>(p, stream);
        if (mb <= 2) return launch<Skinny<2, 64, 4, 5, true>>(p, stream);
        return launch<Skinny<4, 64, 4, 4, true>>(p, stream);
    case 5:   // 128-column slices, 8 waves, 2 stages
        if (mb <= 1) return launch<Skinny<1, 128, 8, 2>>(p, stream);
        if (mb <= 2) return launch<Skinny<2, 128, 8, 2>>(p, stream);
        return launch<Skinny<4, 128, 4, 2>>(p, stream);
    case 6:   // 128-column slices, 4 waves, 4 stages, non-temporal B
        if (mb <= 1) return launch<Skinny<1, 128, 4, 4, true>>(p, stream);
        if (mb <= 2) return launch<Skinny<2, 128, 4, 3, true>>(p, stream);
        return launch<Skinny<4, 128, 4, 2, true>>(p, stream);
    case 7:   // 64-column slices, 8 waves, 3 stages, non-temporal B
        if (mb <= 1) return launch<Skinny<1, 64, 8, 3, true>>(p, stream);
        if (mb <= 2) return launch<Skinny<2, 64, 8, 3, true>>(p, stream);
        return launch<Skinny<4, 64, 8, 2, true>>(p, stream);
    case 8:   // 64-column slices, 4 waves, 8 stages, non-temporal B
        if (mb <= 1) return launch<Skinny<1, 64, 4, 8, true>>(p, stream);
        if (mb <= 2) return launch<Skinny<2, 64, 4, 6, true>>(p, stream);
        return launch<Skinny<4, 64, 4, 4, true>>(p, stream);
    case 9:   // 32-column slices, 8 waves, 4 stages, non-temporal B
        if (mb <= 1) return launch<Skinny<1, 32, 8, 4, true>>(p, stream);
        if (mb <= 2) return launch<Skinny<2, 32, 8, 4, true>>(p, stream);
        return launch<Skinny<4, 32, 8, 3, true>>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace tg
