// Tiled fp16 GEMM + ReLU on gfx950 matrix cores.
//
// The structure follows the GEMM+ReLU tile program of the "TileLang paper
// reading" page (hotelren.com), section 2: one workgroup per BM x BN tile of
// C, operand tiles of A (BM x BK) and B (BK x BN) staged in shared memory
// (LDS), an fp32 accumulator fragment cleared to zero, a pipelined walk over
// K, a ReLU on the accumulator and a copy out to the fp16 C.  Section 3 of
// that page names the AMD pipeline primitives (counter waits and loads into
// LDS) and swizzled layouts for conflict-free shared memory; section 4 names
// L2-friendly block rasterization (a panel-ordered tile walk).  The
// "tilelang practitioner's notes" page (dpshk.com), section 3.4, gives
// 128 x 128 x 32 as the stable starting tile.
//
// What is specific to this gfx950 implementation:
//  * MFMA v_mfma_f32_32x32x16_f16 with the operand roles swapped: the matrix
//    core computes C^T = B^T A^T, so each lane ends up owning 4 consecutive
//    columns of one C row (8-byte stores) instead of single elements.
//  * B is row-major (N contiguous) but a matrix-core operand needs 8
//    consecutive k per lane; ds_read_b64_tr_b16 (gfx950 transpose read) turns
//    a 4-row x 16-column block of the LDS tile into 4 k-values per lane.
//  * LDS tiles are stored in 16-byte chunks permuted by an XOR of the row
//    (swizzle) so that the fragment reads of a wave spread over all banks.
//  * Workgroup ids are renumbered so that each of the 8 XCDs (each with its
//    own L2) receives a contiguous range of tiles, then walked in panels of
//    `groupM` tile rows.
//  * Two LDS stages with register prefetch: the next K-tile's global loads
//    are in flight while the matrix cores work on the current one; one
//    barrier per K-tile.
//  * MODE bit 0 selects bf16 elements (the bf16 matrix-core instruction and
//    a bf16 store), bit 1 a B stored as (N,K): its tile is BN rows of BK
//    contiguous k, loaded, stored and read exactly like the A tile.
#include "tg_internal.h"

namespace tg {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
// the same vectors at 4-byte alignment: gfx950 vector memory instructions
// need only dword alignment
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) f16x8 lds_f16x8;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

// Block tile BM x BN x BK computed by WM x WN waves; every wave owns a
// (BM/WM) x (BN/WN) sub-tile made of 32 x 32 MFMA fragments.
template <int BM_, int BN_, int BK_, int WM_, int WN_, int MODE_ = 0>
struct Tile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr bool BF16 = (MODE_ & 1) != 0;    // bf16 elements (fp16 otherwise)
    static constexpr bool BT = (MODE_ & 2) != 0;      // B stored (N,K)
    static constexpr int NT = 64 * WM * WN;           // threads per workgroup
    static constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
    static constexpr int FM = TM / 32, FN = TN / 32;  // MFMA fragments per wave
    static constexpr int CA = BK / 8;                 // 16-byte chunks per A-tile row
    static constexpr int CB = BN / 8;                 // 16-byte chunks per B-tile row
    static constexpr int A_ELEMS = BM * BK, B_ELEMS = BK * BN;
    static constexpr int STAGE = A_ELEMS + B_ELEMS;   // fp16 elements per LDS stage
    static constexpr int A_LD = BM * CA / NT;         // A chunks per thread per K-tile
    static constexpr int B_CHUNKS = BT ? BN * CA : BK * CB;
    static constexpr int B_LD = B_CHUNKS / NT;        // B chunks per thread per K-tile
    static_assert((BM * CA) % NT == 0 && B_CHUNKS % NT == 0, "tile not divisible by threads");
    static_assert(TM % 32 == 0 && TN % 32 == 0 && BK % 16 == 0, "fragment shape");
};

// Physical 16-byte chunk of logical chunk c in row `row` of the A tile.  A
// fragment read has 16 lanes reading the same chunk of 16 consecutive rows;
// the XOR spreads those rows over the sixteen 16-byte bank groups of a
// 256-byte bank line.
template <int CA>
__device__ __forceinline__ int swz_a(int row, int c)
{
    constexpr int rows_per_line = CA >= 16 ? 1 : 16 / CA;
    return c ^ ((row / rows_per_line) % CA);
}

// Physical chunk of logical chunk c in row k of the B tile.  A transpose read
// touches 4 consecutive rows x 64 bytes per half-wave; the XOR moves the four
// rows into four different 64-byte quarters of the bank line.
template <int CB>
__device__ __forceinline__ int swz_b(int k, int c)
{
    if constexpr (CB >= 16)
        return c ^ ((k & 3) << 2);
    else if constexpr (CB == 8)
        return c ^ (((k >> 1) & 1) << 2);
    else
        return c;
}

__device__ __forceinline__ u32x4 pack8(const uint16_t (&e)[8])
{
    u32x4 v;
    v.x = (uint32_t)e[0] | ((uint32_t)e[1] << 16);
    v.y = (uint32_t)e[2] | ((uint32_t)e[3] << 16);
    v.z = (uint32_t)e[4] | ((uint32_t)e[5] << 16);
    v.w = (uint32_t)e[6] | ((uint32_t)e[7] << 16);
    return v;
}

// Eight consecutive elements p[0..7] of a row whose valid length from p is
// `avail` (elements past it read as zero).  Whole chunks at a 4-byte aligned
// address are one dword-aligned vector load.  Chunks at 2 mod 4 read the
// dword-aligned window starting one element earlier plus one more dword and
// shift by 16 bits; `window_ok` says that p[-1] and p[8] lie inside the
// operand's extent.  Everything else is read element by element.
__device__ __forceinline__ u32x4 load8_masked(const uint16_t *p, int64_t avail, bool window_ok)
{
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    if (avail >= 8) {
        if ((a & 3) == 0)
            return *reinterpret_cast<const u32x4_a4 *>(p);
        if (window_ok) {
            const uint32_t *q = reinterpret_cast<const uint32_t *>(a - 2);
            const u32x4 w = *reinterpret_cast<const u32x4_a4 *>(q);
            const uint32_t w4 = q[4];
            u32x4 r;
            r.x = __builtin_amdgcn_alignbit(w.y, w.x, 16);
            r.y = __builtin_amdgcn_alignbit(w.z, w.y, 16);
            r.z = __builtin_amdgcn_alignbit(w.w, w.z, 16);
            r.w = __builtin_amdgcn_alignbit(w4, w.w, 16);
            return r;
        }
    }
    uint16_t e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        e[i] = (i < avail) ? p[i] : (uint16_t)0;
    return pack8(e);
}

// One K-tile of matrix-core work on LDS stage (As, Bs).
template <class T>
__device__ __forceinline__ void mma_stage(const lds_u16 *As, const lds_u16 *Bs,
                                          f32x16 (&acc)[T::FM][T::FN], int wm, int wn, int lane)
{
#pragma unroll
    for (int kk = 0; kk < T::BK / 16; ++kk) {
        f16x8 af[T::FM];
        f16x8 bf[T::FN];
        // A^T operand: lane holds A[row][8 consecutive k], one 16-byte read.
#pragma unroll
        for (int fm = 0; fm < T::FM; ++fm) {
            const int row = wm * T::TM + fm * 32 + (lane & 31);
            const int c = kk * 2 + (lane >> 5);
            af[fm] = *reinterpret_cast<const lds_f16x8 *>(As + row * T::BK + swz_a<T::CA>(row, c) * 8);
        }
        // B^T operand: lane needs B[8 consecutive k][one n].  An (N,K) B
        // tile holds them contiguously (one 16-byte read, as for A); a (K,N)
        // tile takes two transpose reads of 4 k each: source lane s of each
        // 16-lane group points at row (s / 4) and columns 4 * (s % 4) .. + 3
        // of a 4 x 16 block.
#pragma unroll
        for (int fn = 0; fn < T::FN; ++fn) {
            if constexpr (T::BT) {
                const int row = wn * T::TN + fn * 32 + (lane & 31);
                const int c = kk * 2 + (lane >> 5);
                bf[fn] = *reinterpret_cast<const lds_f16x8 *>(Bs + row * T::BK +
                                                              swz_a<T::CA>(row, c) * 8);
                continue;
            }
            s16x4 h[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int k = kk * 16 + 8 * (lane >> 5) + 4 * hh + ((lane & 15) >> 2);
                const int n = wn * T::TN + fn * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
                const lds_u16 *src = Bs + k * T::BN + swz_b<T::CB>(k, n >> 3) * 8 + (n & 7);
                h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)src);
            }
            bf[fn] = __builtin_bit_cast(f16x8, __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int fm = 0; fm < T::FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < T::FN; ++fn)
                if constexpr (T::BF16)
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, bf[fn]), __builtin_bit_cast(bf16x8, af[fm]),
                        acc[fm][fn], 0, 0, 0);
                else
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[fn], af[fm],
                                                                         acc[fm][fn], 0, 0, 0);
    }
}

// Epilogue: bias (when BIAS) and ReLU (when p.relu) on the fp32
// accumulator, round to nearest even, masked store.  Lane owns C[m][n .. n+3]
// of each 4-register group; the bias of those four columns is loaded once
// for all the wave's rows.
template <class T, bool GENERIC, bool BIAS>
__device__ __forceinline__ void store_c(const f32x16 (&acc)[T::FM][T::FN], const GemmArgs &p,
                                        uint16_t *C, int64_t m0, int64_t n0, int wm, int wn,
                                        int lane)
{
    const int64_t M = p.M, N = p.N;
    const bool relu = p.relu != 0;
#pragma unroll
    for (int fn = 0; fn < T::FN; ++fn) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int64_t n = n0 + wn * T::TN + fn * 32 + 8 * g + 4 * (lane >> 5);
            float bv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if constexpr (BIAS && !GENERIC) {
                load_bias4<T::BF16>(p.bias, n, N, bv);
            } else if constexpr (BIAS) {
                // any alignment: one element at a time, inside the row only
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    if (n + t < N)
                        bv[t] = bits_to_float<T::BF16>(p.bias[n + t]);
            }
#pragma unroll
            for (int fm = 0; fm < T::FM; ++fm) {
                const int64_t m = m0 + wm * T::TM + fm * 32 + (lane & 31);
                if (m >= M)
                    continue;
                const f32x16 &v = acc[fm][fn];
                u32x2 w;
                w.x = epi_pack2<T::BF16>(v[4 * g + 0] + bv[0], v[4 * g + 1] + bv[1], relu);
                w.y = epi_pack2<T::BF16>(v[4 * g + 2] + bv[2], v[4 * g + 3] + bv[3], relu);
                uint16_t *dst = C + m * p.ldc + n;
                if constexpr (!GENERIC) {
                    if (n < N)
                        *reinterpret_cast<u32x2 *>(dst) = w;
                } else {
                    const uintptr_t da = reinterpret_cast<uintptr_t>(dst);
                    if (n + 4 <= N && (da & 3) == 0) {
                        *reinterpret_cast<u32x2_a4 *>(dst) = w;
                    } else if (n + 4 <= N) {
                        // 2 mod 4: one element, one aligned pair, one element
                        dst[0] = (uint16_t)(w.x & 0xffff);
                        *reinterpret_cast<uint32_t *>(dst + 1) = (w.x >> 16) | (w.y << 16);
                        dst[3] = (uint16_t)(w.y >> 16);
                    } else {
                        const uint16_t e[4] = {(uint16_t)(w.x & 0xffff), (uint16_t)(w.x >> 16),
                                               (uint16_t)(w.y & 0xffff), (uint16_t)(w.y >> 16)};
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            if (n + t < N)
                                dst[t] = e[t];
                    }
                }
            }
        }
    }
}

// GENERIC = false requires: A, B, C 16-byte aligned; lda, ldb, ldc, N, K
// multiples of 8 (so a 16-byte chunk is entirely inside or outside the
// matrix).  GENERIC = true accepts any layout and masks per element.
template <class T, bool GENERIC>
__global__ void __launch_bounds__(T::NT) gemm_relu_tile_kernel(GemmArgs p, int tilesM, int tilesN,
                                                               int groupM)
{
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * T::STAGE];
    const lds_u16 *lds = (const lds_u16 *)smem;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / T::WN, wn = wave % T::WN;
    int tm, tn;
    tile_coords(blockIdx.x, tilesM, tilesN, groupM, tm, tn);
    const int64_t bidx = blockIdx.y;
    const uint16_t *A = p.A + bidx * p.sA;
    const uint16_t *B = p.B + bidx * p.sB;
    uint16_t *C = p.C + bidx * p.sC;
    const int64_t M = p.M, N = p.N, K = p.K;
    const int64_t m0 = (int64_t)tm * T::BM, n0 = (int64_t)tn * T::BN;

    // Per-thread load plan: which chunks of the A and B tiles this thread
    // moves, where they live in global memory at K-tile 0 and in LDS.
    const uint16_t *pa[T::A_LD];
    int a_col[T::A_LD], a_dst[T::A_LD];
    bool a_ok[T::A_LD];
    bool a_first[T::A_LD], a_last[T::A_LD];   // first / last row of A
#pragma unroll
    for (int i = 0; i < T::A_LD; ++i) {
        const int q = tid + i * T::NT;
        const int r = q / T::CA, c = q % T::CA;
        a_ok[i] = (m0 + r) < M;
        a_first[i] = (m0 + r) == 0;
        a_last[i] = (m0 + r) == M - 1;
        a_col[i] = c * 8;
        pa[i] = A + (a_ok[i] ? (m0 + r) : 0) * p.lda + c * 8;
        a_dst[i] = r * T::BK + swz_a<T::CA>(r, c) * 8;
    }
    // (K,N) B: chunk (r, c) is row k0 + r, columns n0 + 8c ..; (N,K) B: chunk
    // (r, c) is row n0 + r, k columns k0 + 8c .. (the A plan, on B^T).
    const uint16_t *pb[T::B_LD];
    int b_row[T::B_LD], b_dst[T::B_LD];
    int64_t b_avail[T::B_LD];
    bool b_col0[T::B_LD];   // (K,N): chunk starts at column 0 of B
    bool b_ok[T::B_LD], b_first[T::B_LD], b_last[T::B_LD];   // (N,K): row n in range / first / last
#pragma unroll
    for (int i = 0; i < T::B_LD; ++i) {
        const int q = tid + i * T::NT;
        if constexpr (T::BT) {
            const int r = q / T::CA, c = q % T::CA;
            b_ok[i] = (n0 + r) < N;
            b_first[i] = (n0 + r) == 0;
            b_last[i] = (n0 + r) == N - 1;
            b_row[i] = c * 8;                       // the chunk's k column in the tile
            b_avail[i] = 0;
            b_col0[i] = false;
            pb[i] = B + (b_ok[i] ? (n0 + r) : 0) * p.ldb + c * 8;
            b_dst[i] = T::A_ELEMS + r * T::BK + swz_a<T::CA>(r, c) * 8;
        } else {
            const int r = q / T::CB, c = q % T::CB;
            b_row[i] = r;
            b_avail[i] = N - (n0 + c * 8);
            b_col0[i] = (n0 + c * 8) == 0;
            b_ok[i] = b_first[i] = b_last[i] = false;
            pb[i] = B + r * p.ldb + (b_avail[i] > 0 ? n0 + c * 8 : 0);
            b_dst[i] = T::A_ELEMS + r * T::BN + swz_b<T::CB>(r, c) * 8;
        }
    }

    u32x4 ra[T::A_LD], rb[T::B_LD];
    auto load_tile = [&](int kt) {
        const int64_t k0 = (int64_t)kt * T::BK;
#pragma unroll
        for (int i = 0; i < T::A_LD; ++i) {
            const int64_t kavail = K - (k0 + a_col[i]);
            ra[i] = u32x4{0, 0, 0, 0};
            if (a_ok[i] && kavail > 0) {
                if constexpr (GENERIC) {
                    const int64_t col = k0 + a_col[i];
                    const bool wok = !(a_first[i] && col == 0) && !(a_last[i] && kavail <= 8);
                    ra[i] = load8_masked(pa[i] + k0, kavail, wok);
                } else
                    ra[i] = *reinterpret_cast<const u32x4 *>(pa[i] + k0);
            }
        }
#pragma unroll
        for (int i = 0; i < T::B_LD; ++i) {
            rb[i] = u32x4{0, 0, 0, 0};
            if constexpr (T::BT) {
                const int64_t kavail = K - (k0 + b_row[i]);
                if (b_ok[i] && kavail > 0) {
                    if constexpr (GENERIC) {
                        const int64_t col = k0 + b_row[i];
                        const bool wok = !(b_first[i] && col == 0) && !(b_last[i] && kavail <= 8);
                        rb[i] = load8_masked(pb[i] + k0, kavail, wok);
                    } else
                        rb[i] = *reinterpret_cast<const u32x4 *>(pb[i] + k0);
                }
                continue;
            }
            if (b_avail[i] > 0 && k0 + b_row[i] < K) {
                const uint16_t *src = pb[i] + k0 * p.ldb;
                if constexpr (GENERIC) {
                    const int64_t row = k0 + b_row[i];
                    const bool wok = !(row == 0 && b_col0[i]) && !(row == K - 1 && b_avail[i] <= 8);
                    rb[i] = load8_masked(src, b_avail[i], wok);
                } else
                    rb[i] = *reinterpret_cast<const u32x4 *>(src);
            }
        }
    };
    auto store_tile = [&](int stage) {
        lds_u16 *base = (lds_u16 *)smem + stage * T::STAGE;
#pragma unroll
        for (int i = 0; i < T::A_LD; ++i)
            *reinterpret_cast<lds_u32x4 *>(base + a_dst[i]) = ra[i];
#pragma unroll
        for (int i = 0; i < T::B_LD; ++i)
            *reinterpret_cast<lds_u32x4 *>(base + b_dst[i]) = rb[i];
    };

    f32x16 acc[T::FM][T::FN];
#pragma unroll
    for (int fm = 0; fm < T::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < T::FN; ++fn)
            acc[fm][fn] = f32x16{};

    const int KT = (int)((K + T::BK - 1) / T::BK);
    if (KT > 0) {
        load_tile(0);
        store_tile(0);
        __syncthreads();
        for (int kt = 0; kt < KT; ++kt) {
            const int cur = kt & 1;
            if (kt + 1 < KT)
                load_tile(kt + 1);
            mma_stage<T>(lds + cur * T::STAGE, lds + cur * T::STAGE + T::A_ELEMS, acc, wm, wn, lane);
            if (kt + 1 < KT)
                store_tile(cur ^ 1);
            __syncthreads();
        }
    }

    // Epilogue (the bias-free form when there is no bias: the bias loads
    // otherwise cost the misaligned kernel ~14 % even when skipped at run time)
    if (p.bias != nullptr)
        store_c<T, GENERIC, true>(acc, p, C, m0, n0, wm, wn, lane);
    else
        store_c<T, GENERIC, false>(acc, p, C, m0, n0, wm, wn, lane);
}

template <class T, bool GENERIC>
hipError_t launch_tiles(const GemmArgs &p, hipStream_t stream, int groupM)
{
    const int64_t tilesM = (p.M + T::BM - 1) / T::BM;
    const int64_t tilesN = (p.N + T::BN - 1) / T::BN;
    const int64_t tiles = tilesM * tilesN;
    if (tiles > 0x7fffffff)
        return hipErrorInvalidValue;
    GemmArgs q = p;
    for (int64_t b0 = 0; b0 < p.batch; b0 += 65535) {
        const int64_t nb = (p.batch - b0) < 65535 ? (p.batch - b0) : 65535;
        q.A = p.A + b0 * p.sA;
        q.B = p.B + b0 * p.sB;
        q.C = p.C + b0 * p.sC;
        q.batch = nb;
        hipLaunchKernelGGL((gemm_relu_tile_kernel<T, GENERIC>), dim3((unsigned)tiles, (unsigned)nb),
                           dim3(T::NT), 0, stream, q, (int)tilesM, (int)tilesN, groupM);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

template <int MODE>
using Tile128 = Tile<128, 128, 32, 2, 2, MODE>;
using Tile256 = Tile<256, 256, 32, 2, 2>;
// Any-layout tile: eight waves of 64 x 32 and 64-wide K tiles (two waves per
// SIMD hide the masked loads' latency; half the barriers of BK = 32).  At
// 3001 x 5003 x 1000 with odd ldb and ldc: 98 us against 128 us for the
// four-wave 128 x 128 x 32 tile.
template <int MODE>
using TileAny = Tile<128, 128, 64, 2, 4, MODE>;

}  // namespace

// The any-layout kernel exists for every element type and B layout; the
// aligned register-staged kernels (kept for comparison) for fp16 with a
// (K,N) B only.
hipError_t launch_generic(const GemmArgs &p, hipStream_t stream, int groupM)
{
    switch ((p.bf16 ? 1 : 0) | (p.b_nk ? 2 : 0)) {
    case 0: return launch_tiles<TileAny<0>, true>(p, stream, groupM);
    case 1: return launch_tiles<TileAny<1>, true>(p, stream, groupM);
    case 2: return launch_tiles<TileAny<2>, true>(p, stream, groupM);
    default: return launch_tiles<TileAny<3>, true>(p, stream, groupM);
    }
}

hipError_t launch_tile128(const GemmArgs &p, hipStream_t stream, int groupM)
{
    if (p.bf16 || p.b_nk)
        return hipErrorInvalidValue;
    return launch_tiles<Tile128<0>, false>(p, stream, groupM);
}

hipError_t launch_tile256(const GemmArgs &p, hipStream_t stream, int groupM)
{
    if (p.bf16 || p.b_nk)
        return hipErrorInvalidValue;
    return launch_tiles<Tile256, false>(p, stream, groupM);
}

}  // namespace tg
