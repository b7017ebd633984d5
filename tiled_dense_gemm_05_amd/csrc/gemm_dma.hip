// Aligned fp16 GEMM + ReLU on gfx950 with a multi-stage direct-to-LDS
// pipeline.
//
// The tile program is the GEMM+ReLU of the "TileLang paper reading" page
// (hotelren.com), section 2: one workgroup per output tile, LDS operand tiles,
// an fp32 accumulator cleared to zero, a K loop pipelined over STAGES buffers,
// ReLU on the accumulator, copy to the fp16 C.  Section 3 of that page names
// the AMD pipeline primitives used here directly: loads that write LDS
// without passing through registers (buffer_load ... lds) and counter waits
// (s_waitcnt vmcnt) that release a stage once its loads have landed.
//
// gfx950 specifics:
//  * buffer_load_dwordx4 ... lds: each lane fetches 16 bytes and the wave
//    writes them as one contiguous 1 KiB block of LDS (lane L at byte 16 L,
//    block base in M0).  The XOR swizzle of the LDS tile is realised by
//    choosing, per lane, which global chunk lands in that fixed slot.
//  * Each operand is addressed through a buffer descriptor (SGPRs) whose base
//    advances by one K tile per iteration and one 32-bit VGPR offset per load.
//    Chunks outside the matrix (rows >= M, k >= K, columns >= N) get the
//    offset 2^31, at the descriptor's record count, and the hardware range
//    check returns zeros for them; every stage is fully written and the tails
//    contribute exact zeros.  This needs N and K to be multiples of 8 (a
//    16-byte chunk is wholly inside or outside) and 16-byte aligned rows.
//  * Before tile kt is computed, tiles kt+1 .. kt+STAGES-1 are in flight.
//    The last 16-wide k step of tile kt overlaps the switch to tile kt+1:
//    wait until this wave's loads of tile kt+1 have landed, barrier (every
//    wave is done reading tile kt's stage), then the matrix-core work of that
//    last step is interleaved with the loads of tile kt+STAGES into the stage
//    just released and with the LDS reads of tile kt+1's first fragments.
//  * Inside a tile, the fragments of the next k step are read from LDS while
//    the matrix cores work on the current one (two register sets).
//  * The loads are issued as inline assembly so the compiler does not treat
//    them as LDS stores that every LDS read must wait for; the kernel orders
//    them itself with vmcnt waits and barriers.
//  * Operand roles (the matrix core computes C^T = B^T A^T so a lane owns 4
//    consecutive columns of a C row), transpose reads of the row-major B
//    (ds_read_b64_tr_b16), the swizzles, the XCD-aware tile order and the
//    epilogue are shared with the register-staged kernel.
//  * The epilogue's common case (no bias, ReLU) takes three VALU
//    instructions per pair of outputs (two maxima, one packed conversion);
//    the C tile leaves through non-temporal stores, since no kernel here
//    reads an output again: a stream of many small products (1024 x
//    128x128x64) runs about 8 % faster than with ordinary stores.
#include <type_traits>

#include "tg_internal.h"
#include "tg_lds_dma.h"

namespace tg {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) f16x8 lds_f16x8;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

using dma::block_barrier;
using dma::dma16;
using dma::kOutOfRange;   // == the descriptors' record count
using dma::make_rsrc;
using dma::wait_vmcnt;

template <int BM_, int BN_, int BK_, int WM_, int WN_, int STAGES_, int OCC_ = 1, int KG_ = 1,
          bool SWZ_ = true, int MI_ = 32>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, STAGES = STAGES_;
    // matrix-core product: 32 (v_mfma_f32_32x32x16, 16-wide k steps) or 16
    // (v_mfma_f32_16x16x32, 32-wide k steps)
    static constexpr int MI = MI_;
    static constexpr int KSTEP = MI == 16 ? 32 : 16;
    using Acc = typename std::conditional<MI == 16, f32x4, f32x16>::type;
    static_assert(MI == 16 || MI == 32, "product shape");
    static constexpr int OCC = OCC_;                  // waves per SIMD the registers must allow
    static constexpr int KG = KG_;                    // K groups: wave groups on alternate K tiles
    static constexpr bool SWZ = SWZ_;                 // XOR-swizzled operand tiles (off: ablation)
    static constexpr int NW = WM * WN;                // waves per K group
    static constexpr int NT = 64 * NW * KG;           // threads
    static constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
    static constexpr int FM = TM / MI, FN = TN / MI;  // MIxMI fragments per wave
    static constexpr int CA = BK / 8, CB = BN / 8;    // 16-byte chunks per tile row
    static constexpr int A_ELEMS = BM * BK, B_ELEMS = BK * BN;
    static constexpr int STAGE = A_ELEMS + B_ELEMS;   // fp16 elements per stage
    static constexpr int A_LD = A_ELEMS / 512 / NW;   // 1 KiB loads per wave per tile
    static constexpr int B_LD = B_ELEMS / 512 / NW;
    static constexpr int LOADS = A_LD + B_LD;
    static constexpr int A_RPB = 64 / CA;             // tile rows per 1 KiB block
    static constexpr int B_RPB = 64 / CB;
    static constexpr int KSTEPS = BK / KSTEP;
    static constexpr int READS = FM + 2 * FN;         // LDS reads per k step
    // With 3+ stages the loads of tile kt+STAGES-1 are spread evenly over the
    // k steps of tile kt (DPS per step); with 2 stages the only free stage is
    // released at the last k step, which then issues all of them.
    static constexpr bool SPREAD = STAGES >= 3;
    static constexpr int DPS = SPREAD ? LOADS / KSTEPS : 0;
    static constexpr int AHEAD = SPREAD ? STAGES - 1 : STAGES;   // tile distance of the loads
    static constexpr int PROLOGUE = SPREAD ? STAGES - 1 : STAGES; // tiles issued up front
    // loads of this wave issued after tile kt+1's at the wait before the last k step
    static constexpr int WAIT_LAST = SPREAD ? (STAGES - 3) * LOADS + (KSTEPS - 1) * DPS : 0;
    static_assert(!SPREAD || LOADS % KSTEPS == 0, "loads per k step");
    static_assert((A_ELEMS / 512) % NW == 0 && (B_ELEMS / 512) % NW == 0, "blocks per wave");
    static_assert(CA <= 16 && CB <= 64 && 64 % CA == 0 && 64 % CB == 0, "rows per block");
    static_assert(TM % MI == 0 && TN % MI == 0 && BK % KSTEP == 0, "fragment shape");
    static_assert(LOADS * (STAGES - 1) <= 63, "vmcnt range");
    static_assert(KSTEPS <= 4, "k steps per tile");
    static constexpr int RING = KG * STAGES * STAGE * 2;        // bytes of LDS rings
    static constexpr int RED = (KG - 1) * NW * FM * FN * 64 * (int)sizeof(Acc); // partial sums of groups > 0
    static constexpr int CST = BM * BN * 2;                      // the fp16 C tile (epilogue)
    static constexpr int LDS0 = RING > RED ? RING : RED;
    static constexpr int LDS = LDS0 > CST ? LDS0 : CST;
    static_assert(LDS <= 160 * 1024, "LDS size");
    // a thread's loads of one tile share one swizzled column (see load plan)
    static_assert((NW * A_RPB) % 16 == 0 && (NW * B_RPB) % 4 == 0, "swizzle period");
    // the (K,N) B swizzle that also separates rows 8 apart needs a thread's
    // rows to be 16 apart
    static constexpr int BSWZ = MI == 16 && (NW * B_RPB) % 16 == 0 ? 16 : 32;
    // the fragment sets alternate between k steps and every tile starts on set 0
    static_assert(KSTEPS % 2 == 0, "an even number of k steps per tile");
};

// Element type and B layout of a configuration.  MODE bit 0: bf16 elements
// (fp16 otherwise); bit 1: B stored as (N,K) row-major, whose tile is BN rows
// of BK contiguous k, staged and read exactly like the A tile (no transpose
// read needed).
template <class C, int MODE>
struct Mode : C {
    static constexpr bool BF16 = (MODE & 1) != 0;
    static constexpr bool BT = (MODE & 2) != 0;
    static constexpr int B_RPB = BT ? 64 / C::CA : 64 / C::CB;   // B tile rows per 1 KiB
    static constexpr int READS = C::FM + (BT ? C::FN : 2 * C::FN);
    static_assert(!BT || (C::NW * (64 / C::CA)) % 16 == 0, "swizzle period");
};

template <int CA, bool ON = true>
__device__ __forceinline__ int swz_a(int row, int c)
{
    constexpr int rows_per_line = 16 / CA;
    if constexpr (!ON)
        return c;
    return c ^ ((row / rows_per_line) % CA);
}

// (K,N) B rows: a transpose read fetches 4 consecutive rows x 2 chunks per
// 16-lane group, so rows k .. k+3 move to different quarters of the bank line.
// With 16x16x32 products the two groups a read serves at once take rows 8
// apart at the same columns: bit 3 of the row also moves the chunk by 2.
template <int CB, bool ON = true, int MI = 32>
__device__ __forceinline__ int swz_b(int k, int c)
{
    if constexpr (!ON)
        return c;
    else if constexpr (CB >= 16 && MI == 16)
        return c ^ ((k & 3) << 2) ^ (((k >> 3) & 1) << 1);
    else if constexpr (CB >= 16)
        return c ^ ((k & 3) << 2);
    else if constexpr (CB == 8)
        return c ^ (((k >> 1) & 1) << 2);
    else
        return c;
}

// Piece r of the fragments of k step kk: r < FM is the A^T fragment r (lane
// holds A[row][8 consecutive k], one 16-byte read); FM + 2 fn + hh is half hh
// of the B^T fragment fn (a transpose read: source lane s of each 16-lane
// group points at row s / 4, columns 4 (s % 4) .. + 3 of a 4 x 16 block and
// receives one column's 4 consecutive k).
template <class T, int r>
__device__ __forceinline__ void read_piece(const lds_u16 *As, const lds_u16 *Bs, int kk, int wm,
                                           int wn, int lane, f16x8 (&af)[T::FM],
                                           s16x4 (&bh)[T::FN][2])
{
    // a fragment row is lane % MI; its 8 k are chunk lane / MI of the k step
    constexpr int LR = T::MI - 1, LS = T::MI == 16 ? 4 : 5;
    if constexpr (r < T::FM) {
        const int row = wm * T::TM + r * T::MI + (lane & LR);
        const int c = kk * (T::KSTEP / 8) + (lane >> LS);
        const int ca = swz_a<T::CA, T::SWZ>(row, c);
        af[r] = *reinterpret_cast<const lds_f16x8 *>(As + row * T::BK + ca * 8);
    } else if constexpr (T::BT) {
        // (N,K) B: the fragment is one 16-byte read of a B^T row, like A's
        constexpr int fn = r - T::FM;
        const int row = wn * T::TN + fn * T::MI + (lane & LR);
        const int c = kk * (T::KSTEP / 8) + (lane >> LS);
        const int cb = swz_a<T::CA, T::SWZ>(row, c);
        const s16x8 v = *reinterpret_cast<const __attribute__((address_space(3))) s16x8 *>(
            Bs + row * T::BK + cb * 8);
        bh[fn][0] = __builtin_shufflevector(v, v, 0, 1, 2, 3);
        bh[fn][1] = __builtin_shufflevector(v, v, 4, 5, 6, 7);
    } else {
        // a 32-wide fragment takes two 16-column blocks (lane bit 4), a
        // 16-wide one the lane's 16-lane group's 8 k (lane / 16)
        constexpr int fn = (r - T::FM) / 2, hh = (r - T::FM) % 2;
        const int k = kk * T::KSTEP + 8 * (lane >> LS) + 4 * hh + ((lane & 15) >> 2);
        const int n = wn * T::TN + fn * T::MI + (T::MI == 32 ? 16 * ((lane >> 4) & 1) : 0) +
                      4 * (lane & 3);
        const lds_u16 *src = Bs + k * T::BN + swz_b<T::CB, T::SWZ, T::BSWZ>(k, n >> 3) * 8 + (n & 7);
        bh[fn][hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)src);
    }
}

template <class T, int r = 0>
__device__ __forceinline__ void read_all(const lds_u16 *As, const lds_u16 *Bs, int kk, int wm,
                                         int wn, int lane, f16x8 (&af)[T::FM],
                                         s16x4 (&bh)[T::FN][2])
{
    if constexpr (r < T::READS) {
        read_piece<T, r>(As, Bs, kk, wm, wn, lane, af, bh);
        read_all<T, r + 1>(As, Bs, kk, wm, wn, lane, af, bh);
    }
}

template <class T>
__device__ __forceinline__ void join_b(const s16x4 (&bh)[T::FN][2], f16x8 (&bf)[T::FN])
{
#pragma unroll
    for (int fn = 0; fn < T::FN; ++fn)
        bf[fn] = __builtin_bit_cast(f16x8,
                                    __builtin_shufflevector(bh[fn][0], bh[fn][1], 0, 1, 2, 3, 4, 5, 6, 7));
}

// One matrix-core product (32x32x16 or 16x16x32) in the configuration's
// element type (the fragments hold raw 16-bit patterns either way).
template <class T>
__device__ __forceinline__ typename T::Acc mfma32(const f16x8 &b, const f16x8 &a,
                                                  const typename T::Acc &c)
{
    if constexpr (T::MI == 16) {
        if constexpr (T::BF16)
            return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b),
                                                           __builtin_bit_cast(bf16x8, a), c, 0, 0, 0);
        else
            return __builtin_amdgcn_mfma_f32_16x16x32_f16(b, a, c, 0, 0, 0);
    } else if constexpr (T::BF16) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, b),
                                                       __builtin_bit_cast(bf16x8, a), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(b, a, c, 0, 0, 0);
    }
}

// The four outputs a lane holds in group g of a fragment (four consecutive
// columns of one row), finished and packed: bias, activation and rounding.
// FAST is the common case, no bias and the ReLU, in three VALU instructions
// per pair of outputs (two maxima and one packed conversion).
template <class T, bool FAST>
__device__ __forceinline__ u32x2 finish4(const typename T::Acc &v, int g, const float (&bv)[4],
                                         bool relu)
{
    u32x2 w;
    if constexpr (FAST) {
        w.x = pack2<T::BF16, true>(v[4 * g + 0], v[4 * g + 1]);
        w.y = pack2<T::BF16, true>(v[4 * g + 2], v[4 * g + 3]);
    } else {
        w.x = epi_pack2<T::BF16>(v[4 * g + 0] + bv[0], v[4 * g + 1] + bv[1], relu);
        w.y = epi_pack2<T::BF16>(v[4 * g + 2] + bv[2], v[4 * g + 3] + bv[3], relu);
    }
    return w;
}

// Everything a thread needs to issue its loads of one tile.
template <class T>
struct LoadPlan {
    uint32_t a_voff[T::A_LD];   // byte offsets from the A descriptor, or out of range
    uint32_t b_voff[T::B_LD];
    int a_kcol;                 // the thread's column inside the K tile (A)
    int b_row0;                 // the thread's first row inside the K tile ((K,N) B)
    int b_kcol;                 // the thread's column inside the K tile ((N,K) B)
};

// b_rows_left: for a (K,N) B the rows of this K tile inside K; for an (N,K)
// B, 1 when the thread's k columns are inside K, else 0.
template <class T, int I>
__device__ __forceinline__ void issue_one(const LoadPlan<T> &lp, const i32x4 &ra, const i32x4 &rb,
                                          bool a_kok, int b_rows_left, uint32_t stage_addr,
                                          int wave)
{
    if constexpr (I < T::A_LD) {
        const uint32_t v = a_kok ? lp.a_voff[I] : kOutOfRange;
        dma16(ra, v, stage_addr + (uint32_t)((wave + I * T::NW) * 1024));
    } else {
        constexpr int J = I - T::A_LD;
        // (K,N) B: a whole K tile (BK rows left or more) needs no row test
        const bool ok = T::BT ? b_rows_left != 0
                              : b_rows_left >= T::BK ||
                                    (lp.b_row0 + J * T::NW * T::B_RPB) < b_rows_left;
        const uint32_t v = ok ? lp.b_voff[J] : kOutOfRange;
        dma16(rb, v, stage_addr + (uint32_t)(T::A_ELEMS * 2 + (wave + J * T::NW) * 1024));
    }
}

// One k step: the MFMAs on fragments (af, bf), with loads D0 .. D1-1 of a
// tile and the LDS reads of the next fragments (k step kkn of As/Bs) placed
// between them in program order: MFMA i is followed by load D0 + i and read i.
template <class T, int D0, int D1, int I = 0>
__device__ __forceinline__ void step(typename T::Acc (&acc)[T::FM][T::FN], const f16x8 (&af)[T::FM],
                                     const f16x8 (&bf)[T::FN], const LoadPlan<T> &lp,
                                     const i32x4 &ra, const i32x4 &rb, bool a_kok, int b_rows_left,
                                     uint32_t stage_addr, int wave, const lds_u16 *As,
                                     const lds_u16 *Bs, int kkn, int wm, int wn, int lane,
                                     f16x8 (&afn)[T::FM], s16x4 (&bhn)[T::FN][2])
{
    constexpr int MF = T::FM * T::FN;
    constexpr int ND = D1 - D0;
    constexpr int STEPS = MF > ND ? (MF > T::READS ? MF : T::READS) : (ND > T::READS ? ND : T::READS);
    if constexpr (I < STEPS) {
        if constexpr (I < MF) {
            constexpr int fm = I / T::FN, fn = I % T::FN;
            acc[fm][fn] = mfma32<T>(bf[fn], af[fm], acc[fm][fn]);
        }
        if constexpr (I < ND)
            issue_one<T, D0 + I>(lp, ra, rb, a_kok, b_rows_left, stage_addr, wave);
        if constexpr (I < T::READS)
            read_piece<T, I>(As, Bs, kkn, wm, wn, lane, afn, bhn);
        step<T, D0, D1, I + 1>(acc, af, bf, lp, ra, rb, a_kok, b_rows_left, stage_addr, wave, As,
                               Bs, kkn, wm, wn, lane, afn, bhn);
    }
}

// The k steps 0 .. KSTEPS-2 of a tile: step kk works on fragment set kk & 1,
// reads set (kk+1) & 1 and issues loads kk*DPS .. (kk+1)*DPS-1.
template <class T, int KK = 0>
__device__ __forceinline__ void inner_steps(typename T::Acc (&acc)[T::FM][T::FN], f16x8 (&af)[2][T::FM],
                                            f16x8 (&bf)[2][T::FN], const LoadPlan<T> &lp,
                                            const i32x4 &ra, const i32x4 &rb, bool a_kok,
                                            int b_rows_left, uint32_t stage_addr, int wave,
                                            const lds_u16 *As, const lds_u16 *Bs, int wm, int wn,
                                            int lane)
{
    if constexpr (KK + 1 < T::KSTEPS) {
        s16x4 bh[T::FN][2];
        step<T, KK * T::DPS, (KK + 1) * T::DPS>(acc, af[KK & 1], bf[KK & 1], lp, ra, rb, a_kok,
                                                 b_rows_left, stage_addr, wave, As, Bs, KK + 1, wm,
                                                 wn, lane, af[(KK + 1) & 1], bh);
        join_b<T>(bh, bf[(KK + 1) & 1]);
        inner_steps<T, KK + 1>(acc, af, bf, lp, ra, rb, a_kok, b_rows_left, stage_addr, wave, As,
                               Bs, wm, wn, lane);
    }
}

// f(kt + S, S, whole) for S = S0 .. N-1, S a compile-time constant.
template <int S, int N, class F, class W>
__device__ __forceinline__ void for_stages(F &f, int kt, W whole)
{
    if constexpr (S < N) {
        f(kt + S, std::integral_constant<int, S>{}, whole);
        for_stages<S + 1, N>(f, kt, whole);
    }
}

template <class T, int I = 0>
__device__ __forceinline__ void issue_tile(const LoadPlan<T> &lp, const i32x4 &ra, const i32x4 &rb,
                                           bool a_kok, int b_rows_left, uint32_t stage_addr,
                                           int wave)
{
    if constexpr (I < T::LOADS) {
        issue_one<T, I>(lp, ra, rb, a_kok, b_rows_left, stage_addr, wave);
        issue_tile<T, I + 1>(lp, ra, rb, a_kok, b_rows_left, stage_addr, wave);
    }
}

template <class T>
__global__ void __launch_bounds__(T::NT) __attribute__((amdgpu_waves_per_eu(T::OCC)))
gemm_relu_dma_kernel(GemmArgs p, int tilesM, int tilesN, int groupM)
{
    __shared__ __attribute__((aligned(1024))) uint16_t smem[T::LDS / 2];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
    // K group kg works on K tiles kg, kg + KG, ... with its own LDS ring;
    // `wave` is the wave's index inside its group
    const int kg = wave_all / T::NW;
    const int wave = wave_all % T::NW;
    const lds_u16 *lds = (const lds_u16 *)smem + kg * T::STAGES * T::STAGE;
    const uint32_t lds_base = (uint32_t)(uintptr_t)lds;
    const int wm = wave / T::WN, wn = wave % T::WN;
    int tm, tn;
    tile_coords(blockIdx.x, tilesM, tilesN, groupM, tm, tn);
    const int64_t bidx = blockIdx.y;
    const int64_t M = p.M, N = p.N, K = p.K;
    const int64_t m0 = (int64_t)tm * T::BM, n0 = (int64_t)tn * T::BN;
    // operand panels of this tile; the descriptors advance along K
    const uint16_t *Ab = p.A + bidx * p.sA + m0 * p.lda;
    const uint16_t *Bb = p.B + bidx * p.sB + (T::BT ? n0 * p.ldb : n0);
    uint16_t *C = p.C + bidx * p.sC;

    // Load plan.  Wave w moves 1 KiB blocks w, w + NW, ... of each operand
    // tile; lane L of a block covers its LDS bytes 16 L .. 16 L + 15, i.e.
    // physical chunk L % C of row L / C; the logical chunk stored there is the
    // XOR-swizzled one.  Every block of a thread has the same swizzle.
    LoadPlan<T> lp;
    {
        const int r0 = wave * T::A_RPB + lane / T::CA;
        const int c = swz_a<T::CA, T::SWZ>(r0, lane % T::CA);
        lp.a_kcol = c * 8;
#pragma unroll
        for (int i = 0; i < T::A_LD; ++i) {
            const int row = r0 + i * T::NW * T::A_RPB;
            lp.a_voff[i] = (m0 + row < M) ? (uint32_t)((row * p.lda + c * 8) * 2) : kOutOfRange;
        }
    }
    if constexpr (T::BT) {
        // (N,K) B: rows are output columns n0 + row, chunks run along K
        const int r0 = wave * T::B_RPB + lane / T::CA;
        const int c = swz_a<T::CA, T::SWZ>(r0, lane % T::CA);
        lp.b_kcol = c * 8;
        lp.b_row0 = 0;
#pragma unroll
        for (int j = 0; j < T::B_LD; ++j) {
            const int row = r0 + j * T::NW * T::B_RPB;
            lp.b_voff[j] = (n0 + row < N) ? (uint32_t)((row * p.ldb + c * 8) * 2) : kOutOfRange;
        }
    } else {
        const int r0 = wave * T::B_RPB + lane / T::CB;
        const int c = swz_b<T::CB, T::SWZ, T::BSWZ>(r0, lane % T::CB);
        lp.b_row0 = r0;
        lp.b_kcol = 0;
        const bool col_ok = n0 + c * 8 < N;
#pragma unroll
        for (int j = 0; j < T::B_LD; ++j) {
            const int row = r0 + j * T::NW * T::B_RPB;
            lp.b_voff[j] = col_ok ? (uint32_t)((row * p.ldb + c * 8) * 2) : kOutOfRange;
        }
    }
    // the group's t-th K tile is K tile t * KG + kg
    auto rsrc_a = [&](int t) { return make_rsrc(Ab + ((int64_t)t * T::KG + kg) * T::BK); };
    auto rsrc_b = [&](int t) {
        const int64_t k0 = ((int64_t)t * T::KG + kg) * T::BK;
        return make_rsrc(Bb + (T::BT ? k0 : k0 * p.ldb));
    };
    auto a_kok = [&](int t) { return ((int64_t)t * T::KG + kg) * T::BK + lp.a_kcol < K; };
    auto b_left = [&](int t) {
        const int64_t k0 = ((int64_t)t * T::KG + kg) * T::BK;
        if constexpr (T::BT)
            return (int)(k0 + lp.b_kcol < K);
        const int64_t r = K - k0;
        return (int)(r < 0 ? 0 : (r > T::BK ? T::BK : r));
    };

    typename T::Acc acc[T::FM][T::FN];
#pragma unroll
    for (int fm = 0; fm < T::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < T::FN; ++fn)
            acc[fm][fn] = typename T::Acc{};

    // every group runs the same number of tiles (a group past the end of K
    // loads zeros) so that the workgroup barriers line up
    const int KT = (int)(((K + T::BK - 1) / T::BK + T::KG - 1) / T::KG);
    f16x8 af[2][T::FM], bf[2][T::FN];
    if (KT > 0) {
        // Issue the first tiles (tiles past the end of K load zeros and never
        // touch memory), then wait for tile 0.
#pragma unroll
        for (int s = 0; s < T::PROLOGUE; ++s)
            issue_tile<T>(lp, rsrc_a(s), rsrc_b(s), a_kok(s), b_left(s),
                          lds_base + (uint32_t)(s * T::STAGE * 2), wave);
        wait_vmcnt<(T::PROLOGUE - 1) * T::LOADS>();
        block_barrier();
        s16x4 bh[T::FN][2];
        read_all<T>(lds, lds + T::A_ELEMS, 0, wm, wn, lane, af[0], bh);
        join_b<T>(bh, bf[0]);
    }

    // Iteration kt loads the group's K tile kt + AHEAD.  Its operand
    // addresses and the K left from its first k advance by a fixed step per
    // iteration: a few scalar adds instead of a 64-bit product per tile.
    const int64_t kstep = (int64_t)T::KG * T::BK;
    const int64_t k_first = ((int64_t)T::AHEAD * T::KG + kg) * T::BK;
    const int64_t b_adv = T::BT ? kstep : kstep * p.ldb;
    // descriptors carried from iteration to iteration: only the base moves
    i32x4 ra_c = make_rsrc(Ab + k_first);
    i32x4 rb_c = make_rsrc(Bb + (T::BT ? k_first : k_first * p.ldb));
    const uint64_t a_adv_bytes = (uint64_t)kstep * 2, b_adv_bytes = (uint64_t)b_adv * 2;
    auto advance = [](i32x4 &r, uint64_t by) __attribute__((always_inline)) {
        // the 48-bit base sits in words 0-1 with a zero stride above it
        const uint64_t v = (((uint64_t)(uint32_t)r.y << 32) | (uint32_t)r.x) + by;
        r.x = (int)(uint32_t)v;
        r.y = (int)(uint32_t)(v >> 32);
    };
    int k_rem = (int)(K - k_first);   // negative past the end; K < 2^31
    // One iteration.  S is kt % STAGES when it is known at compile time (-1
    // otherwise): in the unrolled rounds of the ring every stage offset is a
    // constant.  WHOLE: the K tile it loads lies wholly inside K, so no load
    // needs a K test.
    auto iteration = [&](int kt, auto s_ic, auto whole_ic) __attribute__((always_inline)) {
        constexpr int S = decltype(s_ic)::value;
        constexpr bool WHOLE = decltype(whole_ic)::value;
        const int stage = S >= 0 ? S : kt % T::STAGES;
        // loads of tile kt + AHEAD go to the stage that tile held
        const int lstage = S >= 0 ? (S + T::AHEAD) % T::STAGES : (kt + T::AHEAD) % T::STAGES;
        const int nstage = S >= 0 ? (S + 1) % T::STAGES : (kt + 1) % T::STAGES;
        const lds_u16 *As = lds + stage * T::STAGE;
        const lds_u16 *Bs = As + T::A_ELEMS;
        const uint32_t laddr = lds_base + (uint32_t)(lstage * T::STAGE * 2);
        const i32x4 ra = ra_c, rb = rb_c;
        const bool akok = WHOLE || lp.a_kcol < k_rem;
        const int bleft = T::BT ? (int)(WHOLE || lp.b_kcol < k_rem)
                        : WHOLE ? T::BK
                                : (k_rem < 0 ? 0 : (k_rem > T::BK ? T::BK : k_rem));
        inner_steps<T>(acc, af, bf, lp, ra, rb, akok, bleft, laddr, wave, As, Bs, wm, wn, lane);
        constexpr int cur = (T::KSTEPS - 1) & 1, nxt = T::KSTEPS & 1;
        // Tile kt+1 has landed once at most WAIT_LAST later loads of this wave
        // are outstanding.  On the last tile this step still runs (one MFMA
        // chain for the register allocator): its loads are past the end of K
        // and read nothing, its fragment reads are never used.
        wait_vmcnt<T::WAIT_LAST>();
        block_barrier();
        {
            const lds_u16 *An = lds + nstage * T::STAGE;
            s16x4 bh[T::FN][2];
            constexpr int D0 = T::SPREAD ? (T::KSTEPS - 1) * T::DPS : 0;
            step<T, D0, T::LOADS>(acc, af[cur], bf[cur], lp, ra, rb, akok, bleft, laddr, wave, An,
                                  An + T::A_ELEMS, 0, wm, wn, lane, af[nxt], bh);
            join_b<T>(bh, bf[nxt]);
        }
        advance(ra_c, a_adv_bytes);
        advance(rb_c, b_adv_bytes);
        k_rem -= (int)kstep;
    };
    // Rounds of STAGES iterations whose loads all fall on K tiles wholly
    // inside K (the group's t-th tile is whole for t < K / kstep), then the
    // rest one at a time with the K tests.
    const int KTW = (int)(K / kstep);
    int kt = 0;
    for (; kt + T::STAGES + T::AHEAD <= KTW; kt += T::STAGES)
        for_stages<0, T::STAGES>(iteration, kt, std::true_type{});
    for (; kt < KT; ++kt)
        iteration(kt, std::integral_constant<int, -1>{}, std::false_type{});
    // loads issued past the end of K must land before the LDS is released
    wait_vmcnt<0>();

    if constexpr (T::KG > 1) {
        // Groups 1 .. KG-1 hand their partial sums to group 0 through LDS;
        // group 0 adds them in group order (deterministic).
        block_barrier();
        typedef __attribute__((address_space(3))) typename T::Acc lds_acc;
        lds_acc *part = (lds_acc *)smem;
        if (kg > 0) {
#pragma unroll
            for (int fm = 0; fm < T::FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < T::FN; ++fn)
                    part[(((kg - 1) * T::NW + wave) * T::FM * T::FN + fm * T::FN + fn) * 64 + lane] =
                        acc[fm][fn];
        }
        block_barrier();
        if (kg == 0) {
            for (int g = 1; g < T::KG; ++g)
#pragma unroll
                for (int fm = 0; fm < T::FM; ++fm)
#pragma unroll
                    for (int fn = 0; fn < T::FN; ++fn)
                        acc[fm][fn] +=
                            part[(((g - 1) * T::NW + wave) * T::FM * T::FN + fm * T::FN + fn) * 64 + lane];
        }
    }

    // Epilogue: bias, ReLU, round to nearest even, and the fp16 tile staged
    // in LDS (16-byte chunks of each row XOR-swizzled by the row) so that the
    // global stores are whole 16-byte chunks per lane, a wave writing
    // contiguous runs of rows instead of 8 bytes into 32 different rows.
    block_barrier();   // every wave is done with the LDS ring / partial sums
    lds_u16 *cst = (lds_u16 *)smem;
    if (kg == 0) {
        const bool relu = p.relu != 0;
        // a lane holds four consecutive columns of one C row per group g:
        // 32x32 fragments, row lane % 32, columns 8 g + 4 (lane / 32) (g < 4);
        // 16x16 fragments, row lane % 16, columns 4 (lane / 16) (one group)
        constexpr int NG = T::MI == 32 ? 4 : 1;
        auto stage_c = [&](auto fast_c) __attribute__((always_inline)) {
            constexpr bool FAST = decltype(fast_c)::value;
#pragma unroll
            for (int fn = 0; fn < T::FN; ++fn) {
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    // the lane's four columns of this group, the same in every row
                    const int col = wn * T::TN + fn * T::MI +
                                    (T::MI == 32 ? 8 * g + 4 * (lane >> 5) : 4 * (lane >> 4));
                    float bv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                    if constexpr (!FAST)
                        load_bias4<T::BF16>(p.bias, n0 + col, N, bv);
#pragma unroll
                    for (int fm = 0; fm < T::FM; ++fm) {
                        const int row = wm * T::TM + fm * T::MI + (lane & (T::MI - 1));
                        const u32x2 w = finish4<T, FAST>(acc[fm][fn], g, bv, relu);
                        const int phys = (col >> 3) ^ (row % T::CB);
                        *reinterpret_cast<__attribute__((address_space(3))) u32x2 *>(
                            cst + row * T::BN + phys * 8 + (col & 4)) = w;
                    }
                }
            }
        };
        if (p.bias == nullptr && relu)
            stage_c(std::true_type{});
        else
            stage_c(std::false_type{});
    }
    block_barrier();
    // N % 8 == 0 and 16-byte aligned rows: every chunk is wholly in or out
    for (int q = tid; q < T::BM * T::CB; q += T::NT) {
        const int row = q / T::CB, c = q % T::CB;
        const int64_t gm = m0 + row, gn = n0 + c * 8;
        if (gm < M && gn < N) {
            const int phys = c ^ (row % T::CB);
            const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4 *>(
                cst + row * T::BN + phys * 8);
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(C + gm * p.ldc + gn));
        }
    }
}

template <class T>
hipError_t launch_dma(const GemmArgs &p, hipStream_t stream, int groupM)
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
        hipLaunchKernelGGL((gemm_relu_dma_kernel<T>), dim3((unsigned)tiles, (unsigned)nb), dim3(T::NT),
                           0, stream, q, (int)tilesM, (int)tilesN, groupM);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// Persistent form for many short problems (a strided batch of small GEMMs, or
// any call whose K is a few tiles): the work is a list of items, one output
// tile of one batch entry each, and a grid of one workgroup per CU walks the
// list.  The ring of K tiles runs straight across item boundaries, so the
// loads of the next items are in flight while an item's products, epilogue
// and stores run; in the one-tile-per-workgroup launch every workgroup loads,
// then computes, then stores, and the memory system sees all the reads and
// then all the writes.
//
//  * Workgroup g of G takes items g', g' + G, g' + 2G, ... where g' numbers
//    the workgroups XCD by XCD (workgroup g runs on XCD g % 8), so the items
//    an XCD holds at one time are neighbours.
//  * An item's K tiles are positions of the workgroup's stream; position q's
//    tile sits in stage q % STAGES and the loads of position q + STAGES - 1
//    are spread over the k steps of position q, exactly as in
//    gemm_relu_dma_kernel.  Positions past the end load zeros without
//    touching memory.
//  * After an item's last product each wave writes its TM x TN tile through
//    its own LDS area (16-byte chunks XOR-swizzled by the row), reads it back
//    as whole 16-byte chunks of rows and stores them: no workgroup barrier,
//    and the ring is not touched.
//  * The counter waits count only the loads issued after the awaited tile;
//    stores issued in between are awaited too, since loads and stores share
//    the counter and need not complete in order with respect to each other.
template <class T>
__global__ void __launch_bounds__(T::NT) __attribute__((amdgpu_waves_per_eu(T::OCC)))
gemm_relu_dma_stream_kernel(GemmArgs p, int tilesM, int tilesN, int items, int KT)
{
    static_assert(T::KG == 1 && T::SPREAD, "one K group, loads spread over the k steps");
    constexpr int CBW = T::TN / 8;                       // 16-byte chunks per wave-tile row
    constexpr int CW = T::TM * T::TN;                    // fp16 elements of a wave's C area
    static_assert(CBW <= 64 && 64 % CBW == 0 && (CW / 8) % 64 == 0, "wave tile");
    static_assert(T::RING + T::NW * CW * 2 <= 160 * 1024, "LDS size");
    __shared__ __attribute__((aligned(1024))) uint16_t smem[T::RING / 2 + T::NW * CW];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / T::WN, wn = wave % T::WN;
    const lds_u16 *lds = (const lds_u16 *)smem;
    const uint32_t lds_base = (uint32_t)(uintptr_t)lds;
    lds_u16 *cw = (lds_u16 *)smem + T::RING / 2 + wave * CW;

    const int G = gridDim.x;
    const int g = blockIdx.x;
    const int first = (G % 8 == 0) ? (g % 8) * (G / 8) + g / 8 : g;
    const int mine = first < items ? (items - first + G - 1) / G : 0;
    const int Q = mine * KT;
    const int tiles = tilesM * tilesN;
    const int64_t M = p.M, N = p.N, K = p.K;

    // the load-plan parts that do not depend on the item
    int a_r0, a_c, b_r0, b_c;
    if constexpr (T::BT) {
        a_r0 = wave * T::A_RPB + lane / T::CA;
        a_c = swz_a<T::CA, T::SWZ>(a_r0, lane % T::CA);
        b_r0 = wave * T::B_RPB + lane / T::CA;
        b_c = swz_a<T::CA, T::SWZ>(b_r0, lane % T::CA);
    } else {
        a_r0 = wave * T::A_RPB + lane / T::CA;
        a_c = swz_a<T::CA, T::SWZ>(a_r0, lane % T::CA);
        b_r0 = wave * T::B_RPB + lane / T::CB;
        b_c = swz_b<T::CB, T::SWZ, T::BSWZ>(b_r0, lane % T::CB);
    }

    // A cursor holds a position's item (batch entry and tile) and K tile.
    // Advancing moves to the next K tile, or after an item's last one to this
    // workgroup's next item, G items further on; the divisions are done once.
    struct Cursor {
        int b, tm, tn, kt;
    };
    const int dB = G / tiles, dT = G - dB * tiles;
    const int dTM = dT / tilesN, dTN = dT - dTM * tilesN;
    Cursor c0;
    {
        const int f = first < items ? first : 0;
        c0.b = f / tiles;
        const int t = f - c0.b * tiles;
        c0.tm = t / tilesN;
        c0.tn = t - c0.tm * tilesN;
        c0.kt = 0;
    }
    auto advance = [&](Cursor &c) __attribute__((always_inline)) {
        if (++c.kt < KT)
            return;
        c.kt = 0;
        c.b += dB;
        c.tm += dTM;
        c.tn += dTN;
        if (c.tn >= tilesN) {
            c.tn -= tilesN;
            ++c.tm;
        }
        if (c.tm >= tilesM) {
            c.tm -= tilesM;
            ++c.b;
        }
    };

    // Everything the loads of position q need (zeros past the end).
    struct Load {
        LoadPlan<T> lp;
        i32x4 ra, rb;
        bool akok;
        int bleft;
    };
    // (A position past the end reads nothing: every offset is out of range,
    // whatever the cursor holds.)
    auto plan = [&](const Cursor &c, bool live) __attribute__((always_inline)) {
        Load L;
        const int64_t k0 = (int64_t)c.kt * T::BK;
        const int64_t m0 = (int64_t)c.tm * T::BM, n0 = (int64_t)c.tn * T::BN;
        const uint16_t *Ab = p.A + c.b * p.sA + m0 * p.lda + k0;
        const uint16_t *Bb = p.B + c.b * p.sB + (T::BT ? n0 * p.ldb + k0 : k0 * p.ldb + n0);
        L.ra = make_rsrc(Ab);
        L.rb = make_rsrc(Bb);
        L.lp.a_kcol = a_c * 8;
#pragma unroll
        for (int i = 0; i < T::A_LD; ++i) {
            const int row = a_r0 + i * T::NW * T::A_RPB;
            L.lp.a_voff[i] = (live && m0 + row < M) ? (uint32_t)((row * p.lda + a_c * 8) * 2) : kOutOfRange;
        }
        if constexpr (T::BT) {
            L.lp.b_kcol = b_c * 8;
            L.lp.b_row0 = 0;
#pragma unroll
            for (int j = 0; j < T::B_LD; ++j) {
                const int row = b_r0 + j * T::NW * T::B_RPB;
                L.lp.b_voff[j] = (live && n0 + row < N) ? (uint32_t)((row * p.ldb + b_c * 8) * 2) : kOutOfRange;
            }
            L.bleft = live && k0 + L.lp.b_kcol < K;
        } else {
            L.lp.b_kcol = 0;
            L.lp.b_row0 = b_r0;
            const bool col_ok = live && n0 + b_c * 8 < N;
#pragma unroll
            for (int j = 0; j < T::B_LD; ++j) {
                const int row = b_r0 + j * T::NW * T::B_RPB;
                L.lp.b_voff[j] = col_ok ? (uint32_t)((row * p.ldb + b_c * 8) * 2) : kOutOfRange;
            }
            const int64_t r = K - k0;
            L.bleft = live ? (int)(r < 0 ? 0 : (r > T::BK ? T::BK : r)) : 0;
        }
        L.akok = live && k0 + L.lp.a_kcol < K;
        return L;
    };

    typename T::Acc acc[T::FM][T::FN];
#pragma unroll
    for (int fm = 0; fm < T::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < T::FN; ++fn)
            acc[fm][fn] = typename T::Acc{};

    f16x8 af[2][T::FM], bf[2][T::FN];
    Cursor cl = c0, cc = c0;   // positions being loaded / computed
    if (Q > 0) {
#pragma unroll
        for (int s = 0; s < T::PROLOGUE; ++s) {
            const Load L = plan(cl, s < Q);
            advance(cl);
            issue_tile<T>(L.lp, L.ra, L.rb, L.akok, L.bleft, lds_base + (uint32_t)(s * T::STAGE * 2), wave);
        }
        wait_vmcnt<(T::PROLOGUE - 1) * T::LOADS>();
        block_barrier();
        s16x4 bh[T::FN][2];
        read_all<T>(lds, lds + T::A_ELEMS, 0, wm, wn, lane, af[0], bh);
        join_b<T>(bh, bf[0]);
    }

    for (int q = 0; q < Q; ++q) {
        const int stage = q % T::STAGES;
        const lds_u16 *As = lds + stage * T::STAGE;
        const lds_u16 *Bs = As + T::A_ELEMS;
        const int ql = q + T::AHEAD;
        const uint32_t laddr = lds_base + (uint32_t)((ql % T::STAGES) * T::STAGE * 2);
        const Load L = plan(cl, ql < Q);
        advance(cl);
        inner_steps<T>(acc, af, bf, L.lp, L.ra, L.rb, L.akok, L.bleft, laddr, wave, As, Bs, wm, wn, lane);
        constexpr int cur = (T::KSTEPS - 1) & 1, nxt = T::KSTEPS & 1;
        wait_vmcnt<T::WAIT_LAST>();
        block_barrier();
        {
            const lds_u16 *An = lds + ((q + 1) % T::STAGES) * T::STAGE;
            s16x4 bh[T::FN][2];
            constexpr int D0 = (T::KSTEPS - 1) * T::DPS;
            step<T, D0, T::LOADS>(acc, af[cur], bf[cur], L.lp, L.ra, L.rb, L.akok, L.bleft, laddr, wave,
                                  An, An + T::A_ELEMS, 0, wm, wn, lane, af[nxt], bh);
            join_b<T>(bh, bf[nxt]);
        }
        if (cc.kt != KT - 1) {
            advance(cc);
            continue;
        }

        // Epilogue of the item: bias, activation, rounding; the wave's tile
        // through its LDS area; whole 16-byte chunks of rows to C.
        const int64_t rbase = (int64_t)cc.tm * T::BM + wm * T::TM;
        const int64_t cbase = (int64_t)cc.tn * T::BN + wn * T::TN;
        const bool relu = p.relu != 0;
        constexpr int NG = T::MI == 32 ? 4 : 1;
        auto stage_c = [&](auto fast_c) __attribute__((always_inline)) {
            constexpr bool FAST = decltype(fast_c)::value;
#pragma unroll
            for (int fn = 0; fn < T::FN; ++fn) {
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) {
                    const int col = fn * T::MI + (T::MI == 32 ? 8 * gi + 4 * (lane >> 5) : 4 * (lane >> 4));
                    float bv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                    if constexpr (!FAST)
                        load_bias4<T::BF16>(p.bias, cbase + col, N, bv);
#pragma unroll
                    for (int fm = 0; fm < T::FM; ++fm) {
                        const int row = fm * T::MI + (lane & (T::MI - 1));
                        const u32x2 o = finish4<T, FAST>(acc[fm][fn], gi, bv, relu);
                        const int phys = (col >> 3) ^ (row % CBW);
                        *reinterpret_cast<__attribute__((address_space(3))) u32x2 *>(
                            cw + row * T::TN + phys * 8 + (col & 4)) = o;
                    }
                }
            }
        };
        if (p.bias == nullptr && relu)
            stage_c(std::true_type{});
        else
            stage_c(std::false_type{});
        asm volatile("" ::: "memory");   // the wave's LDS writes precede its reads
        uint16_t *Cb = p.C + cc.b * p.sC;
#pragma unroll
        for (int i = 0; i < CW / 8 / 64; ++i) {
            const int qq = i * 64 + lane;
            const int row = qq / CBW, c = qq % CBW;
            const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4 *>(
                cw + row * T::TN + (c ^ (row % CBW)) * 8);
            const int64_t gm = rbase + row, gn = cbase + c * 8;
            if (gm < M && gn < N)
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(Cb + gm * p.ldc + gn));
        }
#pragma unroll
        for (int fm = 0; fm < T::FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < T::FN; ++fn)
                acc[fm][fn] = typename T::Acc{};
        advance(cc);
    }
    // loads issued past the end must land before the workgroup ends
    wait_vmcnt<0>();
}

template <class T>
hipError_t launch_stream(const GemmArgs &p, hipStream_t stream)
{
    const int64_t tilesM = (p.M + T::BM - 1) / T::BM;
    const int64_t tilesN = (p.N + T::BN - 1) / T::BN;
    const int64_t items = tilesM * tilesN * p.batch;
    const int64_t KT = (p.K + T::BK - 1) / T::BK;
    if (items <= 0 || KT <= 0)
        return hipSuccess;
    if (items > 0x3fffffff || KT > 0x3fffffff || items * KT > 0x3fffffff)
        return hipErrorInvalidValue;
    const int cus = host_device_cus();
    if (cus <= 0)
        return hipErrorInvalidDevice;
    // workgroups a CU holds at once: by registers (OCC waves per SIMD) and LDS
    constexpr int kLds = T::RING + T::NW * T::TM * T::TN * 2;
    constexpr int by_regs = 4 * T::OCC / T::NW > 0 ? 4 * T::OCC / T::NW : 1;
    constexpr int per_cu = by_regs < (160 * 1024) / kLds ? by_regs : (160 * 1024) / kLds;
    const int64_t slots = (int64_t)cus * per_cu;
    const int64_t grid = items < slots ? items : slots;
    hipLaunchKernelGGL((gemm_relu_dma_stream_kernel<T>), dim3((unsigned)grid), dim3(T::NT), 0, stream,
                       p, (int)tilesM, (int)tilesN, (int)items, (int)KT);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Ragged layouts: an aligned A (16-byte aligned rows, K a multiple of 8) with a
// (K,N) B and a C whose rows may start at any 2-byte boundary (odd or
// unaligned ldb / ldc, N not a multiple of 8, B or C pointers at 2 mod 16).
//
//  * A is staged exactly as in gemm_relu_dma_kernel (direct to LDS, two
//    stages, loads two K tiles ahead).
//  * B goes through registers.  Each 16-byte chunk of a B row is read as the
//    4-byte aligned window that holds it: one 16-byte load at the dword
//    boundary at or below the chunk and, when the chunk starts at 2 mod 4, one
//    4-byte load for the element that spills past that window; a funnel shift
//    by 0 or 16 bits puts the eight elements in place, and one 16-byte LDS
//    write stores them at the chunk's swizzled slot, where the transpose reads
//    of the aligned kernel find them.  A chunk cut by the N edge reads only the
//    dwords that hold one of its elements and zeroes the rest, so no access
//    leaves the 4-byte words of the operand.  The loads of tile kt+2 are
//    issued after the second k step of tile kt and written to LDS at the same
//    point of tile kt+1, so they have a whole tile of matrix work to land and
//    the LDS writes stay clear of the barrier that ends the tile.
//  * The epilogue stages the C tile in LDS with each row shifted by the parity
//    of its first element's address (row stride BN + 8), so that every
//    interior 16-byte chunk of a row lines up with a 4-byte aligned address
//    and goes out as one 16-byte store; the chunks at the row's two ends are
//    stored element by element.
// Every configuration computes each output with the same sequence of 16-wide
// k steps as the aligned kernel, so both give the same bits.

typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));

template <class T>
struct RaggedPlan {
    static constexpr int NCH = T::B_ELEMS / 8 / T::NT;   // B chunks per thread per tile
    static constexpr int RSTEP = T::NT / T::CB;          // tile rows between them
    static_assert(NCH * RSTEP == T::BK && T::NT % T::CB == 0, "B chunk plan");
    static constexpr int CLD = T::BN + 8;                // staged C row (elements)
    static constexpr int CCH = CLD / 8;                  // 16-byte chunks per staged row
    static constexpr int CST = T::BM * CLD * 2;          // staged C tile (bytes)
    static constexpr int RING = T::STAGES * T::STAGE * 2;
    static constexpr int LDS = RING > CST ? RING : CST;
    static_assert(LDS <= 160 * 1024, "LDS size");
};

// The raw dwords of one thread's B chunks for one K tile.
template <class T>
struct BRegs {
    u32x4 w[RaggedPlan<T>::NCH];   // the 16-byte window (or its first four dwords)
    uint32_t x[RaggedPlan<T>::NCH];   // the dword after it
    uint32_t sh[RaggedPlan<T>::NCH];  // funnel shift: 0 or 16 bits
};

// Issues the loads of this thread's B chunks of the K tile starting at row
// k0: tile row row0 + j * RSTEP, columns n0 + col .. + 7 (nv of them valid).
template <class T>
__device__ __forceinline__ void ragged_b_load(BRegs<T> &br, const uint16_t *Bb, int64_t k0,
                                              int64_t K, int64_t ldb, int64_t n0, int row0,
                                              int col, int64_t nv)
{
    constexpr int NCH = RaggedPlan<T>::NCH, RSTEP = RaggedPlan<T>::RSTEP;
    // descriptor at the dword boundary at or below (k0, n0); d = 1 when that
    // element sits at 2 mod 4
    const uintptr_t a = reinterpret_cast<uintptr_t>(Bb + k0 * ldb + n0);
    const int d = (int)((a >> 1) & 1);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void *>(a & ~(uintptr_t)3), (short)0, (int)kOutOfRange, 0x00020000);
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const int r = row0 + j * RSTEP;
        const bool row_ok = k0 + r < K;
        const int e = d + r * (int)ldb + col;   // element index from the descriptor base
        const int odd = e & 1;
        const int e0 = e - odd;                 // first element of the dword window
        br.sh[j] = odd ? 16u : 0u;
        if (row_ok && nv >= 8) {
            br.w[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, 2 * e0, 0, 0);
            br.x[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, odd ? 2 * (e0 + 8) : (int)kOutOfRange,
                                                          0, 0);
        } else {
            // cut by the N edge (or past it / past K): only the dwords that
            // hold an element of the chunk, the others read as zero
            const int last = e + (int)(nv < 8 ? nv : 8) - 1;   // last valid element
            const bool any = row_ok && nv > 0;
            uint32_t q[5];
#pragma unroll
            for (int t = 0; t < 5; ++t)
                q[t] = __builtin_amdgcn_raw_buffer_load_b32(
                    rs, (any && e0 + 2 * t <= last) ? 2 * (e0 + 2 * t) : (int)kOutOfRange, 0, 0);
            br.w[j] = u32x4{q[0], q[1], q[2], q[3]};
            br.x[j] = q[4];
        }
    }
}

// Funnel-shifts the landed windows into chunks, zeroes columns past N and
// writes them to the B tile of the LDS stage at stage_b.
template <class T>
__device__ __forceinline__ void ragged_b_store(const BRegs<T> &br, lds_u16 *stage_b, int row0,
                                               int c, int64_t nv)
{
    constexpr int NCH = RaggedPlan<T>::NCH, RSTEP = RaggedPlan<T>::RSTEP;
    // dword q keeps both elements when 2q + 1 < nv, the low one when 2q < nv
    uint32_t m[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
        m[q] = (2 * q + 1 < nv) ? 0xffffffffu : (2 * q < nv) ? 0x0000ffffu : 0u;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const int r = row0 + j * RSTEP;
        const u32x4 w = br.w[j];
        const uint32_t s = br.sh[j];
        u32x4 v;
        v.x = __builtin_amdgcn_alignbit(w.y, w.x, s) & m[0];
        v.y = __builtin_amdgcn_alignbit(w.z, w.y, s) & m[1];
        v.z = __builtin_amdgcn_alignbit(w.w, w.z, s) & m[2];
        v.w = __builtin_amdgcn_alignbit(br.x[j], w.w, s) & m[3];
        *reinterpret_cast<__attribute__((address_space(3))) u32x4 *>(
            stage_b + r * T::BN + swz_b<T::CB, T::SWZ, T::BSWZ>(r, c) * 8) = v;
    }
}

template <class T, int I = 0>
__device__ __forceinline__ void issue_a_tile(const LoadPlan<T> &lp, const i32x4 &ra, bool a_kok,
                                             uint32_t stage_addr, int wave)
{
    if constexpr (I < T::A_LD) {
        issue_one<T, I>(lp, ra, ra, a_kok, 0, stage_addr, wave);
        issue_a_tile<T, I + 1>(lp, ra, a_kok, stage_addr, wave);
    }
}

template <class T>
__global__ void __launch_bounds__(T::NT) __attribute__((amdgpu_waves_per_eu(T::OCC)))
gemm_relu_ragged_kernel(GemmArgs p, int tilesM, int tilesN, int groupM)
{
    static_assert(T::STAGES == 2 && T::KG == 1 && !T::BT && T::BK == 64,
                  "ragged kernel: 2 stages, 64-wide K tiles, (K,N) B");
    using RP = RaggedPlan<T>;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[RP::LDS / 2];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const lds_u16 *lds = (const lds_u16 *)smem;
    const uint32_t lds_base = (uint32_t)(uintptr_t)lds;
    const int wm = wave / T::WN, wn = wave % T::WN;
    int tm, tn;
    tile_coords(blockIdx.x, tilesM, tilesN, groupM, tm, tn);
    const int64_t bidx = blockIdx.y;
    const int64_t M = p.M, N = p.N, K = p.K;
    const int64_t m0 = (int64_t)tm * T::BM, n0 = (int64_t)tn * T::BN;
    const uint16_t *Ab = p.A + bidx * p.sA + m0 * p.lda;
    const uint16_t *Bb = p.B + bidx * p.sB;
    uint16_t *C = p.C + bidx * p.sC;

    // A load plan, as in the aligned kernel
    LoadPlan<T> lp;
    {
        const int r0 = wave * T::A_RPB + lane / T::CA;
        const int c = swz_a<T::CA, T::SWZ>(r0, lane % T::CA);
        lp.a_kcol = c * 8;
#pragma unroll
        for (int i = 0; i < T::A_LD; ++i) {
            const int row = r0 + i * T::NW * T::A_RPB;
            lp.a_voff[i] = (m0 + row < M) ? (uint32_t)((row * p.lda + c * 8) * 2) : kOutOfRange;
        }
    }
    auto rsrc_a = [&](int t) { return make_rsrc(Ab + (int64_t)t * T::BK); };
    auto a_kok = [&](int t) { return (int64_t)t * T::BK + lp.a_kcol < K; };
    // B chunk plan: chunk column c, tile rows row0, row0 + RSTEP, ...
    const int bc = tid % T::CB;
    const int brow0 = tid / T::CB;
    const int64_t bnv = N - (n0 + bc * 8);
    BRegs<T> br;
    auto b_load = [&](int t) {
        ragged_b_load<T>(br, Bb, (int64_t)t * T::BK, K, p.ldb, n0, brow0, bc * 8, bnv);
    };
    auto b_store = [&](int t) {
        ragged_b_store<T>(br, (lds_u16 *)smem + (t & 1) * T::STAGE + T::A_ELEMS, brow0, bc, bnv);
    };

    typename T::Acc acc[T::FM][T::FN];
#pragma unroll
    for (int fm = 0; fm < T::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < T::FN; ++fn)
            acc[fm][fn] = typename T::Acc{};

    const int KT = (int)((K + T::BK - 1) / T::BK);
    f16x8 af[2][T::FM], bf[2][T::FN];
    // prologue: tile 0 in stage 0, tile 1's A loads and B registers in flight
    b_load(0);
    issue_a_tile<T>(lp, rsrc_a(0), a_kok(0), lds_base, wave);
    wait_vmcnt<0>();
    b_store(0);
    b_load(1);
    issue_a_tile<T>(lp, rsrc_a(1), a_kok(1), lds_base + (uint32_t)(T::STAGE * 2), wave);
    block_barrier();
    {
        s16x4 bh[T::FN][2];
        read_all<T>(lds, lds + T::A_ELEMS, 0, wm, wn, lane, af[0], bh);
        join_b<T>(bh, bf[0]);
    }

    for (int kt = 0; kt < KT; ++kt) {
        const int stage = kt & 1;
        const lds_u16 *As = lds + stage * T::STAGE;
        const lds_u16 *Bs = As + T::A_ELEMS;
        // the first half of the tile's k steps (one of two, or two of four)
        {
            s16x4 bh[T::FN][2];
            step<T, 0, 0>(acc, af[0], bf[0], lp, i32x4{}, i32x4{}, false, 0, 0u, wave, As, Bs, 1,
                          wm, wn, lane, af[1], bh);
            join_b<T>(bh, bf[1]);
        }
        if constexpr (T::KSTEPS == 4) {
            s16x4 bh[T::FN][2];
            step<T, 0, 0>(acc, af[1], bf[1], lp, i32x4{}, i32x4{}, false, 0, 0u, wave, As, Bs, 2,
                          wm, wn, lane, af[0], bh);
            join_b<T>(bh, bf[0]);
        }
        // Tile kt+1's B registers (issued at this point of tile kt-1) have
        // landed: write them to the other stage, free since the barrier that
        // ended tile kt-1, and reload the registers with tile kt+2.  The
        // scheduling barriers keep the funnel shifts that consume the loads
        // here; hoisted to the top of the tile, they would make the wave wait
        // for the loads two k steps after issuing them.
        wait_vmcnt<0>();
        __builtin_amdgcn_sched_barrier(0);
        b_store(kt + 1);
        b_load(kt + 2);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (T::KSTEPS == 4)
            inner_steps<T, 2>(acc, af, bf, lp, i32x4{}, i32x4{}, false, 0, 0u, wave, As, Bs, wm, wn,
                              lane);
        constexpr int cur = (T::KSTEPS - 1) & 1, nxt = T::KSTEPS & 1;
        block_barrier();
        {
            // last k step of tile kt, with tile kt+2's A loads into the stage
            // just released and the first fragment reads of tile kt+1
            const lds_u16 *An = lds + (stage ^ 1) * T::STAGE;
            const uint32_t laddr = lds_base + (uint32_t)(stage * T::STAGE * 2);
            s16x4 bh[T::FN][2];
            step<T, 0, T::A_LD>(acc, af[cur], bf[cur], lp, rsrc_a(kt + 2), i32x4{}, a_kok(kt + 2), 0,
                                laddr, wave, An, An + T::A_ELEMS, 0, wm, wn, lane, af[nxt], bh);
            join_b<T>(bh, bf[nxt]);
        }
    }
    // loads issued past the end of K must land before the LDS is reused
    wait_vmcnt<0>();

    // Epilogue: bias, ReLU, rounding; the tile staged with row r shifted by
    // the parity of its first element's address.
    block_barrier();
    lds_u16 *cst = (lds_u16 *)smem;
    const int cpar = (int)((reinterpret_cast<uintptr_t>(C) >> 1) & 1);
    const bool relu = p.relu != 0;
    constexpr int NG = T::MI == 32 ? 4 : 1;   // column groups per fragment, as in the aligned kernel
    auto stage_c = [&](auto fast_c) __attribute__((always_inline)) {
        constexpr bool FAST = decltype(fast_c)::value;
#pragma unroll
        for (int fn = 0; fn < T::FN; ++fn) {
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const int col = wn * T::TN + fn * T::MI +
                                (T::MI == 32 ? 8 * g + 4 * (lane >> 5) : 4 * (lane >> 4));
                float bv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                if (!FAST && p.bias != nullptr) {
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        if (n0 + col + t < N)
                            bv[t] = bits_to_float<T::BF16>(p.bias[n0 + col + t]);
                }
#pragma unroll
                for (int fm = 0; fm < T::FM; ++fm) {
                    const int row = wm * T::TM + fm * T::MI + (lane & (T::MI - 1));
                    const int odd = (cpar + (int)(((m0 + row) * p.ldc + n0) & 1)) & 1;
                    const u32x2 w = finish4<T, FAST>(acc[fm][fn], g, bv, relu);
                    lds_u16 *dst = cst + row * RP::CLD + col;
                    if (!odd) {
                        *reinterpret_cast<__attribute__((address_space(3))) u32x2 *>(dst) = w;
                    } else {
                        dst[1] = (uint16_t)(w.x & 0xffff);
                        *reinterpret_cast<__attribute__((address_space(3))) uint32_t *>(dst + 2) =
                            (w.x >> 16) | (w.y << 16);
                        dst[4] = (uint16_t)(w.y >> 16);
                    }
                }
            }
        }
    };
    if (p.bias == nullptr && relu)
        stage_c(std::true_type{});
    else
        stage_c(std::false_type{});
    block_barrier();
    const int64_t nrow = (N - n0) < T::BN ? (N - n0) : T::BN;
    for (int q = tid; q < T::BM * RP::CCH; q += T::NT) {
        const int row = q / RP::CCH, ch = q % RP::CCH;
        const int64_t gm = m0 + row;
        if (gm >= M)
            continue;
        uint16_t *g = C + gm * p.ldc + n0;
        const int odd = (cpar + (int)((gm * p.ldc + n0) & 1)) & 1;
        const int j0 = 8 * ch - odd;   // row element held by the chunk's first slot
        const lds_u16 *src = cst + row * RP::CLD + 8 * ch;
        if (j0 >= 0 && j0 + 8 <= nrow) {
            __builtin_nontemporal_store(
                *reinterpret_cast<const __attribute__((address_space(3))) u32x4 *>(src),
                reinterpret_cast<u32x4_a4 *>(g + j0));
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (j0 + i >= 0 && j0 + i < nrow)
                    g[j0 + i] = src[i];
        }
    }
}

template <class T>
hipError_t launch_ragged(const GemmArgs &p, hipStream_t stream, int groupM)
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
        hipLaunchKernelGGL((gemm_relu_ragged_kernel<T>), dim3((unsigned)tiles, (unsigned)nb),
                           dim3(T::NT), 0, stream, q, (int)tilesM, (int)tilesN, groupM);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

hipError_t launch_all_configs(int cfg, const GemmArgs &p, hipStream_t stream, int groupM)
{
    switch (cfg) {
    case 0: return launch_dma<Mode<Cfg<256, 256, 32, 2, 2, 4>, 0>>(p, stream, groupM);
    case 1: return launch_dma<Mode<Cfg<256, 256, 32, 2, 2, 3>, 0>>(p, stream, groupM);
    case 2: return launch_dma<Mode<Cfg<256, 256, 64, 2, 2, 2>, 0>>(p, stream, groupM);
    case 3: return launch_dma<Mode<Cfg<128, 128, 64, 2, 2, 4>, 0>>(p, stream, groupM);
    case 4: return launch_dma<Mode<Cfg<128, 128, 32, 2, 2, 4>, 0>>(p, stream, groupM);
    case 5: return launch_dma<Mode<Cfg<128, 128, 64, 2, 2, 3>, 0>>(p, stream, groupM);
    case 6: return launch_dma<Mode<Cfg<256, 128, 64, 2, 2, 3>, 0>>(p, stream, groupM);
    // eight waves: two per SIMD, 128x64 or 64x128 wave tiles
    case 7: return launch_dma<Mode<Cfg<256, 256, 32, 2, 4, 4>, 0>>(p, stream, groupM);
    case 8: return launch_dma<Mode<Cfg<256, 256, 64, 2, 4, 2>, 0>>(p, stream, groupM);
    case 9: return launch_dma<Mode<Cfg<256, 256, 32, 4, 2, 4>, 0>>(p, stream, groupM);
    // small LDS footprint: several workgroups per CU for short K
    case 10: return launch_dma<Mode<Cfg<128, 128, 32, 2, 2, 2>, 0>>(p, stream, groupM);
    case 11: return launch_dma<Mode<Cfg<128, 128, 64, 2, 2, 2>, 0>>(p, stream, groupM);
    case 12: return launch_dma<Mode<Cfg<128, 128, 32, 2, 2, 2, 4>, 0>>(p, stream, groupM);
    case 13: return launch_dma<Mode<Cfg<128, 128, 64, 2, 2, 2, 2>, 0>>(p, stream, groupM);
    // two K groups of four waves (two waves per SIMD on alternate K tiles)
    case 14: return launch_dma<Mode<Cfg<128, 128, 64, 2, 2, 2, 2, 2>, 0>>(p, stream, groupM);
    case 15: return launch_dma<Mode<Cfg<128, 128, 32, 2, 2, 4, 2, 2>, 0>>(p, stream, groupM);
    case 16: return launch_dma<Mode<Cfg<128, 128, 32, 2, 2, 3, 2, 2>, 0>>(p, stream, groupM);
    // deep rings for latency-bound mid-size shapes
    case 17: return launch_dma<Mode<Cfg<128, 128, 32, 2, 2, 8>, 0>>(p, stream, groupM);
    case 18: return launch_dma<Mode<Cfg<128, 128, 64, 2, 2, 5>, 0>>(p, stream, groupM);
    // 64x64 tiles for problems with few 128x128 tiles
    case 19: return launch_dma<Mode<Cfg<64, 64, 64, 2, 2, 4>, 0>>(p, stream, groupM);
    case 20: return launch_dma<Mode<Cfg<64, 64, 64, 2, 2, 4, 1, 2>, 0>>(p, stream, groupM);
    // the tile the pages start from: 128 x 128 x 32, 3 stages, 4 waves
    case 21: return launch_dma<Mode<Cfg<128, 128, 32, 2, 2, 3>, 0>>(p, stream, groupM);
    // ablations of the large-shape tile: operand tiles without the XOR
    // swizzle, and a 2-stage ring
    case 22: return launch_dma<Mode<Cfg<256, 256, 32, 2, 2, 4, 1, 1, false>, 0>>(p, stream, groupM);
    case 23: return launch_dma<Mode<Cfg<256, 256, 32, 2, 2, 2>, 0>>(p, stream, groupM);
    // more eight-wave large tiles
    case 24: return launch_dma<Mode<Cfg<256, 256, 64, 4, 2, 2>, 0>>(p, stream, groupM);
    case 25: return launch_dma<Mode<Cfg<256, 256, 32, 2, 4, 3>, 0>>(p, stream, groupM);
    // sixteen waves, 64x64 wave tiles
    case 26: return launch_dma<Mode<Cfg<256, 256, 64, 4, 4, 2>, 0>>(p, stream, groupM);
    case 27: return launch_dma<Mode<Cfg<256, 256, 32, 4, 4, 4>, 0>>(p, stream, groupM);
    // eight-wave 128x128 tiles
    case 28: return launch_dma<Mode<Cfg<128, 128, 64, 2, 4, 4>, 0>>(p, stream, groupM);
    case 29: return launch_dma<Mode<Cfg<128, 128, 64, 4, 2, 4>, 0>>(p, stream, groupM);
    // two workgroups per CU (64 KiB of LDS each): the two waves sharing a SIMD
    // belong to different workgroups and meet different barriers
    case 30: return launch_dma<Mode<Cfg<256, 128, 32, 2, 2, 2, 2>, 0>>(p, stream, groupM);
    case 31: return launch_dma<Mode<Cfg<128, 256, 32, 2, 2, 2, 2>, 0>>(p, stream, groupM);
    // 16x16x32 products (32-wide k steps): configurations 8, 2 and 29 again
    case 32: return launch_dma<Mode<Cfg<256, 256, 64, 2, 4, 2, 1, 1, true, 16>, 0>>(p, stream, groupM);
    case 33: return launch_dma<Mode<Cfg<256, 256, 64, 2, 2, 2, 1, 1, true, 16>, 0>>(p, stream, groupM);
    case 34: return launch_dma<Mode<Cfg<128, 128, 64, 4, 2, 4, 1, 1, true, 16>, 0>>(p, stream, groupM);
    // persistent workgroups walking a list of tiles (many short problems)
    case 35: return launch_stream<Mode<Cfg<128, 128, 64, 4, 2, 3, 1, 1, true, 16>, 0>>(p, stream);
    case 36: return launch_stream<Mode<Cfg<128, 128, 64, 4, 2, 4, 1, 1, true, 16>, 0>>(p, stream);
    case 37: return launch_stream<Mode<Cfg<128, 128, 64, 2, 2, 3, 1, 1, true, 16>, 0>>(p, stream);
    // 64x32 wave tiles (a 2x4 wave grid): each wave's B fragments, read by
    // transpose, serve four A fragments, so a k step needs fewer LDS bytes
    case 38: return launch_dma<Mode<Cfg<128, 128, 64, 2, 4, 4, 1, 1, true, 16>, 0>>(p, stream, groupM);
    // persistent, two workgroups of four waves per CU (80 KiB of LDS each:
    // a 3-stage ring of 32-wide K tiles and the waves' C areas)
    case 39: return launch_stream<Mode<Cfg<128, 128, 32, 2, 2, 3, 2>, 0>>(p, stream);
    // 256x128 tiles of eight waves (one round where 128x128 tiles take two):
    // 64x64 or 128x32 wave tiles with 16x16x32 products, 64x64 with 32x32x16
    case 40: return launch_dma<Mode<Cfg<256, 128, 64, 4, 2, 3, 1, 1, true, 16>, 0>>(p, stream, groupM);
    case 41: return launch_dma<Mode<Cfg<256, 128, 64, 2, 4, 3, 1, 1, true, 16>, 0>>(p, stream, groupM);
    case 42: return launch_dma<Mode<Cfg<256, 128, 64, 4, 2, 2>, 0>>(p, stream, groupM);
    default: return hipErrorInvalidValue;
    }
}


// bf16 and (N,K)-B instances exist for the configurations the dispatcher
// picks by default: 256x256 (32), 128x128 (38), 256x128 (41), short K (39, and
// 36 for very many tiles) and few tiles (20), for the one-tile-per-workgroup short-K tile
// (12), the 4x2 wave grid of 128x128 (34) and the 32x32x16 forms of 32 and 34
// (8, 29).
template <int MODE>
hipError_t launch_default_configs(int cfg, const GemmArgs &p, hipStream_t stream, int groupM)
{
    switch (cfg) {
    case 32: return launch_dma<Mode<Cfg<256, 256, 64, 2, 4, 2, 1, 1, true, 16>, MODE>>(p, stream, groupM);
    case 34: return launch_dma<Mode<Cfg<128, 128, 64, 4, 2, 4, 1, 1, true, 16>, MODE>>(p, stream, groupM);
    case 38: return launch_dma<Mode<Cfg<128, 128, 64, 2, 4, 4, 1, 1, true, 16>, MODE>>(p, stream, groupM);
    case 8: return launch_dma<Mode<Cfg<256, 256, 64, 2, 4, 2>, MODE>>(p, stream, groupM);
    case 29: return launch_dma<Mode<Cfg<128, 128, 64, 4, 2, 4>, MODE>>(p, stream, groupM);
    case 12: return launch_dma<Mode<Cfg<128, 128, 32, 2, 2, 2, 4>, MODE>>(p, stream, groupM);
    case 20: return launch_dma<Mode<Cfg<64, 64, 64, 2, 2, 4, 1, 2>, MODE>>(p, stream, groupM);
    case 36: return launch_stream<Mode<Cfg<128, 128, 64, 4, 2, 4, 1, 1, true, 16>, MODE>>(p, stream);
    case 39: return launch_stream<Mode<Cfg<128, 128, 32, 2, 2, 3, 2>, MODE>>(p, stream);
    case 41: return launch_dma<Mode<Cfg<256, 128, 64, 2, 4, 3, 1, 1, true, 16>, MODE>>(p, stream, groupM);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool dma_layout_ok(const GemmArgs &p)
{
    // 32-bit buffer offsets: a 256-row A panel and a 64-row B tile must stay
    // below 2^31 bytes from their descriptors
    return p.lda <= (1 << 21) && p.ldb <= (1 << 21);
}

bool dma_config_has_mode(int cfg, int mode)
{
    return mode == 0 ? (cfg >= 0 && cfg < kDmaConfigs)
                     : (cfg == 32 || cfg == 34 || cfg == 8 || cfg == 29 || cfg == 12 || cfg == 20 ||
                        cfg == 36 || cfg == 38 || cfg == 39 || cfg == 41);
}

hipError_t launch_ragged_config(int cfg, const GemmArgs &p, hipStream_t stream, int groupM)
{
    if (p.b_nk)
        return hipErrorInvalidValue;
    const bool bf = p.bf16 != 0;
    switch (cfg) {
    case 0:   // 256 x 256 x 64, 8 waves of 128 x 64 (the large-shape geometry)
        return bf ? launch_ragged<Mode<Cfg<256, 256, 64, 2, 4, 2>, 1>>(p, stream, groupM)
                  : launch_ragged<Mode<Cfg<256, 256, 64, 2, 4, 2>, 0>>(p, stream, groupM);
    case 1:   // 128 x 128 x 64, 8 waves of 32 x 64
        return bf ? launch_ragged<Mode<Cfg<128, 128, 64, 4, 2, 2>, 1>>(p, stream, groupM)
                  : launch_ragged<Mode<Cfg<128, 128, 64, 4, 2, 2>, 0>>(p, stream, groupM);
    case 2:   // 0 with 16x16x32 products
        return bf ? launch_ragged<Mode<Cfg<256, 256, 64, 2, 4, 2, 1, 1, true, 16>, 1>>(p, stream, groupM)
                  : launch_ragged<Mode<Cfg<256, 256, 64, 2, 4, 2, 1, 1, true, 16>, 0>>(p, stream, groupM);
    case 3:   // 1 with 16x16x32 products
        return bf ? launch_ragged<Mode<Cfg<128, 128, 64, 4, 2, 2, 1, 1, true, 16>, 1>>(p, stream, groupM)
                  : launch_ragged<Mode<Cfg<128, 128, 64, 4, 2, 2, 1, 1, true, 16>, 0>>(p, stream, groupM);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_dma_config(int cfg, const GemmArgs &p, hipStream_t stream, int groupM)
{
    switch ((p.bf16 ? 1 : 0) | (p.b_nk ? 2 : 0)) {
    case 0: return launch_all_configs(cfg, p, stream, groupM);
    case 1: return launch_default_configs<1>(cfg, p, stream, groupM);
    case 2: return launch_default_configs<2>(cfg, p, stream, groupM);
    default: return launch_default_configs<3>(cfg, p, stream, groupM);
    }
}

}  // namespace tg
