// Weight-only int4 GEMM (W_INT4 / A_FP16, and A_BF16) on gfx950: the
// dequantize GEMM that section 5 of the "TileLang paper reading" page
// (hotelren.com) measures, with the GEMM+ReLU epilogue of its section 2:
//
//   C[i][n] = store(act(sum_k A[i][k] * s[n][k/G] * q[n][k] + bias[n]))
//
// q: signed 4-bit weights, (N,K) with two per byte along k (even k in the
// low nibble), row n at Wq + n*ldw bytes; s: one scale per group of G k per
// row, row n at S + n*lds elements.
//
// Decode-shaped problems (a few rows of A against a large weight) are bound
// by streaming the weight from HBM once; int4 weights are a quarter of the
// bytes of fp16 ones.  Design:
//  * One workgroup per 64 weight rows (64 output columns) and per 16*MB rows
//    of A, made of KG groups of four waves; wave w of a group owns weight
//    rows 16w .. 16w+15.  The K loop takes 256 k per step: a 64 x 128-byte
//    weight block and the 16*MB x 512-byte A block, both staged by
//    buffer_load_dwordx4 ... lds into an S-stage ring per group (one
//    workgroup barrier per step); group g takes steps g, g + KG, ..., and the
//    groups' sums are added in group order at the end.  Two groups put two
//    waves on each SIMD, so one wave's LDS reads and dequantization overlap
//    the other's.
//  * The matrix cores run v_mfma_f32_16x16x32_{f16,bf16} with the weight as
//    the first operand (C^T = W A^T, so a lane owns four consecutive output
//    columns of one row).  A lane's weight fragment is one 4-byte LDS read:
//    eight nibbles, turned into eight exact fp16 / bf16 integers -8..7 in
//    registers (fp16: the bit pattern 0x6400 | (q + 8) is 1024 + q + 8, less
//    1032; bf16: the fp32 pattern 0x4b000000 | (q + 8) is 2^23 + q + 8, less
//    2^23 + 8, then packed).
//  * Products of A with q are exact, and the sums of one group of k run in
//    fp32 on the matrix cores; at the end of each group the lane multiplies
//    its four partial sums by their rows' scales and adds them to the
//    accumulator.  The scales of the workgroup's 64 rows are copied to LDS
//    once, while the first weight steps are in flight.
//  * The kernel is bound by instruction issue on its two waves per SIMD, not
//    by HBM.  When G divides the 256-k step (G = 32, 64, 128, 256: the
//    common formats) the group structure is a template parameter and the
//    step loop is unrolled over the rings' period, so LDS addresses are
//    loop-invariant registers (no address arithmetic per read) and a
//    group's first product starts from a zero accumulator; other G keep a
//    run-time group counter.
//  * Weight chunks past N, A rows past M and k past K read as zeros through
//    the buffer descriptors' range check (a zero byte is two zero weights);
//    when K is a multiple of 256 a step is wholly in or out of K and the
//    check is the descriptor's record count alone.
//  * Workgroups start their K walk at different steps (see `rot`).
// Requirements (checked by the dispatcher): A 16-byte aligned, lda % 8 == 0;
// Wq 16-byte aligned, ldw % 16 == 0; K % G == 0 with G a multiple of 32;
// C 8-byte aligned, ldc and N multiples of 4; bias (if any) 8-byte aligned;
// the scales of 64 rows fit in the LDS left over by the ring.
#include "tg_internal.h"

#include <utility>

namespace tg {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) f16x8 lds_f16x8;
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kRows = 64;     // weight rows per workgroup
constexpr int kKS = 256;      // k per step
constexpr int kLds = 160 * 1024;

// The weight (from HBM) and A (small, L2-resident) have separate rings per K
// group: SW weight stages (loads SW-1 steps ahead) and SA A stages (SA-1
// steps ahead, SA <= SW), so the LDS goes to keeping more weight in flight.
template <int MB_, int SW_, int SA_, bool BF16_, int KG_ = 1, int GS_ = 0>
struct W4Cfg {
    static constexpr int MB = MB_;                   // 16-row blocks of A
    static constexpr int SW = SW_, SA = SA_;         // ring stages per K group
    // GS > 0: a scale group is GS 32-k substeps (G = 32 GS divides the 256-k
    // step), fixed at compile time; 0: any G, tracked at run time
    static constexpr int GS = GS_;
    static constexpr int P = SW % SA == 0 ? SW : SW * SA;   // steps after which both rings repeat
    static constexpr int DW = SW - 1, DA = SA - 1;   // steps of look-ahead
    static constexpr bool BF16 = BF16_;
    static constexpr int KG = KG_;                   // K groups of four waves
    static constexpr int NT = 256 * KG;
    static constexpr int A_BYTES = MB * 16 * kKS * 2;   // 512-byte rows
    static constexpr int W_BYTES = kRows * kKS / 2;     // 128-byte rows
    static constexpr int A_LD = A_BYTES / 1024 / 4;     // 1 KiB blocks per wave
    static constexpr int W_LD = W_BYTES / 1024 / 4;
    static constexpr int W_RING = SW * W_BYTES, A_RING = SA * A_BYTES;   // per group
    static constexpr int GROUP = W_RING + A_RING;
    static constexpr int RING = KG * GROUP;          // all groups' rings
    static constexpr int RED = (KG - 1) * 4 * MB * 64 * 16;   // partial sums of groups > 0
    // loads of this wave issued after step st's A loads when step st is
    // needed: the weight loads of that same step, then DA-1 whole steps
    static constexpr int WAIT = DA * W_LD + (DA - 1) * A_LD;
    static_assert(SA >= 2 && SW > SA, "ring depths: the weight looks further ahead than A");
    static_assert(RED <= RING, "reduction space");
    static_assert((A_BYTES / 1024) % 4 == 0 && (W_BYTES / 1024) % 4 == 0, "blocks per wave");
    static_assert(DW * W_LD + DA * A_LD <= 63, "vmcnt range");
};

// Configurations by A rows: two K groups of four waves (two waves per SIMD:
// one group's dequantization and LDS reads overlap the other's) where the
// rings fit, depths chosen so the rings plus the scales of K/G <= 64..128
// groups fit the 160 KiB of LDS.  The single-group forms serve group sizes
// that do not divide 256.
template <int MB, bool BF16, int GS>
using W4Two = W4Cfg<MB, MB == 1 ? 6 : MB == 2 ? 5 : 3, MB == 1 ? 3 : 2, BF16, 2, GS>;
template <int MB, bool BF16>
using W4One = W4Cfg<MB, MB <= 2 ? 8 : 6, MB == 1 ? 4 : 3, BF16, 1>;

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N <= 63, "vmcnt");
    constexpr int imm = (N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(imm);
    asm volatile("" ::: "memory");
}

// Barrier once this wave's LDS reads have completed.
__device__ __forceinline__ void block_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((3 << 14) | (0 << 8) | (7 << 4) | 15);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ i32x4 make_rsrc(const void *base)
{
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
    r.z = (int)kOutOfRange;
    r.w = 0x00020000;
    return r;
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes per lane from rsrc + voff into the 1 KiB LDS block at lds_addr.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voff, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %2\n\t"
                 "s_nop 0\n\t"
                 "buffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(lds_addr)
                 : "m0");
}

// The same with the non-temporal hint (the weight is streamed once).
__device__ __forceinline__ void dma16_nt(i32x4 rsrc, uint32_t voff, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %2\n\t"
                 "s_nop 0\n\t"
                 "buffer_load_dwordx4 %0, %1, 0 offen nt lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(lds_addr)
                 : "m0");
}
#pragma clang diagnostic pop

// Physical 16-byte chunk of logical chunk c in a 512-byte A row (16 lanes
// read one chunk of 16 consecutive rows) and in a 128-byte weight row (two
// rows share a 256-byte bank line).
__device__ __forceinline__ int swz_a(int row, int c) { return c ^ (row & 15); }
__device__ __forceinline__ int swz_w(int row, int c) { return c ^ ((row >> 1) & 7); }

// Eight signed nibbles (k ascending from the low nibble of the low byte) as
// eight exact fp16 or bf16 values, packed as the matrix-core operand.  With
// u = w ^ 0x88888888 each nibble holds q + 8 in 0..15.  fp16: a byte permute
// copies byte i of u into both halves of a dword, one AND-OR keeps the low
// nibble in the low half and the high nibble (as 16 * (q + 8)) in the high
// half under the exponent bits 0x64, giving the halves 1024 + (q + 8) and
// 1024 + 16 (q + 8); one packed FMA (times 1 and 1/16, less 1032 and 72)
// leaves both q exactly.  bf16: a byte permute places each nibble of the
// masked halves under the fp32 exponent of 2^23, one subtraction leaves q,
// one conversion packs two bf16 (all exact).
// `nib` holds 0x00f0000f in a register: with the mask in a VGPR the AND and
// the OR with the exponent bits fuse into one v_and_or_b32 (a VOP3
// instruction takes no literal here, and two literals would cost two
// instructions).
template <bool BF16>
__device__ __forceinline__ f16x8 dequant8(uint32_t w, uint32_t nib)
{
    const uint32_t u = w ^ 0x88888888u;
    u32x4 out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (!BF16) {
            typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
            const uint32_t sel = 0x0c000c00u | ((uint32_t)i << 16) | (uint32_t)i;
            const uint32_t v = (__builtin_amdgcn_perm(u, u, sel) & nib) | 0x64006400u;
            const f16x2 h = __builtin_elementwise_fma(
                __builtin_bit_cast(f16x2, v), f16x2{(_Float16)1.0f, (_Float16)0.0625f},
                f16x2{(_Float16)-1032.0f, (_Float16)-72.0f});
            out[i] = __builtin_bit_cast(uint32_t, h);
        } else {
            typedef float f32x2 __attribute__((ext_vector_type(2)));
            typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
            const uint32_t y = u & 0x0f0f0f0fu;             // even k: q + 8 per byte
            const uint32_t z = (u >> 4) & 0x0f0f0f0fu;      // odd k
            // byte i under the fp32 exponent of 2^23: 2^23 + q + 8, then
            // less 2^23 + 8 (exact), and both converted in one instruction
            // (exact: small integers)
            const uint32_t sel = 0x070c0c00u | (uint32_t)i;
            const float lo = __builtin_bit_cast(float, __builtin_amdgcn_perm(0x4b000000u, y, sel)) -
                             8388616.0f;
            const float hi = __builtin_bit_cast(float, __builtin_amdgcn_perm(0x4b000000u, z, sel)) -
                             8388616.0f;
            out[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
        }
    }
    return __builtin_bit_cast(f16x8, out);
}

// f(integral_constant<int, I>) for each I of the sequence, in order.
template <class F, int... I>
__device__ __forceinline__ void for_each_index(F &&f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}

template <class T>
__global__ void __launch_bounds__(T::NT) gemm_w4_kernel(W4Args p)
{
    // ring, then the scales of the 64 rows as [group][row]
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kLds];
    const lds_u8 *lds = (const lds_u8 *)smem;
    const uint32_t lds_base = (uint32_t)(uintptr_t)lds;
    lds_u16 *scl = (lds_u16 *)(smem + T::RING);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
    // K group kg takes steps kg, kg + KG, ... with its own ring; `wave` is the
    // wave's index inside its group
    const int kg = wave_all / 4, wave = wave_all % 4;
    const uint32_t wring = lds_base + (uint32_t)(kg * T::GROUP);     // this group's rings
    const uint32_t aring = wring + (uint32_t)T::W_RING;
    const int64_t M = p.M, N = p.N, K = p.K;
    const int64_t n0 = (int64_t)blockIdx.x * kRows;
    const int64_t m0 = (int64_t)blockIdx.y * (16 * T::MB);
    const int groups = (int)(K / p.G);

    // Load plan: A block j (2 rows of 512 bytes): lane L -> row 2j + L / 32,
    // physical chunk L % 32; weight block j (8 rows of 128 bytes): lane L ->
    // row 8j + L / 8, physical chunk L % 8.  Wave w moves blocks w, w + 4, ..
    uint32_t a_voff[T::A_LD];
    int a_col[T::A_LD];
#pragma unroll
    for (int i = 0; i < T::A_LD; ++i) {
        const int row = 2 * (wave + 4 * i) + lane / 32;
        const int c = swz_a(row, lane % 32);
        a_col[i] = c * 8;
        a_voff[i] = (m0 + row < M) ? (uint32_t)((row * p.lda + c * 8) * 2) : kOutOfRange;
    }
    uint32_t w_voff[T::W_LD];
    int w_col[T::W_LD];
#pragma unroll
    for (int i = 0; i < T::W_LD; ++i) {
        const int row = 8 * (wave + 4 * i) + lane / 8;
        const int c = swz_w(row, lane % 8);
        w_col[i] = c * 32;                    // first k of the chunk
        w_voff[i] = (n0 + row < N) ? (uint32_t)(row * p.ldw + c * 16) : kOutOfRange;
    }
    const uint16_t *Ab = p.A + m0 * p.lda;
    const uint8_t *Wb = p.Wq + n0 * p.ldw;
    const int steps = (int)((K + kKS - 1) / kKS);

    // Every workgroup reads the same A; walking K from a workgroup-dependent
    // step spreads their A reads over different k (and so different L2
    // channels) instead of all hitting the same lines at once.  Only when no
    // scale group spans two steps (G divides 256), so that each group's sum
    // is still formed from consecutive pieces.
    const int rot = (kKS % p.G == 0 && steps > 0) ? (int)(blockIdx.x % (unsigned)steps) : 0;
    auto step_of = [&](int gs) { return gs + rot < steps ? gs + rot : gs + rot - steps; };
    // every group runs the same number of steps (a group past the end of K
    // loads zeros) so that the workgroup barriers line up
    const int gsteps = (steps + T::KG - 1) / T::KG;

    // k of this group's st-th step; steps past the last read nothing
    auto k_of = [&](int st) {
        const int gs = st * T::KG + kg;
        return (int64_t)(gs < steps ? step_of(gs) : gs) * kKS;
    };
    // When K is a multiple of the step, a step is either wholly inside K or
    // wholly past it: the descriptor's record count (0 past the end) makes
    // the range check, with no per-lane compare.
    const bool kfull = K % kKS == 0;
    auto issue_a = [&](int st) {
        const int64_t k0 = k_of(st);
        i32x4 ra = make_rsrc(Ab + k0);
        const uint32_t base = aring + (uint32_t)((st % T::SA) * T::A_BYTES);
        if (kfull) {
            ra.z = k0 < K ? (int)kOutOfRange : 0;
#pragma unroll
            for (int i = 0; i < T::A_LD; ++i)
                dma16(ra, a_voff[i], base + (uint32_t)((wave + 4 * i) * 1024));
            return;
        }
#pragma unroll
        for (int i = 0; i < T::A_LD; ++i)
            dma16(ra, k0 + a_col[i] < K ? a_voff[i] : kOutOfRange,
                  base + (uint32_t)((wave + 4 * i) * 1024));
    };
    auto issue_w = [&](int st) {
        const int64_t k0 = k_of(st);
        i32x4 rw = make_rsrc(Wb + k0 / 2);
        const uint32_t base = wring + (uint32_t)((st % T::SW) * T::W_BYTES);
        if (kfull) {
            rw.z = k0 < K ? (int)kOutOfRange : 0;
#pragma unroll
            for (int i = 0; i < T::W_LD; ++i)
                dma16_nt(rw, w_voff[i], base + (uint32_t)((wave + 4 * i) * 1024));
            return;
        }
#pragma unroll
        for (int i = 0; i < T::W_LD; ++i)
            dma16_nt(rw, k0 + w_col[i] < K ? w_voff[i] : kOutOfRange,
                     base + (uint32_t)((wave + 4 * i) * 1024));
    };

    // acc: the scaled sum so far; part: the current group's sum (a group may
    // span steps when G does not divide 256)
    f32x4 acc[T::MB], part[T::MB];
#pragma unroll
    for (int mb = 0; mb < T::MB; ++mb)
        acc[mb] = part[mb] = f32x4{};
    uint32_t nib = 0x00f0000fu;                      // see dequant8
    asm volatile("" : "+v"(nib));
    const int wrow = wave * 16 + (lane & 15);        // the lane's weight row (operand)
    const int orow = wave * 16 + 4 * (lane >> 4);    // the lane's first output column
    const int sub_per_group = p.G / 32;
    int left = sub_per_group;                        // substeps left in the current group
    // groups per step when G divides 256 (every step then starts a group);
    // otherwise (one group of waves, steps in order) the group index simply
    // runs on across steps
    const int gps = (kKS % p.G == 0) ? kKS / p.G : 0;
    int g_cur = 0;
    // the lane's LDS byte offsets inside a stage, per 32-k substep
    uint32_t w_off[kKS / 32], a_off[kKS / 32];
#pragma unroll
    for (int ks = 0; ks < kKS / 32; ++ks) {
        w_off[ks] = (uint32_t)(wrow * 128 + swz_w(wrow, ks) * 16 + (lane >> 4) * 4);
        a_off[ks] = (uint32_t)((lane & 15) * 512 + swz_a(lane & 15, ks * 4 + (lane >> 4)) * 16);
    }

    // Prologue: the weight of steps 0 .. DW-1 and A of steps 0 .. DA-1, in
    // the order the loop issues them (iteration j issues A of step j+DA,
    // then the weight of step j+DW), so that the wait count holds from the
    // first iteration on: weight steps 0 .. DW-DA-1, then (A, weight) pairs.
#pragma unroll
    for (int s = 0; s < T::DW - T::DA; ++s)
        issue_w(s);
#pragma unroll
    for (int s = 0; s < T::DA; ++s) {
        issue_a(s);
        issue_w(s + T::DW - T::DA);
    }
    // Scales of rows n0 .. n0+63, all groups, into LDS as [group][row] (rows
    // past N: 0), loaded while the prologue's weight and A are in flight
    // (the loop's first barrier publishes them).  Threads walk each row's
    // scales in order (coalesced), eight at a time when a row's scales are
    // 16-byte aligned, and every load of a thread is issued before its LDS
    // writes.
    if (p.scales_vec) {
        const int chunks = groups / 8;             // 16-byte chunks per row
        for (int e0 = 0; e0 < chunks * kRows; e0 += 4 * T::NT) {
            u32x4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e = e0 + u * T::NT + tid;
                const int r = e / chunks, c = e % chunks;
                v[u] = u32x4{0, 0, 0, 0};
                if (e < chunks * kRows && n0 + r < N)
                    v[u] = *reinterpret_cast<const u32x4 *>(p.S + (n0 + r) * p.lds + c * 8);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e = e0 + u * T::NT + tid;
                const int r = e / chunks, c = e % chunks;
                if (e < chunks * kRows) {
#pragma unroll
                    for (int t = 0; t < 8; ++t)
                        scl[(c * 8 + t) * kRows + r] = (uint16_t)(v[u][t / 2] >> (16 * (t & 1)));
                }
            }
        }
    } else {
        for (int e0 = 0; e0 < groups * kRows; e0 += 4 * T::NT) {
            uint16_t v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e = e0 + u * T::NT + tid;
                const int r = e / groups, g = e % groups;
                v[u] = (e < groups * kRows && n0 + r < N) ? p.S[(n0 + r) * p.lds + g]
                                                          : (uint16_t)0;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e = e0 + u * T::NT + tid;
                if (e < groups * kRows)
                    scl[(e % groups) * kRows + e / groups] = v[u];
            }
        }
    }

    if constexpr (T::GS > 0) {
        // Fixed group size: the loop is unrolled over the rings' period P so
        // every stage offset is a constant (LDS reads are a per-lane base
        // register plus an immediate), the first product of a group starts
        // from a zero accumulator and the group ends are known.
        uint32_t wb_off[kKS / 32], ab_off[kKS / 32];
#pragma unroll
        for (int ks = 0; ks < kKS / 32; ++ks) {
            wb_off[ks] = (uint32_t)(kg * T::GROUP) + w_off[ks];
            ab_off[ks] = (uint32_t)(kg * T::GROUP + T::W_RING) + a_off[ks];
        }
        const uint8_t *sm = smem;
        constexpr int GPS = 8 / T::GS;                   // groups per step
        auto body = [&](int st, auto u_c) {
            constexpr int u = decltype(u_c)::value;
            wait_vmcnt<T::WAIT>();
            block_barrier();
            issue_a(st + T::DA);
            issue_w(st + T::DW);
            constexpr uint32_t ws = (uint32_t)((u % T::SW) * T::W_BYTES);
            constexpr uint32_t as = (uint32_t)((u % T::SA) * T::A_BYTES);
            const int gs = st * T::KG + kg;
            const int g0 = (gs < steps ? step_of(gs) : gs) * GPS;   // first group of the step
            uint32_t wb[kKS / 32];
#pragma unroll
            for (int ks = 0; ks < kKS / 32; ++ks)
                wb[ks] = *reinterpret_cast<const lds_u32 *>(
                    (const lds_u8 *)sm + (wb_off[ks] + ws));
            f16x8 af[2][T::MB];
#pragma unroll
            for (int mb = 0; mb < T::MB; ++mb)
                af[0][mb] = *reinterpret_cast<const lds_f16x8 *>(
                    (const lds_u8 *)sm + (ab_off[0] + as + mb * 16 * 512));
#pragma unroll
            for (int ks = 0; ks < kKS / 32; ++ks) {
                if (ks + 1 < kKS / 32) {
#pragma unroll
                    for (int mb = 0; mb < T::MB; ++mb)
                        af[(ks + 1) & 1][mb] = *reinterpret_cast<const lds_f16x8 *>(
                            (const lds_u8 *)sm + (ab_off[ks + 1] + as + mb * 16 * 512));
                }
                const f16x8 wf = dequant8<T::BF16>(wb[ks], nib);
                const bool first = ks % T::GS == 0;
#pragma unroll
                for (int mb = 0; mb < T::MB; ++mb) {
                    const f32x4 c = first ? f32x4{} : part[mb];
                    if constexpr (T::BF16)
                        part[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, wf),
                            __builtin_bit_cast(bf16x8, af[ks & 1][mb]), c, 0, 0, 0);
                    else
                        part[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf, af[ks & 1][mb], c, 0,
                                                                          0, 0);
                }
                if (ks % T::GS == T::GS - 1) {
                    const int g = g0 + ks / T::GS;
                    if (g < groups) {
                        const u32x2 sv =
                            *reinterpret_cast<const lds_u32x2 *>(scl + g * kRows + orow);
                        const float s0 = bits_to_float<T::BF16>((uint16_t)(sv.x & 0xffff));
                        const float s1 = bits_to_float<T::BF16>((uint16_t)(sv.x >> 16));
                        const float s2 = bits_to_float<T::BF16>((uint16_t)(sv.y & 0xffff));
                        const float s3 = bits_to_float<T::BF16>((uint16_t)(sv.y >> 16));
#pragma unroll
                        for (int mb = 0; mb < T::MB; ++mb) {
                            acc[mb][0] += s0 * part[mb][0];
                            acc[mb][1] += s1 * part[mb][1];
                            acc[mb][2] += s2 * part[mb][2];
                            acc[mb][3] += s3 * part[mb][3];
                        }
                    }
                }
            }
        };
        for (int st0 = 0; st0 < gsteps; st0 += T::P)
            for_each_index([&](auto u_c) {
                if (st0 + decltype(u_c)::value < gsteps)
                    body(st0 + decltype(u_c)::value, u_c);
            }, std::make_integer_sequence<int, T::P>{});
    } else
    for (int st = 0; st < gsteps; ++st) {
        // this wave's loads of step st have landed once at most WAIT later
        // loads are outstanding (A of step st is the newest of the two); the
        // barrier makes every wave's land and frees the stages of step st-1
        // for A of step st+DA and the weight of step st+DW
        wait_vmcnt<T::WAIT>();
        block_barrier();
        issue_a(st + T::DA);
        issue_w(st + T::DW);
        const lds_u8 *Ws = lds + kg * T::GROUP + (st % T::SW) * T::W_BYTES;
        const lds_u8 *As = lds + kg * T::GROUP + T::W_RING + (st % T::SA) * T::A_BYTES;
        // the lane's weight dwords of the whole step, then A fragments one
        // 32-k substep ahead of the matrix cores
        if (gps != 0) {
            const int gs = st * T::KG + kg;
            g_cur = (gs < steps ? step_of(gs) : gs) * gps;
        }
        uint32_t wb[kKS / 32];
#pragma unroll
        for (int ks = 0; ks < kKS / 32; ++ks)
            wb[ks] = *reinterpret_cast<const lds_u32 *>(Ws + w_off[ks]);
        f16x8 af[2][T::MB];
#pragma unroll
        for (int mb = 0; mb < T::MB; ++mb)
            af[0][mb] = *reinterpret_cast<const lds_f16x8 *>(As + mb * 16 * 512 + a_off[0]);
#pragma unroll
        for (int ks = 0; ks < kKS / 32; ++ks) {
            if (ks + 1 < kKS / 32) {
#pragma unroll
                for (int mb = 0; mb < T::MB; ++mb)
                    af[(ks + 1) & 1][mb] = *reinterpret_cast<const lds_f16x8 *>(
                        As + mb * 16 * 512 + a_off[ks + 1]);
            }
            const f16x8 wf = dequant8<T::BF16>(wb[ks], nib);
#pragma unroll
            for (int mb = 0; mb < T::MB; ++mb) {
                if constexpr (T::BF16)
                    part[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, wf), __builtin_bit_cast(bf16x8, af[ks & 1][mb]),
                        part[mb], 0, 0, 0);
                else
                    part[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf, af[ks & 1][mb],
                                                                      part[mb], 0, 0, 0);
            }
            // end of a group: scale the group's sums by their rows' scales
            if (--left == 0) {
                left = sub_per_group;
                const int g = g_cur++;
                if (g < groups) {
                    const u32x2 sv =
                        *reinterpret_cast<const lds_u32x2 *>(scl + g * kRows + orow);
                    const float s0 = bits_to_float<T::BF16>((uint16_t)(sv.x & 0xffff));
                    const float s1 = bits_to_float<T::BF16>((uint16_t)(sv.x >> 16));
                    const float s2 = bits_to_float<T::BF16>((uint16_t)(sv.y & 0xffff));
                    const float s3 = bits_to_float<T::BF16>((uint16_t)(sv.y >> 16));
#pragma unroll
                    for (int mb = 0; mb < T::MB; ++mb) {
                        acc[mb][0] += s0 * part[mb][0];
                        acc[mb][1] += s1 * part[mb][1];
                        acc[mb][2] += s2 * part[mb][2];
                        acc[mb][3] += s3 * part[mb][3];
                        part[mb] = f32x4{};
                    }
                }
            }
        }
    }
    // loads issued past the end of K must land before the LDS is reused
    wait_vmcnt<0>();
    if constexpr (T::KG > 1) {
        // groups 1 .. KG-1 hand their sums to group 0 through LDS; group 0
        // adds them in group order (deterministic)
        block_barrier();
        typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
        lds_f32x4 *red = (lds_f32x4 *)smem;
        if (kg > 0) {
#pragma unroll
            for (int mb = 0; mb < T::MB; ++mb)
                red[(((kg - 1) * 4 + wave) * T::MB + mb) * 64 + lane] = acc[mb];
        }
        block_barrier();
        if (kg > 0)
            return;
        for (int g2 = 1; g2 < T::KG; ++g2)
#pragma unroll
            for (int mb = 0; mb < T::MB; ++mb)
                acc[mb] += red[(((g2 - 1) * 4 + wave) * T::MB + mb) * 64 + lane];
    }

    // Epilogue: lane owns C[m][n .. n+3], m = m0 + 16 mb + lane % 16.
    const bool relu = p.relu != 0;
    const int64_t n = n0 + orow;
    float bv[4];
    load_bias4<T::BF16>(p.bias, n, N, bv);
#pragma unroll
    for (int mb = 0; mb < T::MB; ++mb) {
        const int64_t m = m0 + mb * 16 + (lane & 15);
        if (m < M && n < N) {
            u32x2 w2;
            w2.x = epi_pack2<T::BF16>(acc[mb][0] + bv[0], acc[mb][1] + bv[1], relu);
            w2.y = epi_pack2<T::BF16>(acc[mb][2] + bv[2], acc[mb][3] + bv[3], relu);
            *reinterpret_cast<u32x2 *>(p.C + m * p.ldc + n) = w2;
        }
    }
}

template <class T>
hipError_t launch_w4(const W4Args &p, hipStream_t stream)
{
    const int64_t gx = (p.N + kRows - 1) / kRows;
    const int64_t gy = (p.M + 16 * T::MB - 1) / (16 * T::MB);
    const size_t lds = (size_t)T::RING + (size_t)(p.K / p.G) * kRows * 2;
    if (gx > 0x7fffffff || gy > 65535 || lds > (size_t)kLds)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_w4_kernel<T>), dim3((unsigned)gx, (unsigned)gy), dim3(T::NT), 0,
                       stream, p);
    return hipGetLastError();
}

// Two K groups with the group size fixed at compile time (G = 32 GS).
template <int GS, bool BF16>
hipError_t launch_two(int64_t mb, const W4Args &p, hipStream_t stream)
{
    if (mb <= 1) return launch_w4<W4Two<1, BF16, GS>>(p, stream);
    if (mb <= 2) return launch_w4<W4Two<2, BF16, GS>>(p, stream);
    return launch_w4<W4Two<3, BF16, GS>>(p, stream);
}

template <bool BF16>
hipError_t launch_w4_mb(const W4Args &p, hipStream_t stream)
{
    // 16-row blocks of A per workgroup: all of M up to 64 rows, else 64-row
    // slabs (the weight is then streamed once per slab).  Two K groups need
    // every scale group inside one 256-k step.
    const int64_t mb = (p.M + 15) / 16;
    const bool two = kKS % p.G == 0;
    if (!two) {
        if (mb <= 1) return launch_w4<W4One<1, BF16>>(p, stream);
        if (mb <= 2) return launch_w4<W4One<2, BF16>>(p, stream);
        if (mb <= 3) return launch_w4<W4One<3, BF16>>(p, stream);
        return launch_w4<W4One<4, BF16>>(p, stream);
    }
    if (mb > 3)
        return launch_w4<W4One<4, BF16>>(p, stream);
    switch (p.G) {
    case 32: return launch_two<1, BF16>(mb, p, stream);
    case 64: return launch_two<2, BF16>(mb, p, stream);
    case 128: return launch_two<4, BF16>(mb, p, stream);
    default: return launch_two<8, BF16>(mb, p, stream);
    }
}

// The plain form: one thread per output, fp32 fused multiply-add over k
// ascending of A times the exact dequantized weight s * q.
__global__ void __launch_bounds__(256) gemm_w4_naive_kernel(W4Args p)
{
    const int64_t total = p.M * p.N;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = e / p.N, j = e - (e / p.N) * p.N;
        const bool bf = p.bf16 != 0;
        auto val = [bf](uint16_t h) { return bf ? bits_to_float<true>(h) : bits_to_float<false>(h); };
        float s = 0.0f;
        for (int64_t k = 0; k < p.K; ++k) {
            const uint8_t byte = p.Wq[j * p.ldw + k / 2];
            const int nib = (k & 1) ? (byte >> 4) : (byte & 15);
            const int q = nib >= 8 ? nib - 16 : nib;
            const float w = val(p.S[j * p.lds + k / p.G]) * (float)q;   // exact
            s = __builtin_fmaf(val(p.A[i * p.lda + k]), w, s);
        }
        if (p.bias != nullptr)
            s += val(p.bias[j]);
        const float r = (p.relu == 0 || s > 0.0f) ? s : 0.0f;
        p.C[i * p.ldc + j] = bf ? __builtin_bit_cast(uint16_t, (__bf16)r)
                                : __builtin_bit_cast(uint16_t, (_Float16)r);
    }
}

}  // namespace

bool w4_layout_ok(const W4Args &p)
{
    const auto a16 = [](const void *q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
    const auto a8 = [](const void *q) { return (reinterpret_cast<uintptr_t>(q) & 7) == 0; };
    if (!a16(p.A) || !a16(p.Wq) || !a8(p.C) || (p.bias != nullptr && !a8(p.bias)))
        return false;
    if ((p.lda & 7) || (p.ldw & 15) || (p.ldc & 3) || (p.N & 3))
        return false;
    if (p.G % 32 || p.K % p.G)
        return false;
    // 32-bit buffer offsets over 64 A rows and 64 weight rows
    if (p.lda > (1 << 24) || p.ldw > (1 << 25))
        return false;
    const int64_t mb = (p.M + 15) / 16;
    const bool two = kKS % p.G == 0;
    const int64_t ring = mb <= 1 ? (two ? W4Two<1, false, 4>::RING : W4One<1, false>::RING)
                         : mb <= 2 ? (two ? W4Two<2, false, 4>::RING : W4One<2, false>::RING)
                         : mb <= 3 ? (two ? W4Two<3, false, 4>::RING : W4One<3, false>::RING)
                                   : W4One<4, false>::RING;
    return ring + (p.K / p.G) * kRows * 2 <= kLds;
}

hipError_t launch_w4(const W4Args &p, hipStream_t stream)
{
    W4Args q = p;
    q.scales_vec = (reinterpret_cast<uintptr_t>(p.S) & 15) == 0 && (p.lds & 7) == 0 &&
                   ((p.K / p.G) & 7) == 0;
    return q.bf16 ? launch_w4_mb<true>(q, stream) : launch_w4_mb<false>(q, stream);
}

hipError_t launch_w4_naive(const W4Args &p, hipStream_t stream)
{
    int64_t blocks = (p.M * p.N + 255) / 256;
    if (blocks > 65536)
        blocks = 65536;
    hipLaunchKernelGGL(gemm_w4_naive_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace tg
