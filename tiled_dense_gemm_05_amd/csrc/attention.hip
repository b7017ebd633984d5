// Fused attention forward on gfx950: O = softmax(scale * Q K^T) V per batch
// and head, fp16 in and out, one pass over K and V (online softmax).
//
// The pages name fused attention (FlashAttention, MLA decode) among the tile
// programs they measure ("TileLang paper reading" page, section 5; the
// "80-line MLA article" page, sections 1-2) without giving the algorithm;
// this kernel reuses the GEMM's tile machinery for the standard one-pass
// form: per query block, walk the key/value tiles, keep a running maximum
// and sum of exponentials per query, rescale the output accumulator when the
// maximum grows (here: by more than 2^8), divide once at the end.
//
// Layout: Q (B, Sq, H, D), K and V (B, Sk, Hkv, D), O (B, Sq, H, D), each
// contiguous; D = 64 or 128; query head h reads key/value head h / (H / Hkv)
// (Hkv = H: multi-head; fewer: grouped-query, one: multi-query).  Key j is
// visible to query i always, or with `causal` when j <= i + (Sk - Sq).
//
// gfx950 design:
//  * One workgroup of NW waves per 32*NW query rows of one (batch,
//    key/value head); the rows are the (position, query head) pairs of the
//    heads that share it, position-major, so a K/V tile serves every head of
//    the group and positions still grow with the row (the causal logic sees
//    row r at position r / g, g = H / Hkv).  Wave w owns rows 32w .. 32w+31.
//    K/V tiles of 64 keys are staged in a 2-stage LDS ring by
//    buffer_load_dwordx4 ... lds (rows past Sk read as zeros and are masked
//    out of the softmax).
//  * Both products run on v_mfma_f32_32x32x16_f16 with the operand roles
//    swapped as in the GEMM kernels: S^T = K Q^T and O^T = V^T P^T.  A lane
//    then holds 32 scores (and, later, 4-column groups of the output) of ONE
//    query, so the softmax statistics need one cross-lane exchange (the lane
//    32 apart holds the query's other keys) and the probabilities, packed to
//    fp16, are already the second operand of the P V product: the key order
//    inside a 16-key step is permuted identically on both operands (the V^T
//    fragments come from transpose reads that fetch exactly those keys).
//  * Q fragments stay in registers for the whole walk; scores use exp2 with
//    |scale| * log2(e) folded into one FMA per score (a negative scale is
//    carried by Q), tiles that every query of a wave sees skip the mask,
//    and the row sums add the fp16 probabilities in pairs (v_dot2).
#include "tg_mla.h"

namespace tg {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) f16x8 lds_f16x8;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kBK = 64;    // keys per tile

template <int D_, int NW_>
struct AttnCfg {
    static constexpr int D = D_;
    static constexpr int NW = NW_;                   // waves; 32 queries each
    static constexpr int BQ = 32 * NW;               // queries per workgroup
    static constexpr int CD = D / 8;                 // 16-byte chunks per row
    static constexpr int TILE = kBK * D;             // fp16 elements of a K (or V) tile
    static constexpr int STAGE = 2 * TILE;           // K then V
    static constexpr int LDS = 2 * STAGE * 2;        // two stages, bytes
    static constexpr int RPB = 64 / CD;              // rows per 1 KiB block
    static constexpr int LD = TILE / 512 / NW;       // 1 KiB blocks per wave per tile
    static_assert((TILE / 512) % NW == 0, "blocks per wave");
    static constexpr int DS = D / 16;                // 16-wide d steps
    static constexpr int DB = D / 32;                // 32-wide d blocks of the output
    static_assert(D == 64 || D == 128, "head dim");
};

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N <= 63, "vmcnt");
    constexpr int imm = (N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(imm);
    asm volatile("" ::: "memory");
}

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
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voff, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %2\n\t"
                 "s_nop 0\n\t"
                 "buffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(lds_addr)
                 : "m0");
}
// The same with the non-temporal hint, for data read once (the latent cache).
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

// K tile rows (keys) are read as 16-byte chunks by 32 lanes of consecutive
// rows: XOR the chunk with the row.  V tile rows are read by transpose reads
// of 4 consecutive rows: move those rows to different quarters of the bank
// line (256-byte rows: XOR with the row's position in the 4; 128-byte rows,
// two to a bank line: XOR with its second bit).  Both stay inside the row.
template <int CD>
__device__ __forceinline__ int swz_k(int row, int c) { return c ^ (row % CD); }
template <int CD>
__device__ __forceinline__ int swz_v(int row, int c)
{
    if constexpr (CD >= 16)
        return c ^ ((row & 3) << 2);
    else
        return c ^ (((row >> 1) & 1) << 2);
}

// Exponentials are taken relative to a running maximum that is raised only
// when a tile's maximum exceeds it by more than this (log2 units): every
// exponential stays <= 2^8, the output accumulator is rescaled rarely, and
// the final division by the sum taken against the same maximum cancels it.
constexpr float kGrowLog2 = 8.0f;

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// The two lanes 32 apart hold the same query: combine their values.
__device__ __forceinline__ float max_pair(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Masks the raw scores of keys at or past `lim` (tile offsets, see below).
template <int KB = 2>
__device__ __forceinline__ void mask_tile(f32x16 (&s)[KB], int lim, int hi)
{
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int ko = kb * 32 + 8 * (r / 4) + 4 * hi + (r % 4);
            s[kb][r] = ko < lim ? s[kb][r] : -__builtin_inff();
        }
    }
}

// One tile's softmax step for this lane's query: raw scores s (16 KB of the
// tile's 32 KB keys: register r of block kb is key 32 kb + 8 (r / 4) +
// 4 hi + r % 4; masked keys hold -inf, and sl2 > 0 turns them into zeros).  Raises
// the running maximum if needed (rescaling the accumulator and the sum),
// writes the fp16 probabilities in the operand order of the P V product and
// adds them to the sum (the rounded values, so the weights applied to V are
// exactly the ones the sum divides by).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// x *= a for an accumulator held in an AGPR, in place: keeps the rare
// rescale from making the compiler move a whole accumulator into VGPRs and
// back on every tile.  The caller has waited out the matrix-core write of x.
__device__ __forceinline__ void scale_agpr(float &x, float a)
{
    float tmp;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\t"
                 "v_mul_f32_e32 %1, %2, %1\n\t"
                 "v_accvgpr_write_b32 %0, %1"
                 : "+a"(x), "=&v"(tmp)
                 : "v"(a));
}
#pragma clang diagnostic pop

template <int DB, int KB = 2, bool AGPR_RESCALE = false>
__device__ __forceinline__ void softmax_tile(f32x16 (&s)[KB], f16x8 (&pf)[2 * KB],
                                             f32x16 (&acc_o)[DB], float &m_run, float &l_run,
                                             float sl2)
{
    float mt = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; r += 2)
            mt = __builtin_fmaxf(mt, __builtin_fmaxf(s[kb][r], s[kb][r + 1]));
    }
    mt = max_pair(mt);
    const float m_tile = __builtin_fmaxf(mt * sl2, -1.0e30f);
    const bool grow = m_tile > m_run + kGrowLog2;
    if (__builtin_amdgcn_ballot_w64(grow)) {
        const float m_new = grow ? m_tile : m_run;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
        if constexpr (AGPR_RESCALE) {
            // the last matrix-core writes of acc_o are a tile back; wait out
            // the longest result latency anyway before reading them
            asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
            for (int db = 0; db < DB; ++db) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float x = acc_o[db][r];
                    scale_agpr(x, alpha);
                    acc_o[db][r] = x;
                }
            }
            asm volatile("s_nop 4" ::: "memory");
        } else {
#pragma unroll
            for (int db = 0; db < DB; ++db)
                acc_o[db] *= alpha;
        }
    }
    const float neg_m = -m_run;
#pragma unroll
    for (int kk = 0; kk < 2 * KB; ++kk) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            pf[kk][j] = (_Float16)__builtin_amdgcn_exp2f(
                __builtin_fmaf(s[kk / 2][8 * (kk % 2) + j], sl2, neg_m));
    }
    float ls[2] = {0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < 2 * KB; ++kk) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            ls[j & 1] = __builtin_amdgcn_fdot2(f16x2{pf[kk][2 * j], pf[kk][2 * j + 1]},
                                               f16x2{(_Float16)1.0f, (_Float16)1.0f}, ls[j & 1], false);
    }
    l_run += ls[0] + ls[1];
}

// Two waves per SIMD: lets the scheduler keep LDS reads in flight ahead of
// the matrix instructions that consume them instead of minimizing registers.
template <class T>
__global__ void __launch_bounds__(64 * T::NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
attention_fwd_kernel(AttnArgs p)
{
    __shared__ __attribute__((aligned(1024))) uint16_t smem[T::LDS / 2];
    const lds_u16 *lds = (const lds_u16 *)smem;
    const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t bh = blockIdx.x;                 // (batch, key/value head)
    const int64_t b = bh / p.Hkv, kvh = bh % p.Hkv;
    const int64_t Sq = p.Sq, Sk = p.Sk;
    const int64_t g = p.H / p.Hkv;                   // query heads per key/value head
    const int64_t rows = Sq * g;
    // Workgroups are dispatched x fastest: every (batch, head) of one query
    // block before the next block.  With the causal mask later query blocks
    // have more keys, so those go first, across all (batch, head) at once.
    const int64_t qj = p.qb0 + (int64_t)blockIdx.y;
    const int64_t qb = p.causal ? p.nqb - 1 - qj : qj;
    const int64_t q0 = qb * T::BQ;                 // first row of the block
    const int64_t rs = p.Hkv * T::D;                 // K/V elements between positions
    const int64_t r = q0 + wave * 32 + (lane & 31);  // this lane's row
    const bool live = r < rows;
    const int64_t q = r / g;                         // its query position
    const int64_t h = kvh * g + r % g;               // and query head
    const int hi = lane >> 5;
    const int64_t shift = Sk - Sq;                   // causal: query i sees keys j <= i + shift
    const int64_t wq0 = (q0 + wave * 32) / g;        // position of the wave's first row
    const int64_t wq1 = (q0 + wave * 32 + 31) / g;   // ... and of its last

    // Keys this block needs: all, or with the causal mask up to the block's
    // last position's horizon.
    int64_t kend = Sk;
    if (p.causal) {
        const int64_t lim = (q0 + T::BQ - 1) / g + shift + 1;
        kend = lim < 0 ? 0 : (lim < Sk ? lim : Sk);
    }
    const int tiles = (int)((kend + kBK - 1) / kBK);

    // Q^T fragments (second operand): lane holds Q[q][16 ds + 8 hi .. + 7].
    f16x8 qf[T::DS];
    {
        const uint16_t *qrow = p.Q + ((b * Sq + (live ? q : 0)) * p.H + (live ? h : 0)) * T::D;
#pragma unroll
        for (int ds = 0; ds < T::DS; ++ds) {
            qf[ds] = f16x8{};
            if (live)
                qf[ds] = *reinterpret_cast<const f16x8 *>(qrow + ds * 16 + 8 * hi);
            // a negative scale is carried by Q (negation is exact), so the
            // scores are scaled by |scale| and their maximum stays a maximum
            if (p.scale < 0.0f)
                qf[ds] = -qf[ds];
        }
    }

    // DMA plan: a K (or V) tile is 64 rows of D fp16; wave w moves 1 KiB
    // blocks w, w + 4, ...: lane L -> row blk * RPB + L / CD, physical chunk
    // L % CD, which holds the swizzled logical chunk.
    uint32_t k_voff[T::LD], v_voff[T::LD];
    int k_row[T::LD];
#pragma unroll
    for (int i = 0; i < T::LD; ++i) {
        const int blk = wave + T::NW * i;
        const int row = blk * T::RPB + lane / T::CD;
        const int pc = lane % T::CD;
        k_row[i] = row;
        k_voff[i] = (uint32_t)((row * rs + swz_k<T::CD>(row, pc) * 8) * 2);
        v_voff[i] = (uint32_t)((row * rs + swz_v<T::CD>(row, pc) * 8) * 2);
    }
    const uint16_t *Kb = p.K + (b * Sk * p.Hkv + kvh) * T::D;
    const uint16_t *Vb = p.V + (b * Sk * p.Hkv + kvh) * T::D;
    auto issue = [&](int t) {
        const int64_t k0 = (int64_t)t * kBK;
        const i32x4 rk = make_rsrc(Kb + k0 * rs);
        const i32x4 rv = make_rsrc(Vb + k0 * rs);
        const uint32_t base = lds_base + (uint32_t)((t & 1) * T::STAGE * 2);
#pragma unroll
        for (int i = 0; i < T::LD; ++i) {
            const bool ok = k0 + k_row[i] < kend;
            dma16(rk, ok ? k_voff[i] : kOutOfRange,
                  base + (uint32_t)((wave + T::NW * i) * 1024));
            dma16(rv, ok ? v_voff[i] : kOutOfRange,
                  base + (uint32_t)(T::TILE * 2 + (wave + T::NW * i) * 1024));
        }
    };

    f32x16 acc_o[T::DB];
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
        acc_o[db] = f32x16{};
    // running maximum (log2 units, finite so a fully masked tile leaves it
    // unchanged) and this lane's share of the sum of probabilities
    float m_run = -1.0e30f, l_run = 0.0f;
    // |scale| * log2(e), kept positive so masked scores (-inf) map to zero
    // (a zero scale becomes 1e-30: every exponential is then 1 to fp32 precision)
    const float sl2 = __builtin_fmaxf(__builtin_fabsf(p.scale) * 1.44269504088896340736f, 1.0e-30f);
    const int64_t horizon = q + shift;

    if (tiles > 0)
        issue(0);
    for (int t = 0; t < tiles; ++t) {
        wait_vmcnt<0>();      // tile t has landed (this wave's part)
        block_barrier();      // ... every wave's part; tile t-1's stage is free
        if (t + 1 < tiles)
            issue(t + 1);
        const int64_t k0 = (int64_t)t * kBK;
        // causal: none of this wave's queries sees the tile (it was loaded
        // for the block's later waves)
        if (p.causal && k0 > wq1 + shift)
            continue;
        const lds_u16 *Ks = lds + (t & 1) * T::STAGE;
        const lds_u16 *Vs = Ks + T::TILE;

        // S^T = K Q^T: two 32-key blocks; lane: query q, keys
        // k0 + 32 kb + 8 (r / 4) + 4 hi + r % 4 for register r.
        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = f32x16{};
            const int row = kb * 32 + (lane & 31);
#pragma unroll
            for (int ds = 0; ds < T::DS; ++ds) {
                const int c = ds * 2 + hi;
                const f16x8 kf = *reinterpret_cast<const lds_f16x8 *>(
                    Ks + row * T::D + swz_k<T::CD>(row, c) * 8);
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[ds], s[kb], 0, 0, 0);
            }
        }
        // mask only where some key of the tile is hidden from some query of
        // the wave
        if (!(k0 + kBK <= kend && (!p.causal || k0 + kBK - 1 <= wq0 + shift))) {
            int64_t lim = kend - k0;
            if (p.causal && horizon + 1 - k0 < lim)
                lim = horizon + 1 - k0;
            lim = lim < 0 ? 0 : (lim > kBK ? kBK : lim);
            mask_tile(s, (int)lim, hi);
        }
        f16x8 pf[4];
        softmax_tile<T::DB>(s, pf, acc_o, m_run, l_run, sl2);
        // O^T += V^T P^T: k-step kk covers keys k0 + 16 kk + {4 hi .. 4 hi + 3,
        // 8 + 4 hi .. 8 + 4 hi + 3} in the order of pf[kk]; two transpose
        // reads fetch V for those keys, column 32 db + lane % 32.
#pragma unroll
        for (int db = 0; db < T::DB; ++db) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                s16x4 vh[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int key = kk * 16 + 4 * hi + 8 * hh + ((lane & 15) >> 2);
                    const int d = db * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
                    const lds_u16 *src = Vs + key * T::D + swz_v<T::CD>(key, d >> 3) * 8 + (d & 7);
                    vh[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)src);
                }
                const f16x8 vf = __builtin_bit_cast(
                    f16x8, __builtin_shufflevector(vh[0], vh[1], 0, 1, 2, 3, 4, 5, 6, 7));
                acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[kk], acc_o[db], 0, 0, 0);
            }
        }
    }
    wait_vmcnt<0>();

    // Output: the query's sum of exponentials is split over lanes l and l^32.
    const float l_all = l_run + __shfl_xor(l_run, 32);
    const float inv = l_all > 0.0f ? 1.0f / l_all : 0.0f;
    if (live) {
        uint16_t *orow = p.O + ((b * Sq + q) * p.H + h) * T::D;
#pragma unroll
        for (int db = 0; db < T::DB; ++db) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = db * 32 + 8 * g + 4 * hi;
                u32x2 w;
                w.x = epi_pack2<false>(acc_o[db][4 * g + 0] * inv, acc_o[db][4 * g + 1] * inv, false);
                w.y = epi_pack2<false>(acc_o[db][4 * g + 2] * inv, acc_o[db][4 * g + 3] * inv, false);
                *reinterpret_cast<u32x2 *>(orow + d) = w;
            }
        }
    }
}

template <int D, int NW>
hipError_t launch_attn(const AttnArgs &p, hipStream_t stream)
{
    // grid x: (batch, key/value head) pairs; grid y: blocks of query rows,
    // in launches of at most 65535
    const int64_t bh = p.B * p.Hkv;
    const int64_t nqb = (p.Sq * (p.H / p.Hkv) + 32 * NW - 1) / (32 * NW);
    if (bh > 0x7fffffff)
        return hipErrorInvalidValue;
    for (int64_t y0 = 0; y0 < nqb; y0 += 65535) {
        AttnArgs q = p;
        q.nqb = nqb;
        q.qb0 = y0;
        const int64_t gy = (nqb - y0) < 65535 ? (nqb - y0) : 65535;
        hipLaunchKernelGGL((attention_fwd_kernel<AttnCfg<D, NW>>), dim3((unsigned)bh, (unsigned)gy),
                           dim3(64 * NW), 0, stream, q);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// The same attention forward on v_mfma_f32_16x16x32_f16 products.  The
// matrix cores run the same flops on twice as many smaller products, which
// draw less power each; on this power-capped part that buys clock.
//
// Layout (operand roles swapped as above: S^T = K Q^T, O^T = V^T P^T):
//  * A wave owns 32 query rows as two blocks of 16 (qb); lane c = lane % 16
//    of 16-lane group g = lane / 16 holds row 16 qb + c of each block.
//  * Score fragment (qb, kb) covers 16 keys of the 64-key tile: the lane
//    holds keys 16 kb + 4 g .. 4 g + 3 of its row.  A row's 64 scores sit in
//    the four lanes c, c + 16, c + 32, c + 48: its maximum and sum take two
//    exchanges (v_permlane16_swap, then v_permlane32_swap).
//  * The probabilities of k step ks (keys 32 ks .. 32 ks + 31) are the P^T
//    operand as they lie: the lane's 8 k values are keys 32 ks + 4 g + 0..3
//    and 32 ks + 16 + 4 g + 0..3; the V^T operand takes the same keys by two
//    transpose reads of 4 consecutive rows each.
//  * Output fragment (qb, db): the lane holds values 16 db + 4 g .. + 3 of
//    its row.

// The maximum of x over the four lanes c, c + 16, c + 32, c + 48.
__device__ __forceinline__ float max_quad(float x)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float m = __builtin_fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    return __builtin_fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// The sum of x over the same four lanes (in a fixed order: every lane gets
// the same bits).
__device__ __forceinline__ float sum_quad(float x)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float s = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <class T>
__global__ void __launch_bounds__(64 * T::NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
attention_fwd16_kernel(AttnArgs p)
{
    constexpr int DS = T::D / 32;    // 32-wide d steps of the scores
    constexpr int DB = T::D / 16;    // 16-wide d blocks of the output
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    __shared__ __attribute__((aligned(1024))) uint16_t smem[T::LDS / 2];
    const lds_u16 *lds = (const lds_u16 *)smem;
    const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int c16 = lane & 15, g4 = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t bh = blockIdx.x;                 // (batch, key/value head)
    const int64_t b = bh / p.Hkv, kvh = bh % p.Hkv;
    const int64_t Sq = p.Sq, Sk = p.Sk;
    const int64_t g = p.H / p.Hkv;                   // query heads per key/value head
    const int64_t rows = Sq * g;
    const int64_t qj = p.qb0 + (int64_t)blockIdx.y;
    const int64_t qblk = p.causal ? p.nqb - 1 - qj : qj;
    const int64_t q0 = qblk * T::BQ;               // first row of the block
    const int64_t rs = p.Hkv * T::D;                 // K/V elements between positions
    const int64_t shift = Sk - Sq;
    const int64_t wq0 = (q0 + wave * 32) / g;        // position of the wave's first row
    const int64_t wq1 = (q0 + wave * 32 + 31) / g;   // ... and of its last
    // this lane's two rows (one per 16-row block): position, head, horizon
    bool live[2];
    int64_t qpos[2], head[2], horizon[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int64_t r = q0 + wave * 32 + qb * 16 + c16;
        live[qb] = r < rows;
        qpos[qb] = r / g;
        head[qb] = kvh * g + r % g;
        horizon[qb] = qpos[qb] + shift;
    }

    int64_t kend = Sk;
    if (p.causal) {
        const int64_t lim = (q0 + T::BQ - 1) / g + shift + 1;
        kend = lim < 0 ? 0 : (lim < Sk ? lim : Sk);
    }
    const int tiles = (int)((kend + kBK - 1) / kBK);

    // Q^T fragments: lane holds Q[row][32 ds + 8 g .. + 7] of each block.
    f16x8 qf[2][DS];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const uint16_t *qrow =
            p.Q + ((b * Sq + (live[qb] ? qpos[qb] : 0)) * p.H + (live[qb] ? head[qb] : 0)) * T::D;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
            qf[qb][ds] = f16x8{};
            if (live[qb])
                qf[qb][ds] = *reinterpret_cast<const f16x8 *>(qrow + ds * 32 + 8 * g4);
            if (p.scale < 0.0f)
                qf[qb][ds] = -qf[qb][ds];
        }
    }

    // DMA plan, as in attention_fwd_kernel.
    uint32_t k_voff[T::LD], v_voff[T::LD];
    int k_row[T::LD];
#pragma unroll
    for (int i = 0; i < T::LD; ++i) {
        const int blk = wave + T::NW * i;
        const int row = blk * T::RPB + lane / T::CD;
        const int pc = lane % T::CD;
        k_row[i] = row;
        k_voff[i] = (uint32_t)((row * rs + swz_k<T::CD>(row, pc) * 8) * 2);
        v_voff[i] = (uint32_t)((row * rs + swz_v<T::CD>(row, pc) * 8) * 2);
    }
    const uint16_t *Kb = p.K + (b * Sk * p.Hkv + kvh) * T::D;
    const uint16_t *Vb = p.V + (b * Sk * p.Hkv + kvh) * T::D;
    auto issue = [&](int t) {
        const int64_t k0 = (int64_t)t * kBK;
        const i32x4 rk = make_rsrc(Kb + k0 * rs);
        const i32x4 rv = make_rsrc(Vb + k0 * rs);
        const uint32_t base = lds_base + (uint32_t)((t & 1) * T::STAGE * 2);
#pragma unroll
        for (int i = 0; i < T::LD; ++i) {
            const bool ok = k0 + k_row[i] < kend;
            dma16(rk, ok ? k_voff[i] : kOutOfRange, base + (uint32_t)((wave + T::NW * i) * 1024));
            dma16(rv, ok ? v_voff[i] : kOutOfRange,
                  base + (uint32_t)(T::TILE * 2 + (wave + T::NW * i) * 1024));
        }
    };

    f32x4 acc_o[2][DB];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int db = 0; db < DB; ++db)
            acc_o[qb][db] = f32x4{};
    float m_run[2] = {-1.0e30f, -1.0e30f}, l_run[2] = {0.0f, 0.0f};
    const float sl2 = __builtin_fmaxf(__builtin_fabsf(p.scale) * 1.44269504088896340736f, 1.0e-30f);

    if (tiles > 0)
        issue(0);
    for (int t = 0; t < tiles; ++t) {
        wait_vmcnt<0>();
        block_barrier();
        if (t + 1 < tiles)
            issue(t + 1);
        const int64_t k0 = (int64_t)t * kBK;
        if (p.causal && k0 > wq1 + shift)
            continue;
        const lds_u16 *Ks = lds + (t & 1) * T::STAGE;
        const lds_u16 *Vs = Ks + T::TILE;

        // S^T = K Q^T: one 16-byte K read per (key block, d step) serves
        // both row blocks.
        f32x4 s[2][4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            s[0][kb] = f32x4{};
            s[1][kb] = f32x4{};
            const int row = kb * 16 + c16;
#pragma unroll
            for (int ds = 0; ds < DS; ++ds) {
                const int c = ds * 4 + g4;
                const f16x8 kf = *reinterpret_cast<const lds_f16x8 *>(
                    Ks + row * T::D + swz_k<T::CD>(row, c) * 8);
                s[0][kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[0][ds], s[0][kb], 0, 0, 0);
                s[1][kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[1][ds], s[1][kb], 0, 0, 0);
            }
        }
        if (!(k0 + kBK <= kend && (!p.causal || k0 + kBK - 1 <= wq0 + shift))) {
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                int64_t lim = kend - k0;
                if (p.causal && horizon[qb] + 1 - k0 < lim)
                    lim = horizon[qb] + 1 - k0;
                lim = lim < 0 ? 0 : (lim > kBK ? kBK : lim);
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        s[qb][kb][i] = kb * 16 + 4 * g4 + i < lim ? s[qb][kb][i] : -__builtin_inff();
            }
        }
        // softmax per row block; probabilities in the P^T operand order
        f16x8 pf[2][2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            float mt = -__builtin_inff();
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                mt = __builtin_fmaxf(mt, __builtin_fmaxf(__builtin_fmaxf(s[qb][kb][0], s[qb][kb][1]),
                                                         __builtin_fmaxf(s[qb][kb][2], s[qb][kb][3])));
            mt = max_quad(mt);
            const float m_tile = __builtin_fmaxf(mt * sl2, -1.0e30f);
            const bool grow = m_tile > m_run[qb] + kGrowLog2;
            if (__builtin_amdgcn_ballot_w64(grow)) {
                const float m_new = grow ? m_tile : m_run[qb];
                const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
                m_run[qb] = m_new;
                l_run[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    acc_o[qb][db] *= alpha;
            }
            const float neg_m = -m_run[qb];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    pf[qb][ks][j] = (_Float16)__builtin_amdgcn_exp2f(
                        __builtin_fmaf(s[qb][2 * ks + j / 4][j % 4], sl2, neg_m));
            float ls[2] = {0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    ls[j & 1] = __builtin_amdgcn_fdot2(f16x2{pf[qb][ks][2 * j], pf[qb][ks][2 * j + 1]},
                                                       f16x2{(_Float16)1.0f, (_Float16)1.0f}, ls[j & 1],
                                                       false);
            l_run[qb] += ls[0] + ls[1];
        }
        // O^T += V^T P^T: one pair of transpose reads per (d block, k step)
        // serves both row blocks.
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                s16x4 vh[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int key = ks * 32 + 16 * hh + 4 * g4 + (c16 >> 2);
                    const int d = db * 16 + 4 * (lane & 3);
                    const lds_u16 *src = Vs + key * T::D + swz_v<T::CD>(key, d >> 3) * 8 + (d & 7);
                    vh[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)src);
                }
                const f16x8 vf = __builtin_bit_cast(
                    f16x8, __builtin_shufflevector(vh[0], vh[1], 0, 1, 2, 3, 4, 5, 6, 7));
                acc_o[0][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[0][ks], acc_o[0][db], 0, 0, 0);
                acc_o[1][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[1][ks], acc_o[1][db], 0, 0, 0);
            }
        }
    }
    wait_vmcnt<0>();

    // Output: a row's sum of exponentials is split over its four lanes.
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const float l_all = sum_quad(l_run[qb]);
        const float inv = l_all > 0.0f ? 1.0f / l_all : 0.0f;
        if (live[qb]) {
            uint16_t *orow = p.O + ((b * Sq + qpos[qb]) * p.H + head[qb]) * T::D;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                u32x2 w;
                w.x = epi_pack2<false>(acc_o[qb][db][0] * inv, acc_o[qb][db][1] * inv, false);
                w.y = epi_pack2<false>(acc_o[qb][db][2] * inv, acc_o[qb][db][3] * inv, false);
                *reinterpret_cast<u32x2 *>(orow + db * 16 + 4 * g4) = w;
            }
        }
    }
}

template <int D, int NW>
hipError_t launch_attn16(const AttnArgs &p, hipStream_t stream)
{
    const int64_t bh = p.B * p.Hkv;
    const int64_t nqb = (p.Sq * (p.H / p.Hkv) + 32 * NW - 1) / (32 * NW);
    if (bh > 0x7fffffff)
        return hipErrorInvalidValue;
    for (int64_t y0 = 0; y0 < nqb; y0 += 65535) {
        AttnArgs q = p;
        q.nqb = nqb;
        q.qb0 = y0;
        const int64_t gy = (nqb - y0) < 65535 ? (nqb - y0) : 65535;
        hipLaunchKernelGGL((attention_fwd16_kernel<AttnCfg<D, NW>>), dim3((unsigned)bh, (unsigned)gy),
                           dim3(64 * NW), 0, stream, q);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// Latent-attention decode (the MLA decode the pages measure: "TileLang paper
// reading" page, section 5; "80-line MLA article" page, sections 1-2, which
// give its 512 + 64 head size).  One query per sequence; every cached token
// holds one row of 576 fp16 values, all of them the key and the first 512 the
// value, shared by every query head.
//
// gfx950 design:
//  * A workgroup of four waves, one per SIMD, serves 128 query heads of one
//    sequence over one range of its keys.  Wave w owns heads 32w .. 32w + 31
//    (one per lane pair) outright: its Q^T (36 fragments, 144 registers)
//    stays in registers and its 32 x 512 fp32 output in the 256 accumulation
//    registers.  The waves share nothing but the staged rows, so a tile costs
//    one barrier (to reuse its stage) and no exchange of partial scores, and
//    each cached row is staged once per 128 heads.
//  * What bounds the product on this part is the LDS read rate: every
//    16-byte K read, and every pair of 8-byte transpose reads of V, feeds one
//    32 x 32 x 16 product, and the LDS returns about one such read per 4
//    clocks per CU whatever its width.  A tile takes 36 + 64 reads per wave
//    (plus its 36 1 KiB stage writes) against 68 products of 32 clocks on
//    each SIMD: about 80 % of the LDS's time, the rest of it hidden behind
//    the matrix cores.
//  * Tiles of 32 cached rows (36 KiB) are staged in a 4-stage LDS ring by
//    buffer_load_dwordx4 ... lds with the non-temporal hint (each row is
//    read once: 2-3 % faster per call); the buffer's record count ends at the
//    range's last visible row, so later rows read as zeros (and are masked
//    out of the softmax).  Each wave moves 9 of a tile's 36 1-KiB blocks,
//    one beside each of the first 9 score products two tiles earlier.
//  * Scores S^T = K Q^T and O^T += V^T P^T as in the attention forward
//    above.  The same LDS rows are read as K (16-byte reads) and as V
//    (transpose reads of the first 512 values), so one chunk swizzle serves
//    both.  Rows are 1152 bytes, so in the 256-byte bank line (64 banks)
//    consecutive rows start alternately at 0 and 128; chunk c of row r sits
//    at c ^ x(r) with x(r) = 2 ((r / 2) mod 4) + (r / 8) mod 2, which with
//    that alternation puts the 16 rows a K fragment read serves at once on
//    16 different 16-byte slots, and the 4 rows x 2 chunks of a transpose
//    read on 8.
//  * Software pipeline, per tile t: tile t's 36 score products run on the
//    matrix cores while the vector units take tile t-1's softmax, one small
//    step beside each product (the order is pinned with scheduling
//    barriers); then tile t-1's 32 value products.  The barrier that frees
//    tile t-1's stage (and shows tile t+1) sits before the last three value
//    products, whose operands are already in registers, so the next tile's
//    first K reads run under them.
//  * When the sequences are too few to fill the chip the keys are split
//    into ranges (flash-decoding); each range writes its output normalised
//    by its own sum as fp16 (half the bytes of an fp32 partial) with its
//    running maximum and sum, and a combine kernel reweights and adds the
//    ranges in a fixed order, so results are deterministic.
namespace mla {
constexpr int D = kMlaDl + kMlaDr;          // 576 values per cached row
constexpr int BK = 32;                      // cached rows per tile
constexpr int TILE = BK * D;                // fp16 elements per tile
constexpr int BLOCKS = TILE * 2 / 1024;     // 1 KiB DMA blocks per tile (36)
constexpr int NW = kMlaHeadsPerBlock / 32;  // waves, 32 heads each (4)
constexpr int STAGES = 4;                   // ring depth (144 KiB of LDS)
constexpr int LD = BLOCKS / NW;             // DMA blocks per wave per tile (9)
constexpr int DS = D / 16;                  // 16-wide score steps (36)
constexpr int DN = kMlaDl / 16;             // of them over the first 512 values (32)
constexpr int QL = (DS - DN) * 512;         // fp16 elements of a wave's Q^T fragments kept in LDS
constexpr int DB = kMlaDl / 32;             // 32-wide output blocks (16)
constexpr int NV = 2 * DB;                  // value products per tile (32)
constexpr int KA = 3;                       // K fragments read ahead of their product
constexpr int VA = 3;                       // V fragments read ahead of their product
static_assert(BLOCKS % NW == 0 && NW == 4, "four waves share a tile's blocks");
static_assert(LD <= DS && VA <= DS && VA < NV, "pipeline steps");
}  // namespace mla

__device__ __forceinline__ int mla_swz(int row, int c)
{
    return c ^ (2 * ((row >> 1) & 3) + ((row >> 3) & 1));
}

__device__ __forceinline__ float fmax3(float a, float b, float c)
{
    return __builtin_fmaxf(a, __builtin_fmaxf(b, c));
}

__global__ void __launch_bounds__(64 * mla::NW) __attribute__((amdgpu_waves_per_eu(1, 1)))
mla_decode_kernel(MlaArgs p)
{
    using namespace mla;
    // the tile ring, then each wave's last four Q^T fragments (160 KiB)
    __shared__ __attribute__((aligned(1024))) uint16_t smem[STAGES * TILE + NW * QL];
    const lds_u16 *lds = (const lds_u16 *)smem;
    const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hi = lane >> 5;
    const int qbase = STAGES * TILE + wave * QL + lane * 8;   // Q^T fragment DN + j at + 512 j
    // grid x: 8 consecutive (sequence, key range) units, then the same 8
    // for the next head block, ...
    const int64_t nhb = (p.H + kMlaHeadsPerBlock - 1) / kMlaHeadsPerBlock;
    const int64_t gid = blockIdx.x;
    const int64_t unit = gid / (8 * nhb) * 8 + gid % 8;
    const int64_t hb = gid / 8 % nhb;
    if (unit >= p.B * p.splits)
        return;
    const int64_t b = unit / p.splits, sp = unit % p.splits;
    const int64_t h = hb * kMlaHeadsPerBlock + wave * 32 + (lane & 31);
    const bool live = h < p.H;

    int64_t n = p.Sk;
    if (p.seqlens) {
        const int64_t v = p.seqlens[b];
        n = v < 0 ? 0 : (v > p.Sk ? p.Sk : v);
    }
    const int64_t kbeg = sp * p.keys_per_split;
    int64_t kend = kbeg + p.keys_per_split;
    kend = kend < n ? kend : n;
    const int tiles = kend > kbeg ? (int)((kend - kbeg + BK - 1) / BK) : 0;

    // Q^T fragments (second operand): lane holds Q[b][h][16 ds + 8 hi .. + 7];
    // the first DN stay in registers, the rest (the 64 values past 512) in
    // LDS, read again for every tile: registers are what this kernel runs
    // short of
    f16x8 qf[DS];
    {
        // dead heads (past H) read head 0's row and keep zeros
        const uint16_t *qrow = p.Q + (b * p.H + (live ? h : 0)) * D;
        const bool neg = p.scale < 0.0f;   // a negative scale is carried by Q
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
            const f16x8 v = *reinterpret_cast<const f16x8 *>(qrow + ds * 16 + 8 * hi);
            const f16x8 q = live ? (neg ? -v : v) : f16x8{};
            if (ds < DN)
                qf[ds] = q;
            else
                *reinterpret_cast<f16x8 *>(smem + qbase + (ds - DN) * 512) = q;
        }
    }

    // DMA plan: slot s (16 bytes) of a tile is row s / 72, physical chunk
    // s % 72, which receives the row's logical chunk mla_swz(row, chunk);
    // wave w moves 1 KiB blocks w, w + 4, ..., w + 32.  The byte offsets
    // (< 36 KiB) are kept two to a register.
    uint32_t voff2[(LD + 1) / 2];
#pragma unroll
    for (int i = 0; i < (LD + 1) / 2; ++i)
        voff2[i] = 0;
#pragma unroll
    for (int i = 0; i < LD; ++i) {
        const int slot = (wave + NW * i) * 64 + lane;
        const int row = slot / (D / 8);
        const int pc = slot % (D / 8);
        voff2[i / 2] |= (uint32_t)((row * D + mla_swz(row, pc) * 8) * 2) << (16 * (i % 2));
    }
    const uint16_t *kvb = p.KV + b * p.Sk * D;
    // the buffer of tile t: its visible rows (none for a tile past the
    // range, whose loads then only write zeros into a stage nobody reads)
    auto tile_rsrc = [&](int t) {
        const int64_t k0 = kbeg + (int64_t)t * BK;
        int64_t rows = kend - k0 < BK ? kend - k0 : BK;
        rows = rows > 0 ? rows : 0;
        i32x4 r = make_rsrc(kvb + (rows > 0 ? k0 : 0) * D);
        r.z = __builtin_amdgcn_readfirstlane((int)(rows * D * 2));
        return r;
    };
    auto dma = [&](const i32x4 &rsrc, int t, int i) __attribute__((always_inline)) {
        dma16_nt(rsrc, (voff2[i / 2] >> (16 * (i % 2))) & 0xffffu,
              lds_base + (uint32_t)((t % STAGES) * TILE * 2 + (wave + NW * i) * 1024));
    };

    // LDS addresses as per-lane bases plus compile-time offsets: a K fragment
    // of step ds sits at kbase[ds % 4] + 64 (ds / 4) elements (adding 8 to a
    // chunk index leaves the XOR-ed low bits alone), a V fragment at
    // vbase[hh][db % 2] + 64 (db / 2) + 576 * 16 kk (its row mod 16 depends
    // on hh, not on kk)
    int kbase[4], vbase[2][2];   // fp16 elements from the stage start
    {
        const int row = lane & 31;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            kbase[j] = row * D + mla_swz(row, 2 * j + hi) * 8;
        const int dl = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int key = 8 * hh + 4 * hi + ((lane & 15) >> 2);
#pragma unroll
            for (int par = 0; par < 2; ++par) {
                const int d = par * 32 + dl;
                vbase[hh][par] = key * D + mla_swz(key, d >> 3) * 8 + (d & 7);
            }
        }
    }
    // the stage offset kept opaque, so the addresses stay base + constant
    auto stage = [&](int t) { return lds + __builtin_amdgcn_readfirstlane((t % STAGES) * TILE); };
    auto qread = [&](int ds) __attribute__((always_inline)) {
        return *reinterpret_cast<const lds_f16x8 *>(lds + qbase + (ds - DN) * 512);
    };
    auto kread = [&](const lds_u16 *S, int ds) __attribute__((always_inline)) {
        return *reinterpret_cast<const lds_f16x8 *>(S + kbase[ds & 3] + (ds >> 2) * 64);
    };
    // V^T fragment of value product i (kk = i / 16 selects the 16 keys, db =
    // i % 16 the 32 values): the transpose reads fetch keys 4 hi .. 4 hi + 3
    // and 8 + 4 hi .. 8 + 4 hi + 3 of the 16, the keys this lane's
    // probabilities hold in that order
    auto vread = [&](const lds_u16 *S, int i) __attribute__((always_inline)) {
        const int kk = i / DB, db = i % DB;
        s16x4 vh[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
            vh[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4 *)(S + vbase[hh][db & 1] + (db >> 1) * 64 + 16 * kk * D));
        return __builtin_bit_cast(f16x8,
                                  __builtin_shufflevector(vh[0], vh[1], 0, 1, 2, 3, 4, 5, 6, 7));
    };

    f32x16 acc_o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
        acc_o[db] = f32x16{};
    float m_run = -1.0e30f, l_run = 0.0f;
    const float sl2 = __builtin_fmaxf(__builtin_fabsf(p.scale) * 1.44269504088896340736f, 1.0e-30f);

    // The softmax of one tile's raw scores s (this lane's head; register r
    // holds key 8 (r / 4) + 4 hi + r % 4) cut into steps, each small enough
    // to sit beside one score product of the next tile: the running maximum
    // (raised only when the tile exceeds it by more than 2^8; `grow` and
    // `alpha` tell the caller to rescale its output), the fp16
    // probabilities pf in the value product's operand order and the running
    // sum of the rounded probabilities.  The arithmetic: the tile maximum
    // of the scores (this lane's 16 and its partner lane's), scaled by sl2
    // and floored at -1e30; grow when it exceeds m_run by more than 2^8, then
    // alpha = exp2(m_run - m_new); p = fp16(exp2(s * sl2 - m_run)); l_run =
    // l_run * alpha + the sum of the fp16 p (dot products with ones).
    float sa0 = 0.f, sa1 = 0.f, sa2 = 0.f, sa3 = 0.f, sa4 = 0.f, sa5 = 0.f;
    float mt = 0.f, m_new = 0.f, alpha = 1.0f, neg_m = 0.f, x_even = 0.f, ls0 = 0.f, ls1 = 0.f;
    bool grow = false;
    f16x8 pf[2] = {f16x8{}, f16x8{}};
    auto sm_step = [&](const f32x16 &s, int k) __attribute__((always_inline)) {
        if (k == 0) {
            sa0 = fmax3(s[0], s[1], s[2]);
            sa1 = fmax3(s[3], s[4], s[5]);
            asm volatile("" ::"v"(sa0), "v"(sa1));
        } else if (k == 1) {
            sa2 = fmax3(s[6], s[7], s[8]);
            sa3 = fmax3(s[9], s[10], s[11]);
            asm volatile("" ::"v"(sa2), "v"(sa3));
        } else if (k == 2) {
            sa4 = fmax3(s[12], s[13], s[14]);
            sa5 = __builtin_fmaxf(s[15], sa0);
            asm volatile("" ::"v"(sa4), "v"(sa5));
        } else if (k == 3) {
            mt = fmax3(fmax3(sa1, sa2, sa3), sa4, sa5);
            asm volatile("" ::"v"(mt));
        } else if (k == 4) {
            mt = max_pair(mt);
            asm volatile("" ::"v"(mt));
        } else if (k == 5) {
            const float m_tile = __builtin_fmaxf(mt * sl2, -1.0e30f);
            grow = m_tile > m_run + kGrowLog2;
            m_new = grow ? m_tile : m_run;
            asm volatile("" ::"v"(m_new));
        } else if (k == 6) {
            alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            neg_m = -m_run;
            asm volatile("" ::"v"(alpha), "v"(neg_m));
        } else if (k >= 7 && k < 23) {
            const int j = k - 7;
            const float x = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j], sl2, neg_m));
            if (j % 2 == 0) {
                x_even = x;
                asm volatile("" ::"v"(x_even));
            } else {
                pf[j / 8][j % 8 - 1] = (_Float16)x_even;
                pf[j / 8][j % 8] = (_Float16)x;
                asm volatile("" ::"v"(pf[j / 8]));
            }
        } else if (k >= 23 && k < 27) {
            const int kk = (k - 23) / 2, o = 4 * ((k - 23) % 2);
            const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
            ls0 = __builtin_amdgcn_fdot2(f16x2{pf[kk][o], pf[kk][o + 1]}, one, ls0, false);
            ls1 = __builtin_amdgcn_fdot2(f16x2{pf[kk][o + 2], pf[kk][o + 3]}, one, ls1, false);
            asm volatile("" ::"v"(ls0), "v"(ls1));
        } else if (k == 27) {
            l_run = l_run * alpha + (ls0 + ls1);
            ls0 = ls1 = 0.0f;
            asm volatile("" ::"v"(l_run));
        }
    };

    // acc_o *= alpha in place in the accumulation registers (rare: the
    // running maximum of some head grew by more than 2^8).  Inside the loop
    // the last value products were issued a whole score loop earlier; after
    // it they were just issued, and `fresh` waits out their result latency
    // (the wait states here are inline assembly, which the compiler's
    // hazard tracking does not cover).
    auto rescale = [&](float a, bool fresh) __attribute__((always_inline)) {
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
        if (fresh)
            asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float x = acc_o[db][r];
                scale_agpr(x, a);
                acc_o[db][r] = x;
            }
        }
        asm volatile("s_nop 4" ::: "memory");
    };

    if (tiles > 0) {
        // tiles 0, 1 and 2 go to stages 0-2; tile t + 2 is loaded beside the
        // score products of tile t, into the stage tile t - 2 left
        // (every tile slot issues its loads, so the counts below are fixed)
        for (int t = 0; t < 3; ++t) {
            const i32x4 rs = tile_rsrc(t);
#pragma unroll
            for (int i = 0; i < LD; ++i)
                dma(rs, t, i);
        }
        wait_vmcnt<2 * LD>();
        block_barrier();                      // tile 0 visible

        // raw scores of the newest tile; only the range's last tile can be
        // partial
        f32x16 s = f32x16{};
        auto mask_last = [&](int t) __attribute__((always_inline)) {
            const int64_t k0 = kbeg + (int64_t)t * BK;
            if (t == tiles - 1 && k0 + BK > kend) {
                f32x16 sm[1] = {s};
                mask_tile<1>(sm, (int)(kend - k0), hi);
                s = sm[0];
            }
        };
        // carried from one tile to the next: the first KA K fragments of the
        // next tile, the V fragments of the last VA value products and the
        // probabilities those use
        f16x8 kn[KA], vt[VA], pv[2];
        {
            const lds_u16 *Ks = stage(0);
            f16x8 kf[DS], qv[DS - DN];
#pragma unroll
            for (int ds = 0; ds < KA; ++ds)
                kf[ds] = kread(Ks, ds);
#pragma unroll
            for (int ds = 0; ds < DS; ++ds) {
                if (ds + KA < DS)
                    kf[ds + KA] = kread(Ks, ds + KA);
                if (ds + KA >= DN && ds + KA < DS)
                    qv[ds + KA - DN] = qread(ds + KA);
                s = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[ds], ds < DN ? qf[ds] : qv[ds - DN], s,
                                                          0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
            mask_last(0);
#pragma unroll
            for (int k = 0; k < DS; ++k)
                sm_step(s, k);
        }
        if (tiles > 1) {
            wait_vmcnt<LD>();
            block_barrier();                  // tile 1 visible
            const lds_u16 *Ks = stage(1);
#pragma unroll
            for (int ds = 0; ds < KA; ++ds)
                kn[ds] = kread(Ks, ds);
        }
        for (int t = 1; t < tiles; ++t) {
            const lds_u16 *Ks = stage(t);
            const lds_u16 *Vs = stage(t - 1);
            const i32x4 rs = tile_rsrc(t + 2);
            f16x8 kf[DS], qv[DS - DN], vf[NV];
#pragma unroll
            for (int ds = 0; ds < KA; ++ds)
                kf[ds] = kn[ds];
            // tile t's scores beside tile t+2's loads; the last products
            // also fetch tile t-1's first V fragments
            s = f32x16{};
#pragma unroll
            for (int ds = 0; ds < DS; ++ds) {
                if (ds + KA < DS)
                    kf[ds + KA] = kread(Ks, ds + KA);
                if (ds + KA >= DN && ds + KA < DS)
                    qv[ds + KA - DN] = qread(ds + KA);
                s = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[ds], ds < DN ? qf[ds] : qv[ds - DN], s,
                                                          0, 0, 0);
                if (ds < LD)
                    dma(rs, t + 2, ds);
                if (ds >= DS - VA)
                    vf[ds - (DS - VA)] = vread(Vs, ds - (DS - VA));
                __builtin_amdgcn_sched_barrier(0);
            }
            // tile t-1's probabilities, before tile t's softmax replaces them;
            // its running maximum raised the output's scale if `grow`
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                pv[kk] = pf[kk];
            if (__builtin_amdgcn_ballot_w64(grow))
                rescale(alpha, false);
            mask_last(t);
            // tile t-1's value products, all but the last VA, beside tile
            // t's softmax
#pragma unroll
            for (int i = 0; i < NV - VA; ++i) {
                vf[i + VA] = vread(Vs, i + VA);
                acc_o[i % DB] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[i], pv[i / DB],
                                                                       acc_o[i % DB], 0, 0, 0);
                sm_step(s, i);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int k = NV - VA; k < DS; ++k)
                sm_step(s, k);
#pragma unroll
            for (int i = 0; i < VA; ++i)
                vt[i] = vf[NV - VA + i];
            if (t + 1 < tiles) {
                wait_vmcnt<LD>();             // tile t+1 landed
                block_barrier();              // tile t-1's stage free, tile t+1 visible
                const lds_u16 *Kn = stage(t + 1);
#pragma unroll
                for (int ds = 0; ds < KA; ++ds)
                    kn[ds] = kread(Kn, ds);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int i = NV - VA; i < NV; ++i)
                acc_o[i % DB] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vt[i - (NV - VA)], pv[i / DB],
                                                                       acc_o[i % DB], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        // the last tile's value products
        if (__builtin_amdgcn_ballot_w64(grow))
            rescale(alpha, true);
        const lds_u16 *Vs = stage(tiles - 1);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const f16x8 v = vread(Vs, i);
            acc_o[i % DB] = __builtin_amdgcn_mfma_f32_32x32x16_f16(v, pf[i / DB], acc_o[i % DB],
                                                                   0, 0, 0);
        }
    }
    wait_vmcnt<0>();

    // this head's sum of exponentials is split over lanes l and l ^ 32
    const float l_all = l_run + __shfl_xor(l_run, 32);
    if (!live)
        return;
    if (p.splits == 1) {
        const float inv = l_all > 0.0f ? 1.0f / l_all : 0.0f;
        uint16_t *orow = p.O + (b * p.H + h) * kMlaDl;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = db * 32 + 8 * g + 4 * hi;
                u32x2 w;
                w.x = epi_pack2<false>(acc_o[db][4 * g + 0] * inv, acc_o[db][4 * g + 1] * inv, false);
                w.y = epi_pack2<false>(acc_o[db][4 * g + 2] * inv, acc_o[db][4 * g + 3] * inv, false);
                *reinterpret_cast<u32x2 *>(orow + d) = w;
            }
        }
        return;
    }
    // a key range's partial: its output normalised by its own sum, rounded
    // to fp16 (a convex combination of cached values, so within their
    // range), with its running maximum and sum
    const int64_t slot = (b * p.H + h) * p.splits + sp;
    uint16_t *po = static_cast<uint16_t *>(p.part) + slot * kMlaDl;
    const float inv = l_all > 0.0f ? 1.0f / l_all : 0.0f;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d = db * 32 + 8 * g + 4 * hi;
            u32x2 w;
            w.x = epi_pack2<false>(acc_o[db][4 * g + 0] * inv, acc_o[db][4 * g + 1] * inv, false);
            w.y = epi_pack2<false>(acc_o[db][4 * g + 2] * inv, acc_o[db][4 * g + 3] * inv, false);
            *reinterpret_cast<u32x2 *>(po + d) = w;
        }
    }
    if (hi == 0) {
        float2 *ml = reinterpret_cast<float2 *>(static_cast<uint16_t *>(p.part) +
                                                p.B * p.H * p.splits * kMlaDl);
        ml[slot] = float2{m_run, l_all};
    }
}

// Combines the key ranges of (sequence, head) rows: with M the largest range
// maximum and w_s = 2^(m_s - M) l_s, O = sum_s w_s o_s / sum_s w_s, ranges
// added in order.  Wave r of a workgroup owns row 4 * blockIdx.x + r, lane t
// its output values 8t .. 8t + 7 (16-byte loads and stores).
constexpr int kCombineRows = 4;
__global__ void __launch_bounds__(64 * kCombineRows) mla_combine_kernel(MlaArgs p)
{
    const int64_t bh = (int64_t)blockIdx.x * kCombineRows + (threadIdx.x >> 6);
    if (bh >= p.B * p.H)
        return;
    const int d = (threadIdx.x & 63) * 8;
    const int S = p.splits;
    const uint16_t *part = static_cast<const uint16_t *>(p.part);
    const float2 *ml = reinterpret_cast<const float2 *>(part + p.B * p.H * S * kMlaDl) + bh * S;
    float M = -1.0e30f;
    for (int s = 0; s < S; ++s)
        M = __builtin_fmaxf(M, ml[s].x);
    float L = 0.0f;
    float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    for (int s = 0; s < S; ++s) {
        const float2 v = ml[s];
        const float w = __builtin_amdgcn_exp2f(v.x - M) * v.y;
        L += w;
        const u32x4 o = *reinterpret_cast<const u32x4 *>(part + (bh * S + s) * kMlaDl + d);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc[2 * j] += w * bits_to_float<false>((uint16_t)(o[j] & 0xffff));
            acc[2 * j + 1] += w * bits_to_float<false>((uint16_t)(o[j] >> 16));
        }
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    u32x4 out;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        out[j] = epi_pack2<false>(acc[2 * j] * inv, acc[2 * j + 1] * inv, false);
    __builtin_nontemporal_store(out, reinterpret_cast<u32x4 *>(p.O + bh * kMlaDl + d));
}

}  // namespace

hipError_t launch_attention(const AttnArgs &p, hipStream_t stream)
{
    // 0 / 1: four / eight waves on 32x32x16 products; 2 / 3: the same on
    // 16x16x32 products
    const int nw = (p.variant & 1) ? 8 : 4;
    if (p.variant >= 2) {
        if (p.D == 64)
            return nw == 8 ? launch_attn16<64, 8>(p, stream) : launch_attn16<64, 4>(p, stream);
        return nw == 8 ? launch_attn16<128, 8>(p, stream) : launch_attn16<128, 4>(p, stream);
    }
    if (p.D == 64)
        return nw == 8 ? launch_attn<64, 8>(p, stream) : launch_attn<64, 4>(p, stream);
    return nw == 8 ? launch_attn<128, 8>(p, stream) : launch_attn<128, 4>(p, stream);
}

}  // namespace tg

namespace tg {

hipError_t launch_mla_decode(const MlaArgs &p, hipStream_t stream)
{
    // the host has checked that the grid fits 2^31 workgroups
    const int64_t nhb = (p.H + kMlaHeadsPerBlock - 1) / kMlaHeadsPerBlock;
    const int64_t units = (p.B * p.splits + 7) / 8 * 8;
    hipLaunchKernelGGL(mla_decode_kernel, dim3((unsigned)(units * nhb)), dim3(64 * mla::NW), 0,
                       stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1)
        return e;
    hipLaunchKernelGGL(mla_combine_kernel,
                       dim3((unsigned)((p.B * p.H + kCombineRows - 1) / kCombineRows)),
                       dim3(64 * kCombineRows), 0, stream, p);
    return hipGetLastError();
}

}  // namespace tg
