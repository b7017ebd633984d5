// Internal interface between the host dispatcher (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tg {

// One strided-batched problem, sizes and strides in elements.  The host has
// validated it; every kernel masks its own edges, so any M, N, K >= 0 is safe
// for the layouts the ABI documents.  The epilogue adds bias[n] (N values
// shared by every row and batch; none when null) and applies the ReLU when
// `relu` is set.  Elements are bf16 when `bf16` is set (fp16 otherwise) and B
// is stored (N,K) when `b_nk` is set ((K,N) otherwise); the tile kernels take
// these two as template parameters and the launcher picks the instance.
struct GemmArgs {
    const uint16_t *A;
    const uint16_t *B;
    uint16_t *C;
    int64_t M, N, K;
    int64_t lda, ldb, ldc;
    int64_t sA, sB, sC;
    int64_t batch;
    const uint16_t *bias;
    int relu;
    int bf16;
    int b_nk;
};

// x if x > 0 else +0, NaN included: v_max_f32 against 0 returns the operand
// that is not a NaN.  Written out because the compiler puts a canonicalising
// max in front of fmaxf on values it cannot prove canonical (matrix-core
// results), one more VALU instruction per element.  The accumulations that
// feed it never produce -0 (their sums start from +0).
__device__ __forceinline__ float relu_f32(float x)
{
    float r;
    asm("v_max_f32 %0, 0, %1" : "=v"(r) : "v"(x));
    return r;
}

// Two outputs rounded to nearest even into fp16 (bf16 when BF16), low | high
// << 16, in one v_cvt_pk instruction; RELU applies relu_f32 first.
template <bool BF16, bool RELU>
__device__ __forceinline__ uint32_t pack2(float a, float b)
{
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    if constexpr (RELU) {
        a = relu_f32(a);
        b = relu_f32(b);
    }
    const f32x2_t v = {a, b};
    if constexpr (BF16)
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
    else
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}

// Epilogue of two outputs: ReLU (x if x > 0 else +0) when `relu`, then round
// to nearest even into fp16 (or bf16 when BF16); packed low | high << 16.
template <bool BF16 = false>
__device__ __forceinline__ uint32_t epi_pack2(float a, float b, bool relu)
{
    return relu ? pack2<BF16, true>(a, b) : pack2<BF16, false>(a, b);
}

// One element's bit pattern (fp16, or bf16 when BF16) as a float.
template <bool BF16 = false>
__device__ __forceinline__ float bits_to_float(uint16_t h)
{
    if constexpr (BF16)
        return __builtin_bit_cast(float, (uint32_t)h << 16);
    else
        return (float)__builtin_bit_cast(_Float16, h);
}

// bias[n .. n+3] as floats, from an 8-byte aligned address; zeros without a
// bias or past the last column (N is a multiple of 4 on the paths that use
// this, so a group of four columns is wholly inside or outside).
template <bool BF16 = false>
__device__ __forceinline__ void load_bias4(const uint16_t *bias, int64_t n, int64_t N,
                                           float (&b)[4])
{
    b[0] = b[1] = b[2] = b[3] = 0.0f;
    if (bias != nullptr && n < N) {
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
        const u32x2_t w = *reinterpret_cast<const u32x2_t *>(bias + n);
        b[0] = bits_to_float<BF16>((uint16_t)(w.x & 0xffff));
        b[1] = bits_to_float<BF16>((uint16_t)(w.x >> 16));
        b[2] = bits_to_float<BF16>((uint16_t)(w.y & 0xffff));
        b[3] = bits_to_float<BF16>((uint16_t)(w.y >> 16));
    }
}

// Tile coordinates of workgroup `pid` of a tilesM x tilesN grid.  The
// hardware hands consecutive workgroup ids to the eight XCDs in turn, and
// each XCD has its own L2; the ids are first renumbered so that each XCD
// receives a contiguous run of tiles, then that run is walked in panels of
// `groupM` tile rows, column by column, so that the tiles resident on one XCD
// at a time share A rows and B columns.  groupM <= 0 turns both off: plain
// row-major order of the workgroup ids (the ablation baseline).
__device__ __forceinline__ void tile_coords(int pid, int tilesM, int tilesN, int groupM, int &tm,
                                            int &tn)
{
    if (groupM <= 0) {
        tm = pid / tilesN;
        tn = pid - tm * tilesN;
        return;
    }
    const int T = tilesM * tilesN;
    const int q = T >> 3, r = T & 7;
    const int xcd = pid & 7, local = pid >> 3;
    const int id = (xcd < r) ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
    const int per_group = groupM * tilesN;
    const int g = id / per_group;
    const int first_m = g * groupM;
    const int gsz = min(tilesM - first_m, groupM);
    const int in = id - g * per_group;
    tm = first_m + in % gsz;
    tn = in / gsz;
}

// One weight-only int4 problem: C = act(A * W + bias), W(k, n) =
// S[n*lds + k/G] * q, q the signed nibble (k odd: high) of Wq[n*ldw + k/2]
// (ldw in bytes, the rest in elements).
struct W4Args {
    const uint16_t *A;
    const uint8_t *Wq;
    const uint16_t *S;
    uint16_t *C;
    const uint16_t *bias;
    int64_t M, N, K, G;
    int64_t lda, ldw, lds, ldc;
    int relu;
    int bf16;
    int scales_vec;   // set by launch_w4: scale rows 16-byte aligned, groups % 8 == 0
};
hipError_t launch_w4(const W4Args &p, hipStream_t stream);
hipError_t launch_w4_naive(const W4Args &p, hipStream_t stream);
bool w4_layout_ok(const W4Args &p);

// One attention forward: O = softmax(scale * Q K^T) V for every (batch, head)
// of Q (B, Sq, H, D), K and V (B, Sk, H, D), O (B, Sq, H, D), contiguous;
// D is 64 or 128; with `causal`, key j is visible to query i iff
// j <= i + (Sk - Sq).  Needs H <= 65535 and H * D < 2^24.
struct AttnArgs {
    const uint16_t *Q, *K, *V;
    uint16_t *O;
    int64_t B, Sq, Sk, H, Hkv, D;     // Hkv divides H
    float scale;
    int causal;
    int variant;      // 0: four waves per workgroup, 1: eight
    int64_t nqb, qb0; // query blocks in all, and the first one of this launch (set by the launcher)
};
hipError_t launch_attention(const AttnArgs &p, hipStream_t stream);

// Host helpers of the entry points (defined in api.cpp): the per-device
// architecture check (TG_OK or an error status), the current device's
// compute-unit count (0 when it cannot be had) and the record of the last
// path used.
int host_check_device();
int host_device_cus();
void host_set_last_path(int path);

// Every launcher enqueues on `stream` and returns hipGetLastError().  The
// tile launchers take the raster setting of tile_coords.
hipError_t launch_naive(const GemmArgs &p, hipStream_t stream);
hipError_t launch_generic(const GemmArgs &p, hipStream_t stream, int groupM);
hipError_t launch_tile128(const GemmArgs &p, hipStream_t stream, int groupM);
hipError_t launch_tile256(const GemmArgs &p, hipStream_t stream, int groupM);

// Direct-to-LDS pipelined kernels (aligned layouts only).  `cfg` selects the
// block tile / K tile / stage count; see gemm_dma.hip.
// Every configuration exists for fp16 with a (K,N) B (mode 0); bf16 and (N,K)
// B (mode bits 1 and 2) exist for the default configurations only.
constexpr int kDmaConfigs = 43;
hipError_t launch_dma_config(int cfg, const GemmArgs &p, hipStream_t stream, int groupM);
// Ragged layouts (see gemm_dma.hip): A as for the direct-to-LDS kernels
// (16-byte aligned rows, K a multiple of 8), B stored (K,N) with any 2-byte
// alignment and leading dimension, C likewise, N any.  cfg 0: 256x256x64
// tiles, cfg 1: 128x128x64.
hipError_t launch_ragged_config(int cfg, const GemmArgs &p, hipStream_t stream, int groupM);
bool dma_config_has_mode(int cfg, int mode);
// Skinny-M kernels (M <= 64, aligned layouts); `cfg` selects slice width,
// waves and stages; see gemm_skinny.hip.
// bf16 and (N,K) B exist for configurations 0 and 4 only.
constexpr int kSkinnyConfigs = 10;
hipError_t launch_skinny_config(int cfg, const GemmArgs &p, hipStream_t stream);
bool skinny_config_has_mode(int cfg, int mode);
bool skinny_layout_ok(const GemmArgs &p);
// Whether the leading dimensions fit the kernels' 32-bit buffer offsets.
bool dma_layout_ok(const GemmArgs &p);

}  // namespace tg
