// C ABI of the library: argument validation, device checks, kernel-path
// selection and launch.  Declarations and the contract are in include/tg.h.
#include "tg.h"

#include <atomic>
#include <cstdlib>
#include <cstring>
#include <cstdint>

#include "tg_internal.h"

namespace {

std::atomic<int> g_forced_path{TG_PATH_AUTO};
std::atomic<int> g_last_path{TG_PATH_AUTO};
std::atomic<int> g_tile_variant{-1};

// Default direct-to-LDS configurations of the tile paths.
// 128x128x64, 4 stages, 8 waves (2x4, 64x32 wave tiles), 16x16x32 products
constexpr int kTile128Default = 38;
// 256x256x64, 2 stages, 8 waves (2 per SIMD), 16x16x32 products
constexpr int kTile256Default = 32;
// 256x128x64, 3 stages, 8 waves (2x4, 128x32 wave tiles), 16x16x32 products
constexpr int kTile256x128 = 41;
constexpr int kRagged256 = 2;       // the ragged kernel's 256x256 and 128x128 configurations
constexpr int kRagged128 = 3;       // (16x16x32 products)
// short K: persistent workgroups walking the list of 128x128 tiles, two per
// CU (39), or one per CU with a deeper ring when the list is very long (36)
constexpr int kStream128 = 39;
constexpr int kStream128Long = 36;
constexpr int kTile64 = 20;          // 64x64x64, 4 stages, two K groups: grids with few tiles
constexpr int kRegStaged128 = 100;   // register-staged kernels, kept for comparison
constexpr int kRegStaged256 = 101;
constexpr int kSkinnyDefault = 7;   // 64-column slices, 8 waves, 3 stages, non-temporal B
std::atomic<int> g_skinny_variant{-1};
// tile order of the tile kernels: panels of this many tile rows after the XCD
// renumbering (0: plain row-major order)
constexpr int kGroupMDefault = 8;
std::atomic<int> g_group_m{kGroupMDefault};
// attention kernel configuration (0: four waves per workgroup, 1: eight)
constexpr int kAttnDefault = 1;
std::atomic<int> g_attn_variant{kAttnDefault};

// Per-device architecture check, done once per device: 0 unknown, 1 gfx950,
// 2 something else.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_state[kMaxDevices];
std::atomic<int> g_cus[kMaxDevices];   // compute units per device (0: not yet asked)

constexpr int64_t kMaxDim = 0x7fffffff;
constexpr __int128 kMaxExtent = (__int128)1 << 62;

int check_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return TG_ERR_NO_DEVICE;
    }
    if (dev >= kMaxDevices)
        return TG_ERR_UNSUPPORTED_DEVICE;
    int st = g_arch_state[dev].load(std::memory_order_relaxed);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return TG_ERR_NO_DEVICE;
        }
        st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
        g_arch_state[dev].store(st, std::memory_order_relaxed);
    }
    return st == 1 ? TG_OK : TG_ERR_UNSUPPORTED_DEVICE;
}

// Largest element offset touched by a strided-batched operand, or -1 when it
// is too large to address.
__int128 extent(int64_t rows, int64_t cols, int64_t ld, int64_t stride, int64_t batch)
{
    if (rows == 0 || cols == 0 || batch == 0)
        return 0;
    __int128 s = stride < 0 ? -(__int128)stride : (__int128)stride;
    return (__int128)(batch - 1) * s + (__int128)(rows - 1) * ld + cols;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// b_nk: B is stored (N,K) (leading dimension over k) instead of (K,N).
int validate(const void *A, const void *B, const void *C, int64_t M, int64_t N, int64_t K,
             int64_t lda, int64_t ldb, int64_t ldc, int64_t sA, int64_t sB, int64_t sC,
             int64_t batch, bool b_nk)
{
    if (M < 0 || N < 0 || K < 0 || batch < 0)
        return TG_ERR_INVALID_ARG;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim || batch > kMaxDim)
        return TG_ERR_INVALID_ARG;
    const int64_t ldb_min = b_nk ? (K > 1 ? K : 1) : (N > 1 ? N : 1);
    if (lda < (K > 1 ? K : 1) || ldb < ldb_min || ldc < (N > 1 ? N : 1))
        return TG_ERR_INVALID_ARG;
    if (M == 0 || N == 0 || batch == 0)
        return TG_OK;
    if (C == nullptr)
        return TG_ERR_INVALID_ARG;
    if (K > 0 && (A == nullptr || B == nullptr))
        return TG_ERR_INVALID_ARG;
    // elements are 2 bytes: an odd address is not an element
    if (((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(B) |
          reinterpret_cast<uintptr_t>(C)) & 1) != 0)
        return TG_ERR_INVALID_ARG;
    const __int128 b_ext = b_nk ? extent(N, K, ldb, sB, batch) : extent(K, N, ldb, sB, batch);
    if (extent(M, K, lda, sA, batch) > kMaxExtent || b_ext > kMaxExtent ||
        extent(M, N, ldc, sC, batch) > kMaxExtent)
        return TG_ERR_INVALID_ARG;
    if (batch > 1) {
        const __int128 span = (__int128)(M - 1) * ldc + N;
        const __int128 s = sC < 0 ? -(__int128)sC : (__int128)sC;
        if (s < span)
            return TG_ERR_INVALID_ARG;
    }
    return TG_OK;
}

// Whether the 16-byte-chunk kernels can serve this call.
bool fast_layout(const tg::GemmArgs &p)
{
    if (!aligned16(p.A) || !aligned16(p.B) || !aligned16(p.C))
        return false;
    if (p.bias != nullptr && !aligned16(p.bias))
        return false;
    if ((p.lda | p.ldb | p.ldc | p.N | p.K) & 7)
        return false;
    if (p.batch > 1 && ((p.sA | p.sB | p.sC) & 7))
        return false;
    return p.K > 0 && tg::dma_layout_ok(p);
}

// Whether the ragged kernel can serve a call: A as for the 16-byte-chunk
// kernels, B stored (K,N); B, C and the bias at any 2-byte alignment.
bool ragged_layout(const tg::GemmArgs &p)
{
    if (p.b_nk || p.K <= 0 || !aligned16(p.A) || ((p.lda | p.K) & 7))
        return false;
    if (p.batch > 1 && (p.sA & 7))
        return false;
    return tg::dma_layout_ok(p);
}

// Rounds of one workgroup per compute unit for square tiles of side `t`.
int64_t tile_rounds(const tg::GemmArgs &p, int64_t tm, int64_t tn)
{
    const int64_t tiles = ((p.M + tm - 1) / tm) * ((p.N + tn - 1) / tn) * p.batch;
    return (tiles + 255) / 256;
}

// Both tile kernels (aligned and ragged) run one workgroup per CU, so a
// launch takes ceil(tiles / 256) rounds.  A round of 256x256 tiles does four
// times the work of a round of 128x128 tiles and takes about 2.6 times as
// long (measured from 2048^2 to 8192^2, K >= 1000); pick the cheaper one.
bool prefer_256(const tg::GemmArgs &p)
{
    return (double)tile_rounds(p, 256, 256) * 2.6 < (double)tile_rounds(p, 128, 128);
}

// A round of 256x128 tiles (twice the work of a 128x128 round) takes about
// 1.8 times as long (seven shapes from 2048x2048 to 6144x4096, K 1024 and
// 2048): worth it where it saves whole rounds, e.g. one round instead of two.
bool prefer_256x128(const tg::GemmArgs &p)
{
    return (double)tile_rounds(p, 256, 128) * 1.8 < (double)tile_rounds(p, 128, 128);
}

int choose_path(const tg::GemmArgs &p)
{
    if (!fast_layout(p))
        return (ragged_layout(p) && p.M > 64) ? TG_PATH_RAGGED : TG_PATH_GENERIC;
    if (p.M <= 64 && tg::skinny_layout_ok(p))
        return TG_PATH_SKINNY;
    // Short K (the batched shapes) stays on 128x128 tiles, walked by
    // persistent workgroups.
    if (p.K <= 64)
        return TG_PATH_TILE128;
    return prefer_256(p) ? TG_PATH_TILE256 : TG_PATH_TILE128;
}

int run(const void *A, const void *B, void *C, const void *bias, bool relu, bool bf16, bool b_nk,
        int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int64_t sA,
        int64_t sB, int64_t sC, int64_t batch, hipStream_t stream)
{
    int st = validate(A, B, C, M, N, K, lda, ldb, ldc, sA, sB, sC, batch, b_nk);
    if (st != TG_OK)
        return st;
    if ((reinterpret_cast<uintptr_t>(bias) & 1) != 0)
        return TG_ERR_INVALID_ARG;
    if (M == 0 || N == 0 || batch == 0)
        return TG_OK;
    st = check_device();
    if (st != TG_OK)
        return st;

    tg::GemmArgs p;
    p.A = static_cast<const uint16_t *>(A);
    p.B = static_cast<const uint16_t *>(B);
    p.C = static_cast<uint16_t *>(C);
    p.M = M; p.N = N; p.K = K;
    p.lda = lda; p.ldb = ldb; p.ldc = ldc;
    p.sA = batch > 1 ? sA : 0;
    p.sB = batch > 1 ? sB : 0;
    p.sC = batch > 1 ? sC : 0;
    p.batch = batch;
    p.bias = static_cast<const uint16_t *>(bias);
    p.relu = relu ? 1 : 0;
    p.bf16 = bf16 ? 1 : 0;
    p.b_nk = b_nk ? 1 : 0;
    const int mode = p.bf16 | (p.b_nk << 1);

    int path = g_forced_path.load(std::memory_order_relaxed);
    if (path == TG_PATH_AUTO || path == TG_PATH_W4 || path == TG_PATH_ATTENTION ||
        path == TG_PATH_MLA)
        path = choose_path(p);
    else if (path == TG_PATH_RAGGED && !ragged_layout(p))
        path = TG_PATH_GENERIC;
    else if (path != TG_PATH_NAIVE && path != TG_PATH_GENERIC && path != TG_PATH_RAGGED &&
             !fast_layout(p))
        path = TG_PATH_GENERIC;
    else if (path == TG_PATH_SKINNY && !tg::skinny_layout_ok(p))
        path = TG_PATH_TILE128;

    hipError_t e;
    switch (path) {
    case TG_PATH_NAIVE: e = tg::launch_naive(p, stream); break;
    case TG_PATH_TILE128:
    case TG_PATH_TILE256: {
        int v = g_tile_variant.load(std::memory_order_relaxed);
        // bf16 and (N,K) B exist in the default configurations only
        if (v >= 0 && (v >= tg::kDmaConfigs ? mode != 0 : !tg::dma_config_has_mode(v, mode)))
            v = -1;
        if (v < 0) {
            const int64_t tiles128 = ((p.M + 127) / 128) * ((p.N + 127) / 128) * p.batch;
            // short K: persistent workgroups, so that loads, products and
            // stores of different tiles overlap
            const int cus = tg::host_device_cus();
            v = path == TG_PATH_TILE256            ? kTile256Default
                : p.K <= 64 && tiles128 >= 8 * cus ? kStream128Long
                : p.K <= 64                        ? kStream128
                : tiles128 < 128                   ? kTile64
                : prefer_256x128(p)                ? kTile256x128
                                                   : kTile128Default;
        }
        const int gm = g_group_m.load(std::memory_order_relaxed);
        if (v == kRegStaged128)
            e = tg::launch_tile128(p, stream, gm);
        else if (v == kRegStaged256)
            e = tg::launch_tile256(p, stream, gm);
        else
            e = tg::launch_dma_config(v, p, stream, gm);
        break;
    }
    case TG_PATH_RAGGED: {
        // tg_set_tile_variant 0 / 1 forces the 256x256 / 128x128 configuration
        // with 32x32x16 products, 2 / 3 the same with 16x16x32 products
        int v = g_tile_variant.load(std::memory_order_relaxed);
        if (v < 0 || v > 3)
            v = prefer_256(p) ? kRagged256 : kRagged128;
        e = tg::launch_ragged_config(v, p, stream, g_group_m.load(std::memory_order_relaxed));
        break;
    }
    case TG_PATH_SKINNY: {
        int v = g_skinny_variant.load(std::memory_order_relaxed);
        if (v < 0 || !tg::skinny_config_has_mode(v, mode))
            v = kSkinnyDefault;
        e = tg::launch_skinny_config(v, p, stream);
        break;
    }
    default:
        e = tg::launch_generic(p, stream, g_group_m.load(std::memory_order_relaxed));
        path = TG_PATH_GENERIC;
        break;
    }
    if (e != hipSuccess)
        return TG_ERR_HIP;
    g_last_path.store(path, std::memory_order_relaxed);
    return TG_OK;
}

}  // namespace

namespace tg {
int host_check_device() { return check_device(); }
int host_device_cus()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return 0;
    }
    int n = g_cus[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
            (void)hipGetLastError();
            return 0;
        }
        g_cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}
void host_set_last_path(int path) { g_last_path.store(path, std::memory_order_relaxed); }
}  // namespace tg

extern "C" {

int tg_gemm_relu_f16(const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K,
                     int64_t lda, int64_t ldb, int64_t ldc, hipStream_t stream)
{
    return run(A, B, C, nullptr, true, false, false, M, N, K, lda, ldb, ldc, 0, 0, 0, 1, stream);
}

int tg_gemm_relu_f16_strided_batched(const void *A, const void *B, void *C, int64_t M, int64_t N,
                                     int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                                     int64_t strideA, int64_t strideB, int64_t strideC,
                                     int64_t batch, hipStream_t stream)
{
    return run(A, B, C, nullptr, true, false, false, M, N, K, lda, ldb, ldc, strideA, strideB,
               strideC, batch, stream);
}

int tg_gemm_ex(int dtype, int b_layout, int activation, const void *A, const void *B, void *C,
               const void *bias, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
               int64_t ldc, int64_t strideA, int64_t strideB, int64_t strideC, int64_t batch,
               hipStream_t stream)
{
    if (dtype != TG_DTYPE_F16 && dtype != TG_DTYPE_BF16)
        return TG_ERR_INVALID_ARG;
    if (b_layout != TG_B_KN && b_layout != TG_B_NK)
        return TG_ERR_INVALID_ARG;
    if (activation != TG_ACT_NONE && activation != TG_ACT_RELU)
        return TG_ERR_INVALID_ARG;
    return run(A, B, C, bias, activation == TG_ACT_RELU, dtype == TG_DTYPE_BF16,
               b_layout == TG_B_NK, M, N, K, lda, ldb, ldc, strideA, strideB, strideC, batch,
               stream);
}

int tg_gemm_w4(int dtype, int activation, const void *A, const void *Wq, const void *scales,
               void *C, const void *bias, int64_t M, int64_t N, int64_t K, int64_t group_size,
               int64_t lda, int64_t ldw, int64_t lds, int64_t ldc, hipStream_t stream)
{
    if (dtype != TG_DTYPE_F16 && dtype != TG_DTYPE_BF16)
        return TG_ERR_INVALID_ARG;
    if (activation != TG_ACT_NONE && activation != TG_ACT_RELU)
        return TG_ERR_INVALID_ARG;
    if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim)
        return TG_ERR_INVALID_ARG;
    if (group_size <= 0 || group_size > kMaxDim || K % group_size != 0)
        return TG_ERR_INVALID_ARG;
    const int64_t groups = K / group_size;
    if (lda < (K > 1 ? K : 1) || ldw < ((K + 1) / 2 > 1 ? (K + 1) / 2 : 1) ||
        lds < (groups > 1 ? groups : 1) || ldc < (N > 1 ? N : 1))
        return TG_ERR_INVALID_ARG;
    if (M == 0 || N == 0)
        return TG_OK;
    if (C == nullptr || (K > 0 && (A == nullptr || Wq == nullptr || scales == nullptr)))
        return TG_ERR_INVALID_ARG;
    if (extent(M, K, lda, 0, 1) > kMaxExtent || extent(N, (K + 1) / 2, ldw, 0, 1) > kMaxExtent ||
        extent(N, groups, lds, 0, 1) > kMaxExtent || extent(M, N, ldc, 0, 1) > kMaxExtent)
        return TG_ERR_INVALID_ARG;
    int st = check_device();
    if (st != TG_OK)
        return st;

    tg::W4Args p;
    p.A = static_cast<const uint16_t *>(A);
    p.Wq = static_cast<const uint8_t *>(Wq);
    p.S = static_cast<const uint16_t *>(scales);
    p.C = static_cast<uint16_t *>(C);
    p.bias = static_cast<const uint16_t *>(bias);
    p.M = M; p.N = N; p.K = K; p.G = group_size;
    p.lda = lda; p.ldw = ldw; p.lds = lds; p.ldc = ldc;
    p.relu = activation == TG_ACT_RELU ? 1 : 0;
    p.bf16 = dtype == TG_DTYPE_BF16 ? 1 : 0;

    const int forced = g_forced_path.load(std::memory_order_relaxed);
    const bool plain = forced == TG_PATH_NAIVE || forced == TG_PATH_GENERIC || !tg::w4_layout_ok(p);
    const hipError_t e = plain ? tg::launch_w4_naive(p, stream) : tg::launch_w4(p, stream);
    if (e != hipSuccess)
        return TG_ERR_HIP;
    g_last_path.store(plain ? TG_PATH_NAIVE : TG_PATH_W4, std::memory_order_relaxed);
    return TG_OK;
}

int tg_attention_fwd_f16_gqa(const void *Q, const void *K, const void *V, void *O,
                             int64_t batch, int64_t seq_q, int64_t seq_k, int64_t heads,
                             int64_t kv_heads, int64_t head_dim, float scale, int causal,
                             hipStream_t stream)
{
    if (batch < 0 || seq_q < 0 || seq_k < 0 || heads < 0 || kv_heads < 0 || batch > kMaxDim ||
        seq_q > kMaxDim || seq_k > kMaxDim || heads > kMaxDim)
        return TG_ERR_INVALID_ARG;
    if (heads > 0 && (kv_heads == 0 || heads % kv_heads != 0))
        return TG_ERR_INVALID_ARG;
    if ((__int128)batch * kv_heads > kMaxDim)   // (batch, key/value head) pairs run along grid x
        return TG_ERR_INVALID_ARG;
    if (head_dim != 64 && head_dim != 128)
        return TG_ERR_INVALID_ARG;
    if (!(scale == scale) || scale > 3.0e38f || scale < -3.0e38f || (causal != 0 && causal != 1))
        return TG_ERR_INVALID_ARG;
    if (heads * head_dim >= (1 << 24))
        return TG_ERR_INVALID_ARG;
    if (batch == 0 || seq_q == 0 || heads == 0)
        return TG_OK;
    if ((__int128)seq_q * (heads / kv_heads) > kMaxDim)   // query rows of one key/value head
        return TG_ERR_INVALID_ARG;
    if (Q == nullptr || O == nullptr || (seq_k > 0 && (K == nullptr || V == nullptr)))
        return TG_ERR_INVALID_ARG;
    if (!aligned16(Q) || !aligned16(O) || (seq_k > 0 && (!aligned16(K) || !aligned16(V))))
        return TG_ERR_INVALID_ARG;
    const __int128 rows_q = (__int128)batch * seq_q * heads * head_dim;
    const __int128 rows_k = (__int128)batch * seq_k * kv_heads * head_dim;
    if (rows_q > kMaxExtent || rows_k > kMaxExtent)
        return TG_ERR_INVALID_ARG;
    int st = check_device();
    if (st != TG_OK)
        return st;
    tg::AttnArgs p;
    p.Q = static_cast<const uint16_t *>(Q);
    p.K = static_cast<const uint16_t *>(K);
    p.V = static_cast<const uint16_t *>(V);
    p.O = static_cast<uint16_t *>(O);
    p.B = batch; p.Sq = seq_q; p.Sk = seq_k; p.H = heads; p.Hkv = kv_heads; p.D = head_dim;
    p.scale = scale;
    p.causal = causal;
    p.variant = g_attn_variant.load(std::memory_order_relaxed);
    if (tg::launch_attention(p, stream) != hipSuccess)
        return TG_ERR_HIP;
    g_last_path.store(TG_PATH_ATTENTION, std::memory_order_relaxed);
    return TG_OK;
}

int tg_attention_fwd_f16(const void *Q, const void *K, const void *V, void *O, int64_t batch,
                         int64_t seq_q, int64_t seq_k, int64_t heads, int64_t head_dim,
                         float scale, int causal, hipStream_t stream)
{
    return tg_attention_fwd_f16_gqa(Q, K, V, O, batch, seq_q, seq_k, heads, heads, head_dim,
                                    scale, causal, stream);
}


const char *tg_status_string(int status)
{
    switch (status) {
    case TG_OK: return "TG_OK";
    case TG_ERR_INVALID_ARG: return "TG_ERR_INVALID_ARG: invalid size, leading dimension, stride or pointer";
    case TG_ERR_NO_DEVICE: return "TG_ERR_NO_DEVICE: no usable HIP device";
    case TG_ERR_UNSUPPORTED_DEVICE: return "TG_ERR_UNSUPPORTED_DEVICE: the current device is not gfx950";
    case TG_ERR_HIP: return "TG_ERR_HIP: a HIP call or kernel launch failed";
    default: return "unknown tg_status";
    }
}

int tg_set_path(int path)
{
    if (path < 0 || path >= TG_PATH_COUNT)
        return -1;
    return g_forced_path.exchange(path);
}

int tg_last_path(void) { return g_last_path.load(std::memory_order_relaxed); }

int tg_set_skinny_variant(int variant)
{
    if (!(variant == -1 || (variant >= 0 && variant < tg::kSkinnyConfigs)))
        return -2;
    return g_skinny_variant.exchange(variant);
}

int tg_set_tile_variant(int variant)
{
    if (!(variant == -1 || (variant >= 0 && variant < tg::kDmaConfigs) ||
          variant == kRegStaged128 || variant == kRegStaged256))
        return -2;
    return g_tile_variant.exchange(variant);
}

int tg_set_attention_variant(int variant)
{
    if (variant == -1)
        variant = kAttnDefault;
    if (variant < 0 || variant > 3)
        return -2;
    return g_attn_variant.exchange(variant);
}

int tg_set_raster(int group_m)
{
    if (group_m == -1)
        group_m = kGroupMDefault;
    if (group_m < 0 || group_m > 64)
        return -2;
    return g_group_m.exchange(group_m);
}

const char *tg_path_name(int path)
{
    switch (path) {
    case TG_PATH_AUTO: return "auto";
    case TG_PATH_NAIVE: return "naive";
    case TG_PATH_GENERIC: return "generic";
    case TG_PATH_TILE128: return "tile128";
    case TG_PATH_TILE256: return "tile256";
    case TG_PATH_SKINNY: return "skinny";
    case TG_PATH_W4: return "w4";
    case TG_PATH_ATTENTION: return "attention";
    case TG_PATH_MLA: return "mla";
    case TG_PATH_RAGGED: return "ragged";
    default: return "unknown";
    }
}

}  // extern "C"
