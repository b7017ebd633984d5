// C ABI of the latent-attention decode: argument validation, the choice of
// key ranges per sequence and launch.  Declarations and the contract are in
// include/tg.h.
#include "tg.h"

#include <atomic>
#include <cstdint>

#include "tg_mla.h"

namespace {

constexpr int64_t kMaxDim = 0x7fffffff;
constexpr __int128 kMaxExtent = (__int128)1 << 62;
// forced number of key ranges (0: chosen from the sizes)
std::atomic<int> g_mla_splits{0};

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

extern "C" {

// Key ranges per sequence for the latent-attention decode: enough (sequence,
// range, head block) workgroups to give each of the 256 CUs one, with at
// least 8 tiles of 32 keys per range; then as many as the workspace holds.
constexpr int64_t kMlaTile = 32;
constexpr int64_t kMlaCUs = 256;

static int64_t mla_bytes_per_split(int64_t batch, int64_t heads)
{
    // per (sequence, head): 512 fp16 values and an fp32 (maximum, sum) pair
    return batch * heads * (tg::kMlaDl * 2 + 2 * (int64_t)sizeof(float));
}

static int64_t mla_splits(int64_t batch, int64_t heads, int64_t seq_k, int64_t workspace_bytes)
{
    const int64_t tiles = (seq_k + kMlaTile - 1) / kMlaTile;
    const int64_t nhb = (heads + tg::kMlaHeadsPerBlock - 1) / tg::kMlaHeadsPerBlock;
    const int64_t wgs = batch * nhb;
    int64_t s = g_mla_splits.load(std::memory_order_relaxed);
    if (s <= 0) {
        s = (kMlaCUs + wgs - 1) / wgs;
        if (s > tiles / 8)
            s = tiles / 8;
    }
    if (s > tiles)
        s = tiles;
    if (s > 1) {
        const int64_t per = mla_bytes_per_split(batch, heads);
        const int64_t fit = workspace_bytes / per;
        if (s > fit)
            s = fit;
    }
    return s < 1 ? 1 : s;
}

static bool mla_sizes_ok(int64_t batch, int64_t heads, int64_t seq_k)
{
    if (batch < 0 || heads < 0 || seq_k < 0 || batch > kMaxDim || heads > kMaxDim ||
        seq_k > kMaxDim)
        return false;
    const __int128 row = tg::kMlaDl + tg::kMlaDr;
    if ((__int128)batch * seq_k * row > kMaxExtent || (__int128)batch * heads * row > kMaxExtent)
        return false;
    // the grid holds (sequence, range) units rounded up to 8, times the head
    // blocks; ranges <= tiles <= 2^26
    const __int128 nhb = (heads + tg::kMlaHeadsPerBlock - 1) / tg::kMlaHeadsPerBlock;
    const __int128 tiles = (seq_k + kMlaTile - 1) / kMlaTile;
    const __int128 units = ((__int128)batch * (tiles > 0 ? tiles : 1) + 7) / 8 * 8;
    return units * nhb <= kMaxDim && (__int128)batch * heads <= kMaxDim;
}

int64_t tg_mla_decode_workspace_bytes(int64_t batch, int64_t heads, int64_t seq_k)
{
    if (!mla_sizes_ok(batch, heads, seq_k))
        return -1;
    if (batch == 0 || heads == 0 || seq_k == 0)
        return 0;
    const int64_t s = mla_splits(batch, heads, seq_k, INT64_MAX);
    return s > 1 ? s * mla_bytes_per_split(batch, heads) : 0;
}

int tg_mla_decode_f16(const void *Q, const void *KV, void *O, const int32_t *seqlens,
                      int64_t batch, int64_t heads, int64_t seq_k, float scale, void *workspace,
                      int64_t workspace_bytes, hipStream_t stream)
{
    if (!mla_sizes_ok(batch, heads, seq_k) || workspace_bytes < 0)
        return TG_ERR_INVALID_ARG;
    if (!(scale == scale) || scale > 3.0e38f || scale < -3.0e38f)
        return TG_ERR_INVALID_ARG;
    if (batch == 0 || heads == 0)
        return TG_OK;
    if (Q == nullptr || O == nullptr || (seq_k > 0 && KV == nullptr))
        return TG_ERR_INVALID_ARG;
    if (!aligned16(Q) || !aligned16(O) || (seq_k > 0 && !aligned16(KV)))
        return TG_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(seqlens) & 3) != 0)
        return TG_ERR_INVALID_ARG;
    if (workspace == nullptr)
        workspace_bytes = 0;
    if (workspace_bytes > 0 && !aligned16(workspace))
        return TG_ERR_INVALID_ARG;
    int st = tg::host_check_device();
    if (st != TG_OK)
        return st;
    tg::MlaArgs p;
    p.Q = static_cast<const uint16_t *>(Q);
    p.KV = static_cast<const uint16_t *>(KV);
    p.O = static_cast<uint16_t *>(O);
    p.seqlens = seqlens;
    p.part = workspace;
    p.B = batch; p.H = heads; p.Sk = seq_k;
    p.scale = scale;
    const int64_t s = mla_splits(batch, heads, seq_k, workspace_bytes);
    const int64_t tiles = (seq_k + kMlaTile - 1) / kMlaTile;
    const int64_t per = (tiles + s - 1) / s;                 // tiles per range
    p.keys_per_split = per * kMlaTile;
    p.splits = (int)(per > 0 ? (tiles + per - 1) / per : 1);   // no empty trailing range
    if (p.splits < 1)
        p.splits = 1;
    if (seq_k == 0) {
        p.splits = 1;
        p.keys_per_split = kMlaTile;
    }
    if (tg::launch_mla_decode(p, stream) != hipSuccess)
        return TG_ERR_HIP;
    tg::host_set_last_path(TG_PATH_MLA);
    return TG_OK;
}

int tg_set_mla_splits(int splits)
{
    if (splits < -1)
        return -2;
    return g_mla_splits.exchange(splits < 0 ? 0 : splits);
}

}  // extern "C"
