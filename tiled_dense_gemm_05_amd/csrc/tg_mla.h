// Internal interface of the latent-attention decode: entry point
// (mla_api.cpp) to kernels (attention.hip).
#pragma once

#include "tg_internal.h"

namespace tg {

// One latent-attention decode: for every sequence b and query head h,
// O[b][h][:512] = softmax_j(scale * Q[b][h][:] . KV[b][j][:]) KV[b][j][:512]
// over the first n_b cached rows (n_b = seqlens[b] clamped to [0, Sk], or Sk
// without seqlens).  Q (B, H, 576), KV (B, Sk, 576), O (B, H, 512) fp16,
// contiguous.  With splits > 1 the keys of a sequence are cut into `splits`
// ranges of keys_per_split (a multiple of 32) and each range writes a
// partial to `part`: B * H * splits rows of 512 fp16 values (the range's
// output divided by its own sum of exponentials), then B * H * splits
// fp32 (maximum, sum) pairs, which a second kernel combines.
struct MlaArgs {
    const uint16_t *Q, *KV;
    uint16_t *O;
    const int32_t *seqlens;
    void *part;
    int64_t B, H, Sk;
    float scale;
    int splits;
    int64_t keys_per_split;
};
constexpr int kMlaDl = 512, kMlaDr = 64, kMlaHeadsPerBlock = 128;
hipError_t launch_mla_decode(const MlaArgs &p, hipStream_t stream);

}  // namespace tg
