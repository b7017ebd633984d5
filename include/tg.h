/*
 * tg.h -- C ABI of the MI355X (gfx950) fused fp16 GEMM + ReLU library.
 *
 * The operation is the GEMM+ReLU tile program of the "TileLang paper reading"
 * page (hotelren.com), section 2: A is an (M,K) fp16 tensor, B a (K,N) fp16
 * tensor, the product is accumulated in an fp32 fragment that starts at zero,
 * is clamped below at zero, and is stored into the (M,N) fp16 output.  The
 * "tilelang practitioner's notes" page (dpshk.com), sections 3.2-3.3, adds
 * that K is a serial accumulation in a type wider than fp16 and that the
 * compiled kernel is called on device tensors and may run asynchronously.
 *
 *   C[i*ldc + j] = fp16_rne( max(0, sum_k A[i*lda + k] * B[k*ldb + j]) )
 *
 * with the sum in fp32 (order of summation unspecified), ReLU mapping every
 * value that is not > 0 to +0.0, and the fp32 -> fp16 conversion rounding to
 * nearest, ties to even, with subnormals kept.
 *
 * Conventions shared by every entry point:
 *  - Elements are IEEE binary16; A, B, C are DEVICE pointers (void* so that a
 *    framework's data pointer passes straight through).  All matrices are
 *    row-major with leading dimensions in elements.
 *  - Ownership: the caller owns A, B and C.  The library allocates nothing per
 *    call and keeps no pointer after it returns.
 *  - Asynchrony: work is enqueued on `stream` (0 = the default stream) and the
 *    call returns without waiting; the buffers must stay alive until the
 *    stream reaches the call.  Calls are reentrant.
 *  - Errors are returned, never thrown.  Argument errors are detected before
 *    any HIP call.  M = 0, N = 0 or batch = 0 is a no-op returning TG_OK;
 *    K = 0 writes +0.0 to the whole M x N window (the empty sum).
 *  - Only the M x N window of C is written; the ldc padding is untouched.
 *    C overlapping A or B is undefined.
 *  - Any 2-byte-aligned pointer and any leading dimension are accepted;
 *    16-byte-aligned pointers with leading dimensions and N, K that are
 *    multiples of 8 take the fastest kernels.
 *  - Results are deterministic: the same inputs, shape and device give the
 *    same bits on every call (no floating-point atomics).
 *  - Calls only enqueue kernels on `stream` (no allocation, copy, memset or
 *    synchronisation; besides the launches they read the current device, its
 *    architecture once per device, and the launch status), so they can be
 *    captured into a HIP graph and replayed.
 */
#ifndef TG_H
#define TG_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TG_OK = 0,
    TG_ERR_INVALID_ARG = 1,         /* bad size, leading dimension, stride or null pointer */
    TG_ERR_NO_DEVICE = 2,           /* no HIP device is usable from this process */
    TG_ERR_UNSUPPORTED_DEVICE = 3,  /* the current device is not gfx950 */
    TG_ERR_HIP = 4                  /* a HIP runtime call or kernel launch failed */
} tg_status;

/*
 * C = ReLU(A * B) for one matrix.
 *   A      (M,K) fp16, row-major, leading dimension lda >= max(1,K)
 *   B      (K,N) fp16, row-major, leading dimension ldb >= max(1,N)
 *   C      (M,N) fp16, row-major, leading dimension ldc >= max(1,N)
 *   M,N,K  sizes, each in [0, 2^31 - 1]
 * A and B may be NULL only when the matrix they hold is empty (M*K == 0,
 * K*N == 0); C may be NULL only when M*N == 0.
 * Returns a tg_status.
 */
int tg_gemm_relu_f16(const void *A, const void *B, void *C,
                     int64_t M, int64_t N, int64_t K,
                     int64_t lda, int64_t ldb, int64_t ldc,
                     hipStream_t stream);

/*
 * Strided-batched form: for b in [0, batch),
 *   C + b*strideC = ReLU((A + b*strideA) * (B + b*strideB))
 * with each slice laid out as in tg_gemm_relu_f16.  Strides are in elements;
 * strideA or strideB may be 0 (the operand is shared by every slice).  When
 * batch > 1 the C slices must not overlap: |strideC| >= (M-1)*ldc + N.
 * batch is in [0, 2^31 - 1].
 */
int tg_gemm_relu_f16_strided_batched(const void *A, const void *B, void *C,
                                     int64_t M, int64_t N, int64_t K,
                                     int64_t lda, int64_t ldb, int64_t ldc,
                                     int64_t strideA, int64_t strideB, int64_t strideC,
                                     int64_t batch, hipStream_t stream);

/*
 * Extended form: C = act(A * B + bias), strided-batched, with a choice of
 * element type and B layout.
 *
 * The bias-add and activation are the epilogue of the same tile program (the
 * "TileLang paper reading" page, section 2, whose epilogue is the ReLU), with
 * the neighbouring element-wise operator fused into the GEMM as section 2.2 of
 * the "tilelang practitioner's notes" page describes for fused kernels:
 *
 *   C[b][i*ldc + j] = rne( act( sum_k A[b][i*lda + k] * B(b, k, j) + bias[j] ) )
 *
 *   dtype       TG_DTYPE_F16: A, B, bias and C are IEEE binary16;
 *               TG_DTYPE_BF16: they are bfloat16 (8 exponent, 7 stored
 *               significand bits), stored with round to nearest even.
 *   b_layout    TG_B_KN: B is (K,N) row-major, B(b,k,j) = B[b*strideB + k*ldb + j],
 *               ldb >= max(1,N);
 *               TG_B_NK: B is (N,K) row-major (a transposed weight, the (BN,BK)
 *               B tile of section 3.2 of the practitioner's notes page),
 *               B(b,k,j) = B[b*strideB + j*ldb + k], ldb >= max(1,K).
 *   activation  TG_ACT_NONE: act(x) = x;  TG_ACT_RELU: x if x > 0 else +0.0.
 *   bias        DEVICE pointer to N elements shared by every row and batch
 *               slice, or NULL for no bias (the sum alone).  The bias is added
 *               to the fp32 sum before the activation, in fp32.
 * Everything else (sizes, leading dimensions, strides, batch, NULL rules,
 * errors, asynchrony, determinism) is as for tg_gemm_relu_f16_strided_batched;
 * batch = 1 is the single-matrix form (strides ignored).  With
 * TG_ACT_RELU and a NULL bias this is exactly tg_gemm_relu_f16[_strided_batched].
 * An unknown dtype, layout or activation returns TG_ERR_INVALID_ARG.  A bias
 * that is not 16-byte aligned takes the any-alignment kernel.  The tuning
 * knobs tg_set_tile_variant / tg_set_skinny_variant apply to bf16 and (N,K) B
 * only for the default configurations (others fall back to the default).
 */
enum { TG_DTYPE_F16 = 0, TG_DTYPE_BF16 = 1 };
enum { TG_B_KN = 0, TG_B_NK = 1 };
enum { TG_ACT_NONE = 0, TG_ACT_RELU = 1 };
int tg_gemm_ex(int dtype, int b_layout, int activation,
               const void *A, const void *B, void *C, const void *bias,
               int64_t M, int64_t N, int64_t K,
               int64_t lda, int64_t ldb, int64_t ldc,
               int64_t strideA, int64_t strideB, int64_t strideC,
               int64_t batch, hipStream_t stream);

/*
 * Weight-only int4 GEMM (W_INT4 / A_FP16 or A_BF16): the dequantize GEMM that
 * section 5 of the "TileLang paper reading" page measures, with the
 * epilogue of tg_gemm_ex:
 *
 *   C[i*ldc + j] = rne( act( sum_k A[i*lda + k] * W(k, j) + bias[j] ) )
 *   W(k, j)      = scales[j*lds + k/group_size] * q(j, k)   (exactly)
 *   q(j, k)      = the signed 4-bit value (two's complement, -8..7) in bits
 *                  4*(k%2) .. 4*(k%2)+3 of the byte Wq[j*ldw + k/2]
 *
 * i.e. the weight is stored (N,K) like a linear layer's, two values per byte
 * along k (even k in the low nibble), ldw in BYTES (>= ceil(K/2)); one scale
 * of the element type per group of group_size consecutive k of each weight
 * row, row j at scales + j*lds elements (lds >= K/group_size).  The pages
 * name the configuration but not its format: this layout is the reading
 * taken.  A (M,K), bias (N values or NULL) and C (M,N) have element type
 * dtype (TG_DTYPE_F16 or TG_DTYPE_BF16); A, Wq, scales, bias and C are DEVICE
 * pointers.  activation is TG_ACT_NONE or TG_ACT_RELU.  The products of A with
 * q are exact; each group's sum is formed in fp32 and multiplied by its
 * scale in fp32.
 *
 * Requirements: sizes in [0, 2^31 - 1]; group_size > 0 and K % group_size
 * == 0; lda >= max(1,K), ldc >= max(1,N).  Fast kernel (any M; rows of A
 * beyond 64 stream the weight once per 64 rows): A and Wq 16-byte aligned,
 * lda % 8 == 0, ldw % 16 == 0, group_size a multiple of 32, C and bias
 * 8-byte aligned, ldc and N multiples of 4, and (K/group_size) * 128 bytes of
 * scales per 64 weight rows within the LDS the kernel leaves free (e.g.
 * K/group_size <= 512 for M <= 16); other calls take a plain one-thread-per-
 * output kernel.  Errors, asynchrony and determinism as for the other entry
 * points; M = 0 or N = 0 is a no-op, K = 0 writes act(bias) (or +0).
 */
int tg_gemm_w4(int dtype, int activation, const void *A, const void *Wq, const void *scales,
               void *C, const void *bias, int64_t M, int64_t N, int64_t K, int64_t group_size,
               int64_t lda, int64_t ldw, int64_t lds, int64_t ldc, hipStream_t stream);

/*
 * Fused attention forward (softmax attention), fp16:
 *
 *   O[b][i][h][:] = sum_j p_ij V[b][j][h][:],
 *   p_ij = exp(s_ij - max_j s_ij) / sum_j exp(s_ij - max_j s_ij),
 *   s_ij = scale * sum_d Q[b][i][h][d] K[b][j][h][d]
 *
 * over the keys j visible to query i: all j < seq_k, or with causal = 1 only
 * j <= i + (seq_k - seq_q) (a query with no visible key gets O = 0).  The
 * pages name fused attention kernels (FlashAttention, MLA decode) among the
 * tile programs they measure ("TileLang paper reading" page, section 5; the
 * "80-line MLA article" page) without their formulas: this is the standard
 * definition, computed in one pass with a running maximum.
 *   Q, O  (batch, seq_q, heads, head_dim) fp16, contiguous, DEVICE pointers
 *   K, V  (batch, seq_k, heads, head_dim) fp16, contiguous, DEVICE pointers
 *   head_dim 64 or 128; heads * head_dim < 2^24 and batch * heads < 2^31;
 *   all four pointers 16-byte aligned; scale finite (e.g. 1/sqrt(head_dim)).
 * Scores and sums are fp32, probabilities enter the value product as fp16
 * (the products with V are accumulated in fp32).  Errors, asynchrony and
 * determinism as for the other entry points; batch, seq_q or heads = 0 is a
 * no-op; seq_k = 0 writes zeros.
 */
int tg_attention_fwd_f16(const void *Q, const void *K, const void *V, void *O,
                         int64_t batch, int64_t seq_q, int64_t seq_k, int64_t heads,
                         int64_t head_dim, float scale, int causal, hipStream_t stream);

/*
 * The same with grouped-query heads: K and V hold kv_heads heads, laid out
 * (batch, seq_k, kv_heads, head_dim), and query head h reads key/value head
 * h / (heads / kv_heads) (kv_heads = heads: tg_attention_fwd_f16; 1:
 * multi-query attention).  The standard grouped-query form of the definition
 * above (the pages' MLA decode shares one latent key/value across all query
 * heads in the same way).  kv_heads must divide heads; batch * kv_heads and
 * seq_q * (heads / kv_heads) must stay below 2^31.  The query heads of a
 * group run in the same workgroups, so every K/V tile is read once per group
 * of heads.  Otherwise as tg_attention_fwd_f16.
 */
int tg_attention_fwd_f16_gqa(const void *Q, const void *K, const void *V, void *O,
                             int64_t batch, int64_t seq_q, int64_t seq_k, int64_t heads,
                             int64_t kv_heads, int64_t head_dim, float scale, int causal,
                             hipStream_t stream);

/*
 * The skinny GEMM+ReLU split along K (the split-K form of the decode-shaped
 * path, kept as an alternative to tg_gemm_relu_f16's single-pass skinny
 * kernel for comparison): C = ReLU(A B) exactly as tg_gemm_relu_f16, computed
 * as `splits` chunks of K (whole 32-k steps) whose fp32 partial sums are
 * written to the caller's workspace and then added in chunk order, before
 * the ReLU, by a second kernel (deterministic).  The same ReLU-after-the-
 * full-sum rule as the tile program: K accumulates serially.
 *   M <= 64; A, B, C, workspace DEVICE pointers, 16-byte aligned; N, K,
 *   lda, ldb, ldc multiples of 8; 1 <= splits <= 65535 and, for K > 0,
 *   splits <= ceil(K / 32); workspace_bytes >= splits * M * N * 4
 *   (tg_gemm_splitk_workspace_bytes).  The workspace is scratch for this
 *   call only (calls that may overlap need their own).  M = 0 or N = 0 is a
 *   no-op; K = 0 writes zeros.  Errors and asynchrony as tg_gemm_relu_f16.
 */
int tg_gemm_relu_f16_splitk(const void *A, const void *B, void *C, int64_t M, int64_t N,
                            int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int64_t splits,
                            void *workspace, int64_t workspace_bytes, hipStream_t stream);

/* Workspace bytes tg_gemm_relu_f16_splitk needs, or -1 for sizes it rejects. */
int64_t tg_gemm_splitk_workspace_bytes(int64_t M, int64_t N, int64_t splits);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * tg_gemm_relu_f16_splitk with its fp32 partial sums in a scratch array the
 * library keeps on each device (TG_SPLITK_NOALLOC_SCRATCH_BYTES = 16 MiB,
 * held from the first call on that device until the process ends) instead
 * of a caller workspace.  Same arguments, results (bit for bit), errors and
 * asynchrony as tg_gemm_relu_f16_splitk without the workspace; in addition
 * splits * M * N * 4 > TG_SPLITK_NOALLOC_SCRATCH_BYTES returns
 * TG_ERR_INVALID_ARG before any GPU work.  The call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine).  Every call on a device
 * shares that device's array: calls that may overlap on one device (other
 * streams, other host threads) race on it and must be serialized by the
 * caller.  Every partial sum is written before it is read, so the previous
 * call's contents need no clearing.
 */
#define TG_SPLITK_NOALLOC_SCRATCH_BYTES (16ll << 20)
int tg_gemm_relu_f16_splitk_noalloc(const void *A, const void *B, void *C, int64_t M, int64_t N,
                                    int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                                    int64_t splits, hipStream_t stream);

/*
 * Latent-attention decode (MLA), fp16: one query per sequence, every query
 * head reading one shared cached row per token of 512 + 64 values (the head
 * size the pages give for the MLA decode they measure: "TileLang paper
 * reading" page, section 5; "80-line MLA article" page, sections 1-2).  The
 * pages give no formula; this is the absorbed form, written out:
 *
 *   s_j = scale * sum_{d < 576} Q[b][h][d] KV[b][j][d]        (j < n_b)
 *   O[b][h][d] = sum_j softmax(s)_j KV[b][j][d]              (d < 512)
 *
 * i.e. the first 512 values of a cached row are key and value, the last 64
 * a rotary key part, and n_b = seqlens[b] (every seq_k tokens when seqlens
 * is NULL; entries are clamped to [0, seq_k] on the device); n_b = 0 gives
 * O = 0.
 *   Q   (batch, heads, 576) fp16, contiguous, DEVICE pointer, 16-byte aligned
 *   KV  (batch, seq_k, 576) fp16, contiguous, DEVICE pointer, 16-byte aligned
 *   O   (batch, heads, 512) fp16, contiguous, DEVICE pointer, 16-byte aligned
 *   seqlens  NULL or batch int32 values, DEVICE pointer
 *   workspace  NULL or a DEVICE buffer of workspace_bytes (16-byte aligned),
 *     owned by the caller, used as scratch by this call only (it must not be
 *     shared by calls that may overlap).  With fewer sequences than the chip
 *     has compute units the keys of each sequence are split into ranges whose
 *     partial results live there (each range's output divided by its own
 *     sum, as fp16, with its fp32 maximum and sum: 1032 bytes per sequence,
 *     head and range); tg_mla_decode_workspace_bytes gives the size the call
 *     would use.  A smaller (or no) workspace is accepted
 *     and only lowers the number of ranges (results stay within the same
 *     accuracy; the same workspace size gives the same bits).
 * Scores and sums are fp32, probabilities enter the value product as fp16.
 * scale must be finite (the absorbed form uses 1/sqrt(192)).  batch or
 * heads = 0 is a no-op.  Errors, asynchrony and determinism as for the other
 * entry points.
 */
int tg_mla_decode_f16(const void *Q, const void *KV, void *O, const int32_t *seqlens,
                      int64_t batch, int64_t heads, int64_t seq_k, float scale,
                      void *workspace, int64_t workspace_bytes, hipStream_t stream);

/*
 * Workspace bytes tg_mla_decode_f16 uses for these sizes (0: none needed),
 * or -1 for sizes it rejects.  Host-only: no HIP call.
 */
int64_t tg_mla_decode_workspace_bytes(int64_t batch, int64_t heads, int64_t seq_k);

/*
 * Test knob: the number of key ranges per sequence tg_mla_decode_f16 uses
 * (0 or -1: chosen from the sizes, the default; still capped by the number
 * of 32-key tiles and the workspace).  Returns the previous setting (0 for
 * the default), or -2 for a value below -1.
 */
int tg_set_mla_splits(int splits);

/* A static, human-readable name for a tg_status value. */
const char *tg_status_string(int status);

/*
 * Kernel-path selection, for tests and benchmarks.  TG_PATH_AUTO (the default)
 * lets the library pick from the shape and alignment; any other value forces
 * that path for every later call in the process (a path that cannot serve a
 * call's alignment falls back to TG_PATH_GENERIC).  tg_set_path returns the
 * previous setting, or -1 for an unknown path (the setting is unchanged).
 */
enum {
    TG_PATH_AUTO = 0,
    TG_PATH_NAIVE = 1,      /* one thread per output; a slow, plain kernel */
    TG_PATH_GENERIC = 2,    /* 128x128 tiles, any alignment, masked loads */
    TG_PATH_TILE128 = 3,    /* aligned operands, mid shapes: 128x128x64 tiles of 8 waves;
                               256x128 where that saves whole rounds; persistent
                               workgroups when K <= 64; 64x64 when tiles are few */
    TG_PATH_TILE256 = 4,    /* 256x256x64 tiles of 8 waves for large shapes, aligned operands */
    TG_PATH_SKINNY = 5,     /* M <= 64: column slices streaming B, K steps dealt to waves */
    TG_PATH_W4 = 6,         /* tg_gemm_w4's int4-weight kernel (reported, not forced) */
    TG_PATH_ATTENTION = 7,  /* the attention entry points' kernel (reported, not forced) */
    TG_PATH_MLA = 8,        /* tg_mla_decode_f16's kernels (reported, not forced) */
    TG_PATH_RAGGED = 9,     /* aligned A, any-alignment (K,N) B and C: A direct to LDS, B via
                               registers, C stored through a parity-shifted LDS tile */
    TG_PATH_COUNT = 10
};
int tg_set_path(int path);

/* The path the most recent successful launch from this process used. */
int tg_last_path(void);

/*
 * Tuning knob for benchmarks: selects the kernel configuration (block tile,
 * K tile, pipeline depth, matrix-core product shape) that the tile paths use.
 * -1 restores the defaults; 0..42 are the direct-to-LDS configurations (32..38,
 * 40 and 41 use 16x16x32 products, the rest 32x32x16; 35..37 and 39 are the
 * persistent form that walks a list of tiles; 40..42 use 256x128 tiles), 100
 * and 101 the register-staged 128x128 and 256x256 kernels.  Returns the
 * previous setting, or -2 for an
 * unknown variant (the setting is unchanged).  Results are identical within
 * the accuracy contract for every variant; only speed changes.  22 and 23 are
 * ablations of configuration 0 (operand tiles without the XOR swizzle; a
 * 2-stage ring).  On the ragged path (TG_PATH_RAGGED) 0 and 1 select its
 * 256x256 and 128x128 configurations with 32x32x16 products, 2 and 3 the same
 * with 16x16x32 products (the defaults); other values pick by shape.
 */
int tg_set_tile_variant(int variant);

/*
 * The same for the skinny path (M <= 64): 0..9 select the column-slice width,
 * wave count, pipeline depth and cache hint; -1 restores the default.  Returns the
 * previous setting, or -2 for an unknown variant.
 */
int tg_set_skinny_variant(int variant);

/*
 * Tuning knob for benchmarks: the order in which the tile kernels (generic,
 * tile128, tile256) walk their output tiles.  group_m in 1..64: the workgroup
 * ids are renumbered so that each of the eight XCDs (each with its own L2)
 * takes a contiguous run of tiles, walked in panels of group_m tile rows,
 * column by column, so that tiles resident together share operand rows and
 * columns (the L2-friendly rasterisation primitive of the "TileLang paper
 * reading" page (hotelren.com), section 4, and of the primitive list of the
 * "TileLang DSL explainer" page (lzwjava.github.io), adapted to one L2 per
 * XCD).  0: plain row-major order of the workgroup ids, no renumbering.  -1
 * restores the default (8).  Returns the previous setting, or -2 for a value
 * outside -1..64 (unchanged).  Results are bitwise identical for every
 * setting.
 */
int tg_set_raster(int group_m);

/*
 * Tuning knob for benchmarks: the attention forward's workgroup shape, 0 =
 * four waves (128 queries per workgroup), 1 = eight waves (256 queries, K/V
 * tiles shared by twice the queries), on 32x32x16 matrix-core products; 2
 * and 3 = the same two shapes on 16x16x32 products; -1 restores the default
 * (1).  Returns the previous setting, or -2 for an unknown value.  Results
 * are identical within the attention tolerance for all four.
 */
int tg_set_attention_variant(int variant);

/* A static name for a path number ("auto", "naive", ...), or "unknown". */
const char *tg_path_name(int path);

#ifdef __cplusplus
}
#endif

#endif /* TG_H */
