/*
 * gqa.h - C ABI of libgqa.so: grouped-query attention forward pass on MI355X (gfx950).
 *
 * Grouped-query attention splits H_q query heads into H_kv groups of
 * g = H_q / H_kv consecutive heads; every head of a group reads the same K/V
 * head, kv_head = q_head / g (blog.gitcode.com, "3个GQA核心优化技巧", sections
 * "GQA的分组共享机制" and "Flash-Attention的稀疏分组优化"; azimuth.plus GQA
 * digest, "Idea 2: grouped attention": G = H is MHA, G = 1 is MQA).
 * The result is textbook attention, softmax(scale * Q K^T) V over the valid
 * keys (aifullclass.xyz BERT self-attention article, LowRankSelfAttention
 * example), computed FlashAttention-style: K/V are processed in tiles with a
 * running max and running sum, and the score matrix never reaches HBM
 * (webturing.pages.dev "FlashAttention Serisi", section "Ana fikir").
 *
 * Conventions shared by every entry point:
 *   - All array pointers are DEVICE pointers into memory the caller owns. The
 *     library never allocates or frees memory and keeps no pointer after a call
 *     returns. The only state it keeps between calls is set up once per device,
 *     on the first call on that device: the compute-unit count, for each kernel
 *     its dynamic-LDS attribute and how many of its workgroups a compute unit
 *     holds, and the device address of gqa_decode_noalloc's static scratch array
 *     (part of the library's device code, not an allocation).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and the call returns right after the enqueue. No call synchronises the
 *     host or reads device memory from the host.
 *   - Argument errors are detected on the host before any launch; the call then
 *     returns a non-zero gqa_status_t, launches nothing and prints nothing.
 *   - Lengths live in device memory and cannot be checked without a
 *     synchronisation, so the kernels clamp each length to [0, capacity].
 *   - Every buffer base must be 16-byte aligned (128-bit loads and stores).
 *   - Results are deterministic: the same inputs and arguments give
 *     bitwise-identical outputs (no floating-point atomics).
 */
#ifndef GQA_H
#define GQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GQA_OK = 0,
    GQA_ERR_INVALID_ARG = 1, /* bad shape, NULL required pointer, misalignment, H_q % H_kv != 0 */
    GQA_ERR_UNSUPPORTED = 2, /* head size or dtype the library does not provide            */
    GQA_ERR_WORKSPACE = 3,   /* decode workspace missing or smaller than required           */
    GQA_ERR_HIP = 4          /* the HIP runtime reported an error at launch                 */
} gqa_status_t;

typedef enum {
    GQA_DTYPE_F32 = 0,  /* IEEE binary32 in, binary32 out, fp32 arithmetic          */
    GQA_DTYPE_BF16 = 1  /* bfloat16 in, bfloat16 out (round to nearest even), fp32
                           accumulation and softmax                               */
} gqa_dtype_t;

/* Library version, major * 10000 + minor * 100 + patch. */
int gqa_version(void);

/* Static, human-readable text for a status code (never NULL). */
const char *gqa_status_string(int status);

/*
 * gqa_prefill - self-attention over a whole sequence, bidirectional (BERT
 * style) or causal.
 *
 * The pages' FlashAttention call takes separate query and K/V head counts,
 * `causal`, `softmax_scale` (1/sqrt(d_head) by default) and a padding mask
 * (gitcode page, "Flash-Attention的稀疏分组优化" and "阶段二：高级优化参数").
 * Here the padding mask is given as per-sequence key lengths.
 *
 *   dtype          GQA_DTYPE_F32 (d in {32, 64, 128}) or GQA_DTYPE_BF16
 *                  (d in {32, 64, 128}).
 *   q              [B, S, Hq, d] contiguous, row-major (BSHD).
 *   k, v           [B, S, Hkv, d] contiguous.
 *   o              [B, S, Hq, d] output, same dtype as q. Every row is written.
 *   lse            [B, Hq, S] fp32 natural-log log-sum-exp of the scaled scores
 *                  of each row, or NULL. A row with no valid key gets -inf
 *                  and O = 0.
 *   seqlens        [B] int32 valid KEY lengths (keys j >= seqlens[b] are masked
 *                  for every query row of sequence b; rows i >= seqlens[b] are
 *                  still computed), or NULL for "all S keys valid". K/V rows at
 *                  or past a length are never read, so they may hold anything.
 *   softmax_scale  multiplies Q K^T before the softmax. Any finite value.
 *   causal         0: every query sees every valid key. 1: query i sees keys
 *                  j <= i (and j < seqlens[b]).
 *   stream         hipStream_t or NULL.
 * Returns GQA_OK, GQA_ERR_INVALID_ARG (B, S, Hq, Hkv <= 0, Hq % Hkv != 0,
 * NULL q/k/v/o, misaligned base, a non-finite scale, causal not 0 or 1, or a
 * problem whose row or workgroup counts overflow the kernels' 32-bit indices),
 * GQA_ERR_UNSUPPORTED (dtype, d, or a bf16 problem whose K or V rows of one
 * sequence span more than 2^31 - 1 bytes: S x Hkv x d x 2) or GQA_ERR_HIP.
 */
int gqa_prefill(int dtype, const void *q, const void *k, const void *v, void *o, float *lse,
                const int32_t *seqlens, int B, int S, int Hq, int Hkv, int d,
                float softmax_scale, int causal, void *stream);

/*
 * gqa_prefill_ex - gqa_prefill with two optional score modifiers.
 *
 *   window         0: none. w > 0 (causal only): query i sees only keys
 *                  j > i - w, i.e. its own key and the w - 1 before it (the
 *                  sliding window of Mistral-style models, which the
 *                  azimuth.plus GQA digest's timeline pairs with GQA, entry
 *                  "2023: Mistral 7B"). Key tiles outside every row's window
 *                  are skipped. A window of S or more keys changes nothing.
 *   alibi_slopes   [Hq] fp32 device array, or NULL. The score of query i and
 *                  key j in head h becomes softmax_scale * <q_i, k_j> -
 *                  alibi_slopes[h] * |i - j| before the softmax (the pages'
 *                  attention signature has an `alibi_slopes` argument, gitcode
 *                  page, section "GQA的分组共享机制"; the bias form is the usual
 *                  ALiBi one). The LSE output includes the bias.
 * Every other argument is as for gqa_prefill. Additionally returns
 * GQA_ERR_INVALID_ARG for window < 0 or a misaligned alibi_slopes, and
 * GQA_ERR_UNSUPPORTED for a window on non-causal attention.
 */
int gqa_prefill_ex(int dtype, const void *q, const void *k, const void *v, void *o, float *lse,
                   const int32_t *seqlens, int B, int S, int Hq, int Hkv, int d,
                   float softmax_scale, int causal, int window, const float *alibi_slopes,
                   void *stream);

/*
 * gqa_decode_workspace_bytes - device workspace gqa_decode needs for these
 * arguments. The decode splits each cache's keys into pieces (the pages'
 * `num_splits` knob, gitcode page, "阶段二：高级优化参数"); a piece that does
 * not cover a whole sequence leaves a partial result, a normalised fp32 output
 * row per query head plus its log-sum-exp, for the merge. The workspace holds
 * (split workgroups + units) x 32 such rows, units = B x Hkv x ceil(g / 32).
 * Host arithmetic only (no HIP call). Returns 0 for invalid arguments.
 */
size_t gqa_decode_workspace_bytes(int B, int Hq, int Hkv, int d, int max_len, int num_splits);

/*
 * gqa_decode_num_workgroups - number of split workgroups gqa_decode launches
 * for these arguments: the `num_splits` knob of the gitcode page ("阶段二：
 * 高级优化参数") turned into a count of equal shares of the key work. With
 * num_splits == 0 (automatic) it is max(units, 256), one workgroup per compute
 * unit of the GPU at least; with n > 0 it is n x units; never more than the
 * total number of 32-key tiles of max_len-long caches. Host arithmetic only.
 * Returns 0 for invalid arguments.
 */
int gqa_decode_num_workgroups(int B, int Hq, int Hkv, int max_len, int num_splits);

/*
 * gqa_decode - one new query token per sequence attending to its KV cache.
 *
 * Each step of autoregressive generation reads the whole cached K and V of
 * every sequence, so decode is bound by memory bandwidth, and the cache holds
 * 2 x layers x G x d_k x n values for G K/V heads (azimuth.plus GQA digest,
 * "the bottleneck" section and its KV-cache size formula). The work over the
 * keys is split into pieces (the pages' `num_splits` knob, gitcode page,
 * "阶段二：高级优化参数"); the pieces are merged with their log-sum-exp
 * weights, which gives the same result as one pass over all keys.
 *
 *   dtype          GQA_DTYPE_BF16 (d in {64, 128}); fp32 is GQA_ERR_UNSUPPORTED.
 *   q              [B, Hq, d] contiguous: the newest token of each sequence.
 *   k_cache,
 *   v_cache        [B, Hkv, max_len, d] contiguous.
 *   cache_lens     [B] int32 valid lengths (keys j < cache_lens[b] are
 *                  attended, rows at or past it are never read), or NULL for
 *                  "all max_len rows valid". A zero length gives O = 0 and
 *                  LSE = -inf.
 *   o              [B, Hq, d] output, same dtype.
 *   lse            [B, Hq] fp32 natural-log log-sum-exp, or NULL.
 *   softmax_scale  any finite value.
 *   num_splits     0 = automatic. n > 0: the total key work is divided into
 *                  n x B x Hkv x ceil(g / 32) equal shares, one workgroup each;
 *                  a sequence is split into as many pieces as shares overlap
 *                  it, so longer caches get more splits.
 *   workspace      device buffer of at least gqa_decode_workspace_bytes(...)
 *                  bytes (may be NULL when that size is 0). Its contents on
 *                  entry do not matter; calls that share a workspace must not
 *                  overlap in time.
 * Returns GQA_OK, GQA_ERR_INVALID_ARG, GQA_ERR_UNSUPPORTED, GQA_ERR_WORKSPACE
 * or GQA_ERR_HIP.
 */
int gqa_decode(int dtype, const void *q, const void *k_cache, const void *v_cache,
               const int32_t *cache_lens, void *o, float *lse, int B, int Hq, int Hkv, int d,
               int max_len, float softmax_scale, int num_splits, void *workspace,
               size_t workspace_bytes, void *stream);

/*
 * gqa_decode_ex - gqa_decode over a contiguous or paged KV cache, with an
 * optional sliding window and ALiBi bias. The query is the token at position
 * cache_lens[b] - 1.
 *
 *   block_table    NULL: k_cache, v_cache are [B, Hkv, max_len, d] as for
 *                  gqa_decode. Otherwise a paged cache (the azimuth.plus GQA
 *                  digest, "the bigger picture": GQA composes with paged
 *                  attention): k_cache and v_cache are page pools
 *                  [num_pages, Hkv, page_size, d] and block_table is a
 *                  [B, max_blocks] int32 device array; key j of sequence b is
 *                  row j % page_size of page block_table[b][j / page_size].
 *                  Entries past a sequence's length are never read; a page id
 *                  outside [0, num_pages) reads as zeros (no fault).
 *   page_size      keys per page, a positive multiple of 32 (paged only).
 *   max_blocks     columns of block_table; max_len must equal
 *                  max_blocks * page_size (paged only).
 *   num_pages      pages in each pool (paged only).
 *   window         0: none. w > 0: only the last w keys of each sequence
 *                  (j > cache_lens[b] - 1 - w) are attended; the work split
 *                  covers only those keys.
 *   alibi_slopes   [Hq] fp32 device array, or NULL: the score of key j becomes
 *                  softmax_scale * <q, k_j> - alibi_slopes[h] * (L_b - 1 - j).
 * Every other argument is as for gqa_decode (the workspace size is the same).
 * Additionally returns GQA_ERR_INVALID_ARG for window < 0, misaligned
 * alibi_slopes or block_table, or inconsistent paging arguments.
 */
int gqa_decode_ex(int dtype, const void *q, const void *k_cache, const void *v_cache,
                  const int32_t *cache_lens, const int32_t *block_table, int page_size,
                  int max_blocks, int num_pages, void *o, float *lse, int B, int Hq, int Hkv,
                  int d, int max_len, float softmax_scale, int window,
                  const float *alibi_slopes, int num_splits, void *workspace,
                  size_t workspace_bytes, void *stream);

/* Size of the device scratch gqa_decode_noalloc uses instead of a workspace (32 MiB). */
#define GQA_DECODE_SCRATCH_BYTES (32u << 20)

/*
 * gqa_decode_noalloc - gqa_decode_ex without a workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. The split partials go to a
 * scratch array of GQA_DECODE_SCRATCH_BYTES that the library holds in device
 * memory (one per GPU it runs on, kept until the process ends); the call itself
 * allocates nothing. The first call on a device looks the array's address up
 * once (a HIP query, no allocation).
 *
 * Every argument and result is as for gqa_decode_ex. Additionally returns
 * GQA_ERR_WORKSPACE when the call needs more than GQA_DECODE_SCRATCH_BYTES,
 * i.e. when gqa_decode_workspace_bytes(B, Hq, Hkv, d, max_len, num_splits)
 * exceeds it (nothing is launched). The scratch keeps the last call's contents;
 * no call relies on what it holds on entry. All calls on one GPU share that
 * GPU's scratch, so calls that overlap in time on one GPU (different streams or
 * threads) race and must be serialised by the caller.
 */
int gqa_decode_noalloc(int dtype, const void *q, const void *k_cache, const void *v_cache,
                       const int32_t *cache_lens, const int32_t *block_table, int page_size,
                       int max_blocks, int num_pages, void *o, float *lse, int B, int Hq,
                       int Hkv, int d, int max_len, float softmax_scale, int window,
                       const float *alibi_slopes, int num_splits, void *stream);

/*
 * gqa_mean_pool_heads - convert per-head K or V projection weights of a
 * multi-head checkpoint to G groups: each group's projection becomes the mean
 * of its H/G consecutive heads (azimuth.plus GQA digest, "Idea 1", step 1, the
 * conversion that is followed by a short continued pre-training).
 *
 *   dtype      GQA_DTYPE_BF16 or GQA_DTYPE_F32 (input and output); the sums
 *              run in fp32, a bf16 output is rounded to nearest even.
 *   w          [H, per_head] device array: head h's weights are the contiguous
 *              per_head elements starting at h * per_head (for a projection
 *              [H * d_head, d_model] that is per_head = d_head * d_model).
 *   H, G       heads before and after; H % G == 0 (G = 1: MQA, G = H: copy).
 *   per_head   elements per head, a positive multiple of 8.
 *   out        [G, per_head] device array; must not overlap w.
 *   stream     hipStream_t or NULL.
 * Returns GQA_OK, GQA_ERR_INVALID_ARG (shapes, NULL or misaligned pointers),
 * GQA_ERR_UNSUPPORTED (dtype) or GQA_ERR_HIP.
 */
int gqa_mean_pool_heads(int dtype, const void *w, int H, int G, int64_t per_head, void *out,
                        void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_H */
