/*
 * oracle.c - plain, slow, fp64 CPU reference for grouped-query attention.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may include, link,
 * load or call this file: only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark use it. It shares no code, header or helper
 * with the HIP library.
 *
 * What it computes (all arithmetic in IEEE double; inputs are decoded exactly,
 * bf16 -> double by a 16-bit shift, float -> double by widening):
 *
 *   Textbook scaled-dot-product attention with an explicit, full softmax
 *   (aifullclass.xyz, BERT self-attention article, LowRankSelfAttention
 *   example: scores = Q K^T times a scale, masked_fill, softmax over keys,
 *   weights times V). FlashAttention only reorganises where the intermediate
 *   values live and reaches the same result (webturing.pages.dev,
 *   "FlashAttention Serisi", sections "Ana fikir" and the FAQ entry on whether
 *   the softmax formula changes), so the plain definition is the reference.
 *
 *   Grouped-query attention: H_q query heads split into H_kv groups of
 *   g = H_q / H_kv consecutive heads, each group sharing one K/V head
 *   (blog.gitcode.com, "3个GQA核心优化技巧", section "Flash-Attention的稀疏分组
 *   优化": kv head = q head / group size; azimuth.plus GQA digest, section
 *   "Idea 2: grouped attention" and its mean-pooling code, which groups
 *   contiguous slices of heads). H_q % H_kv != 0 is rejected (gitcode page,
 *   section "GQA的分组共享机制", the divisibility assertion).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - layout: prefill Q/K/V/O are [B, S, H, d] row-major; the decode cache is
 *     [B, H_kv, max_len, d]; decode q/o are [B, H_q, d];
 *   - padding: seqlens[b] masks KEYS j >= L_b; every query row is computed;
 *   - an empty valid-key set gives O = 0 and LSE = -inf;
 *   - causal means key j is visible to query i iff j <= i (self-attention);
 *   - the decode query sees every cached key j < L_b and sits at position L_b - 1;
 *   - sliding window w > 0: key j is also required to satisfy j > i - w (the
 *     window of Mistral-style models, which the azimuth.plus GQA digest's
 *     timeline pairs with GQA, "2023: Mistral 7B"; the window is given in keys,
 *     the query's own key included);
 *   - ALiBi: the pages' attention signature has an `alibi_slopes` argument
 *     (gitcode page, section "GQA的分组共享机制") but no formula; the reading
 *     used is the usual one, score(i, j) = scale * <q_i, k_j> - slope_h * |i - j|,
 *     the bias added after scaling and before the softmax;
 *   - paged KV cache (the azimuth.plus digest, "the bigger picture": GQA is
 *     orthogonal to paged attention and composes with it): K/V rows live in a
 *     pool of pages [num_pages, H_kv, page_size, d]; key j of sequence b is row
 *     j % page_size of page block_table[b][j / page_size].
 *
 * Pins (tests/test_oracle_pins.py) tie this file to things other than itself:
 * torch's fp64 scaled_dot_product_attention, closed forms (uniform scores give
 * the mean of V, a two-key hand-worked case, V = 1 gives O = 1), GQA = MHA with
 * replicated K/V heads, G = 1 = MQA, key-permutation invariance, decode = last
 * causal-prefill row, and the split/log-sum-exp identity.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F64 = 0, ORC_F32 = 1, ORC_BF16 = 2 };

/* Exact decode of one stored element into double. */
static double ld(const void *p, int dtype, size_t idx) {
    if (dtype == ORC_F64) return ((const double *)p)[idx];
    if (dtype == ORC_F32) return (double)((const float *)p)[idx];
    uint32_t bits = (uint32_t)((const uint16_t *)p)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/*
 * One attention row, written out as the definition:
 *   for every key j in the valid set:  s_j = scale * <q, k_j> + bias_j
 *   m = max_j s_j,  p_j = exp(s_j - m),  l = sum_j p_j,  P_j = p_j / l
 *   o = sum_j P_j v_j,  lse = m + ln l
 * valid[j] != 0 marks the valid keys among n_keys. K row j starts at element
 * k_off + j * kv_row_stride (likewise V). q starts at q_off. p_out (n_keys
 * entries, may be NULL) receives the explicit probability row (0 for masked
 * keys). bias (n_keys entries) is the additive ALiBi term, or NULL for none.
 * Returns the number of valid keys.
 */
static int attend_row(const void *q, int qt, size_t q_off,
                      const void *k, const void *v, int kvt,
                      size_t k_off, size_t v_off, size_t kv_row_stride,
                      const unsigned char *valid, const double *bias, int n_keys, int d,
                      double scale, double *s /* scratch [n_keys] */,
                      double *o, double *lse, double *p_out) {
    int n_valid = 0;
    double m = -INFINITY;
    for (int j = 0; j < n_keys; ++j) {
        if (!valid[j]) continue;
        double dot = 0.0;
        for (int t = 0; t < d; ++t)
            dot += ld(q, qt, q_off + t) * ld(k, kvt, k_off + (size_t)j * kv_row_stride + t);
        s[j] = scale * dot + (bias ? bias[j] : 0.0);
        if (s[j] > m) m = s[j];
        ++n_valid;
    }
    for (int t = 0; t < d; ++t) o[t] = 0.0;
    if (n_valid == 0) {
        *lse = -INFINITY;
        if (p_out) for (int j = 0; j < n_keys; ++j) p_out[j] = 0.0;
        return 0;
    }
    double l = 0.0;
    for (int j = 0; j < n_keys; ++j) {
        if (!valid[j]) continue;
        s[j] = exp(s[j] - m); /* s now holds the unnormalised p_j */
        l += s[j];
    }
    for (int j = 0; j < n_keys; ++j) {
        double pj = valid[j] ? s[j] / l : 0.0;
        if (p_out) p_out[j] = pj;
        if (!valid[j]) continue;
        for (int t = 0; t < d; ++t)
            o[t] += pj * ld(v, kvt, v_off + (size_t)j * kv_row_stride + t);
    }
    *lse = m + log(l);
    return n_valid;
}

static int check_heads(int Hq, int Hkv) {
    return Hq > 0 && Hkv > 0 && Hq % Hkv == 0;
}

/* Clamp a caller length to [0, cap]. */
static int clamp_len(const int32_t *lens, int b, int cap) {
    if (!lens) return cap;
    int L = lens[b];
    if (L < 0) L = 0;
    if (L > cap) L = cap;
    return L;
}

/*
 * Prefill for an explicit list of query rows.
 *   q, k, v: [B, S, Hq, d] / [B, S, Hkv, d] / [B, S, Hkv, d], row-major
 *   rows:    n_rows triples (b, h, i)
 *   o:       [n_rows, d]   lse: [n_rows]   p_rows (optional): [n_rows, S]
 * Returns 0, or -1 on invalid shapes.
 */
int oracle_prefill_rows_ex(int dtype, const void *q, const void *k, const void *v,
                           const int32_t *seqlens, int B, int S, int Hq, int Hkv, int d,
                           double scale, int causal, int window, const double *alibi_slopes,
                           const int64_t *rows, int64_t n_rows,
                           double *o, double *lse, double *p_rows, int n_threads) {
    if (B <= 0 || S <= 0 || d <= 0 || !check_heads(Hq, Hkv) || window < 0) return -1;
    const int g = Hq / Hkv;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
    int bad = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)S);
        double *bias = alibi_slopes ? (double *)malloc(sizeof(double) * (size_t)S) : NULL;
        unsigned char *valid = (unsigned char *)malloc((size_t)S);
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < n_rows; ++r) {
            const int b = (int)rows[3 * r], h = (int)rows[3 * r + 1], i = (int)rows[3 * r + 2];
            if (b < 0 || b >= B || h < 0 || h >= Hq || i < 0 || i >= S) { bad = 1; continue; }
            const int kvh = h / g; /* contiguous grouping */
            const int L = clamp_len(seqlens, b, S);
            for (int j = 0; j < S; ++j) {
                valid[j] = (unsigned char)(j < L && (!causal || j <= i) &&
                                           (window == 0 || j > i - window));
                if (bias) bias[j] = -alibi_slopes[h] * fabs((double)(i - j));
            }
            const size_t q_off = (((size_t)b * S + i) * Hq + h) * (size_t)d;
            const size_t kv_off = ((size_t)b * S * Hkv + kvh) * (size_t)d;
            attend_row(q, dtype, q_off, k, v, dtype, kv_off, kv_off, (size_t)Hkv * d,
                       valid, bias, S, d, scale, s, o + (size_t)r * d, lse + r,
                       p_rows ? p_rows + (size_t)r * S : NULL);
        }
        free(s);
        free(bias);
        free(valid);
    }
    return bad ? -1 : 0;
}

int oracle_prefill_rows(int dtype, const void *q, const void *k, const void *v,
                        const int32_t *seqlens, int B, int S, int Hq, int Hkv, int d,
                        double scale, int causal, const int64_t *rows, int64_t n_rows,
                        double *o, double *lse, double *p_rows, int n_threads) {
    return oracle_prefill_rows_ex(dtype, q, k, v, seqlens, B, S, Hq, Hkv, d, scale, causal, 0,
                                  NULL, rows, n_rows, o, lse, p_rows, n_threads);
}

/*
 * Full prefill: o [B, S, Hq, d] (same layout as q), lse [B, Hq, S].
 */
int oracle_prefill_ex(int dtype, const void *q, const void *k, const void *v,
                      const int32_t *seqlens, int B, int S, int Hq, int Hkv, int d,
                      double scale, int causal, int window, const double *alibi_slopes,
                      double *o, double *lse, int n_threads) {
    if (B <= 0 || S <= 0 || d <= 0 || !check_heads(Hq, Hkv)) return -1;
    const int64_t n = (int64_t)B * S * Hq;
    int64_t *rows = (int64_t *)malloc(sizeof(int64_t) * 3 * (size_t)n);
    double *o_rows = (double *)malloc(sizeof(double) * (size_t)n * d);
    double *l_rows = (double *)malloc(sizeof(double) * (size_t)n);
    if (!rows || !o_rows || !l_rows) { free(rows); free(o_rows); free(l_rows); return -2; }
    int64_t r = 0;
    for (int b = 0; b < B; ++b)
        for (int i = 0; i < S; ++i)
            for (int h = 0; h < Hq; ++h, ++r) {
                rows[3 * r] = b; rows[3 * r + 1] = h; rows[3 * r + 2] = i;
            }
    int rc = oracle_prefill_rows_ex(dtype, q, k, v, seqlens, B, S, Hq, Hkv, d, scale, causal,
                                    window, alibi_slopes, rows, n, o_rows, l_rows, NULL,
                                    n_threads);
    if (rc == 0) {
        /* rows were enumerated in [B, S, Hq] order, matching o's layout */
        memcpy(o, o_rows, sizeof(double) * (size_t)n * d);
        r = 0;
        for (int b = 0; b < B; ++b)
            for (int i = 0; i < S; ++i)
                for (int h = 0; h < Hq; ++h, ++r)
                    lse[((size_t)b * Hq + h) * S + i] = l_rows[r];
    }
    free(rows); free(o_rows); free(l_rows);
    return rc;
}

int oracle_prefill(int dtype, const void *q, const void *k, const void *v,
                   const int32_t *seqlens, int B, int S, int Hq, int Hkv, int d,
                   double scale, int causal, double *o, double *lse, int n_threads) {
    return oracle_prefill_ex(dtype, q, k, v, seqlens, B, S, Hq, Hkv, d, scale, causal, 0, NULL,
                             o, lse, n_threads);
}

/*
 * Decode for an explicit list of (b, h) pairs: one query token per sequence
 * over a KV cache.
 *   q: [B, Hq, d];  lens: [B] or NULL;  pairs: n_pairs (b, h);  o: [n_pairs, d];
 *   lse: [n_pairs].
 *   Contiguous cache (block_table == NULL): k_cache, v_cache [B, Hkv, max_len, d].
 *   Paged cache: k_cache, v_cache are page pools [num_pages, Hkv, page_size, d],
 *   block_table [B, max_blocks] page ids, max_len = max_blocks * page_size; the
 *   valid keys of each sequence are first gathered into a contiguous buffer.
 *   The query sits at position L_b - 1: window > 0 keeps keys j > L_b - 1 - window,
 *   ALiBi adds -slope_h * (L_b - 1 - j).
 *   key range: keys j in [j_lo, j_hi) are also required (j_lo = 0, j_hi = max_len
 *   is the whole cache; a sub-range is used only to check the split identity).
 */
int oracle_decode_pairs_ex(int dtype, const void *q, const void *k_cache, const void *v_cache,
                           const int32_t *lens, const int32_t *block_table, int page_size,
                           int max_blocks, int num_pages, int B, int Hq, int Hkv, int d,
                           int max_len, double scale, int window, const double *alibi_slopes,
                           int j_lo, int j_hi, const int64_t *pairs, int64_t n_pairs,
                           double *o, double *lse, int n_threads) {
    if (B <= 0 || max_len <= 0 || d <= 0 || !check_heads(Hq, Hkv) || window < 0) return -1;
    if (block_table && (page_size <= 0 || max_blocks <= 0 || num_pages <= 0 ||
                        (int64_t)page_size * max_blocks != max_len))
        return -1;
    const int g = Hq / Hkv;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
    int bad = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)max_len);
        double *bias = alibi_slopes ? (double *)malloc(sizeof(double) * (size_t)max_len) : NULL;
        unsigned char *valid = (unsigned char *)malloc((size_t)max_len);
        double *kg = NULL, *vg = NULL;
        if (block_table) {
            kg = (double *)malloc(sizeof(double) * (size_t)max_len * d);
            vg = (double *)malloc(sizeof(double) * (size_t)max_len * d);
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n_pairs; ++r) {
            const int b = (int)pairs[2 * r], h = (int)pairs[2 * r + 1];
            if (b < 0 || b >= B || h < 0 || h >= Hq) { bad = 1; continue; }
            const int kvh = h / g;
            const int L = clamp_len(lens, b, max_len);
            const int qpos = L - 1;
            for (int j = 0; j < max_len; ++j) {
                valid[j] = (unsigned char)(j < L && j >= j_lo && j < j_hi &&
                                           (window == 0 || j > qpos - window));
                if (bias) bias[j] = -alibi_slopes[h] * fabs((double)(qpos - j));
            }
            const size_t q_off = ((size_t)b * Hq + h) * (size_t)d;
            if (!block_table) {
                const size_t kv_off = ((size_t)b * Hkv + kvh) * (size_t)max_len * d;
                attend_row(q, dtype, q_off, k_cache, v_cache, dtype, kv_off, kv_off, (size_t)d,
                           valid, bias, max_len, d, scale, s, o + (size_t)r * d, lse + r, NULL);
                continue;
            }
            /* gather: key j of sequence b is row j % page_size of page table[b][j / page_size] */
            for (int j = 0; j < L; ++j) {
                const int page = block_table[(size_t)b * max_blocks + j / page_size];
                if (page < 0 || page >= num_pages) { bad = 1; break; }
                const size_t src = (((size_t)page * Hkv + kvh) * page_size + j % page_size) * d;
                for (int t = 0; t < d; ++t) {
                    kg[(size_t)j * d + t] = ld(k_cache, dtype, src + t);
                    vg[(size_t)j * d + t] = ld(v_cache, dtype, src + t);
                }
            }
            attend_row(q, dtype, q_off, kg, vg, ORC_F64, 0, 0, (size_t)d, valid, bias, max_len,
                       d, scale, s, o + (size_t)r * d, lse + r, NULL);
        }
        free(s);
        free(bias);
        free(valid);
        free(kg);
        free(vg);
    }
    return bad ? -1 : 0;
}

int oracle_decode_pairs(int dtype, const void *q, const void *k_cache, const void *v_cache,
                        const int32_t *lens, int B, int Hq, int Hkv, int d, int max_len,
                        double scale, int j_lo, int j_hi,
                        const int64_t *pairs, int64_t n_pairs,
                        double *o, double *lse, int n_threads) {
    return oracle_decode_pairs_ex(dtype, q, k_cache, v_cache, lens, NULL, 0, 0, 0, B, Hq, Hkv, d,
                                  max_len, scale, 0, NULL, j_lo, j_hi, pairs, n_pairs, o, lse,
                                  n_threads);
}

/* Full decode: o [B, Hq, d], lse [B, Hq]. */
int oracle_decode_ex(int dtype, const void *q, const void *k_cache, const void *v_cache,
                     const int32_t *lens, const int32_t *block_table, int page_size,
                     int max_blocks, int num_pages, int B, int Hq, int Hkv, int d, int max_len,
                     double scale, int window, const double *alibi_slopes, double *o,
                     double *lse, int n_threads) {
    if (B <= 0 || Hq <= 0) return -1;
    const int64_t n = (int64_t)B * Hq;
    int64_t *pairs = (int64_t *)malloc(sizeof(int64_t) * 2 * (size_t)n);
    if (!pairs) return -2;
    for (int64_t r = 0; r < n; ++r) { pairs[2 * r] = r / Hq; pairs[2 * r + 1] = r % Hq; }
    int rc = oracle_decode_pairs_ex(dtype, q, k_cache, v_cache, lens, block_table, page_size,
                                    max_blocks, num_pages, B, Hq, Hkv, d, max_len, scale, window,
                                    alibi_slopes, 0, max_len, pairs, n, o, lse, n_threads);
    free(pairs);
    return rc;
}

int oracle_decode(int dtype, const void *q, const void *k_cache, const void *v_cache,
                  const int32_t *lens, int B, int Hq, int Hkv, int d, int max_len,
                  double scale, double *o, double *lse, int n_threads) {
    return oracle_decode_ex(dtype, q, k_cache, v_cache, lens, NULL, 0, 0, 0, B, Hq, Hkv, d,
                            max_len, scale, 0, NULL, o, lse, n_threads);
}

/*
 * Mean-pool conversion of per-head K or V projection weights from H heads to
 * G groups of H/G consecutive heads (azimuth.plus GQA digest, "Idea 1" step 1
 * and its code listing: each group's projection is the average of its heads).
 *   w: [H, rows, cols] row-major  ->  out: [G, rows, cols]
 */
int oracle_mean_pool_heads(int dtype, const void *w, int H, int G, int64_t per_head,
                           double *out) {
    if (H <= 0 || G <= 0 || H % G != 0 || per_head <= 0) return -1;
    const int hpg = H / G;
    for (int grp = 0; grp < G; ++grp)
        for (int64_t e = 0; e < per_head; ++e) {
            double acc = 0.0;
            for (int t = 0; t < hpg; ++t)
                acc += ld(w, dtype, (size_t)(grp * hpg + t) * (size_t)per_head + (size_t)e);
            out[(size_t)grp * (size_t)per_head + (size_t)e] = acc / hpg;
        }
    return 0;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
