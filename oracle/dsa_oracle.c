/*
 * dsa_oracle.c -- plain, slow, fp64 CPU oracle for the DeepSeek Sparse
 * Attention (DSA) hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header or table with the HIP path.
 *
 * Sources (titles of the pages; no code is printed on any of them):
 *  [DD]  "DeepSeek-V3.2-Exp 稀疏注意力机制(DSA)技术深度解析：从原理到 TaoToken API
 *        实测效率提升" (sheratonhq.com/news/139095), section 1: a light indexer
 *        scores every history token of each query with low-dimensional q/k,
 *        few heads, index_head_dim 128, ReLU in place of softmax and FP8
 *        arithmetic; a top-k selector keeps the k highest-scoring KV; the main
 *        attention then looks only at the selected subset, O(n^2) -> O(n*k).
 *  [V4]  "DeepSeek-V4 百万 token 上下文的工程实现" (blog.hotdry.top), section
 *        "从 O(N²) 到 O(N・k)": the same two stages (Lightning Indexer ->
 *        fine-grained selector -> attention over the kept top-k tokens).
 *
 * Readings taken where the pages are silent (each is also listed in the design
 * notes):
 *  - score:   I[t,s] = sum_h w[t,h] * ReLU( q_I[t,h] . k_I[s] ), no scale, no bias;
 *  - history: keys s <= pos(t) (the query's own position included);
 *  - top-k:   m = min(k, pos(t)+1) keys, highest score first, lower index first
 *             among equal scores; slots m..k-1 hold -1; the kept set is reported
 *             in ascending position order;
 *  - FP8:     OCP E4M3 (bias 7, 3 mantissa bits, subnormals, no inf, S.1111.111
 *             is NaN) times one fp32 scale per token row;
 *  - main attention: ordinary softmax(scale * q.k) over the kept rows, one
 *             selection per query shared by all heads; grouped-query heads map
 *             h -> h / (Hq/Hkv); in latent mode the value is the first d_v
 *             entries of the key row.
 *
 * Everything is computed in double precision with plain sequential sums, in
 * the order the definition is written.  Sizes are int64_t; arrays are
 * row-major and contiguous.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORA_F32 = 0, ORA_BF16 = 1, ORA_E4M3 = 2 };

/* Threads the parallel loops below use. */
int ora_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the thread count of the parallel loops below (n >= 1). */
void ora_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* OCP FP8 E4M3 ("E4M3FN"): 1 sign bit, 4 exponent bits with bias 7, 3
 * mantissa bits.  Exponent field 0 encodes subnormals m/8 * 2^-6.  There is no
 * infinity; exponent 15 with mantissa 7 is NaN, so the largest finite value is
 * 1.75 * 2^8 = 448. */
double ora_e4m3_value(uint8_t code)
{
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double mag;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, -6);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* bfloat16 is the upper half of an IEEE binary32 word. */
double ora_bf16_value(uint16_t bits)
{
    uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

static double load_elem(const void *base, int dtype, int64_t i)
{
    switch (dtype) {
    case ORA_F32:  return (double)((const float *)base)[i];
    case ORA_BF16: return ora_bf16_value(((const uint16_t *)base)[i]);
    default:       return ora_e4m3_value(((const uint8_t *)base)[i]);
    }
}

/* Dequantise a contiguous run of n stored values into fp64, times `scale`
 * (1 for unscaled formats). */
static void load_row(const void *base, int dtype, int64_t off, int64_t n,
                     double scale, double *dst)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = load_elem(base, dtype, off + i) * scale;
}

/* Scale of K/V row r (token * Hkv + kv head): the row's fp32 scale for FP8
 * caches, 1 for unscaled formats (scales == NULL). */
static double kv_row_scale(const float *scales, int64_t r)
{
    return scales ? (double)scales[r] : 1.0;
}

/*
 * Lightning-indexer scores of one sequence [DD §1].
 *   iq  [n_q, H, D]  (dtype), iq_scale [n_q] fp32 or NULL (treated as 1)
 *   ik  [n_k, D]     (dtype), ik_scale [n_k] fp32 or NULL
 *   iw  [n_q, H]     fp32
 *   pos [n_q]        last visible key of each query
 *   out [n_q, n_k]   fp64; -INFINITY for s > pos[t]
 */
void ora_index_scores(int64_t n_q, int64_t n_k, int64_t H, int64_t D, int dtype,
                      const void *iq, const float *iq_scale,
                      const void *ik, const float *ik_scale,
                      const float *iw, const int64_t *pos, double *out)
{
    double *q = (double *)malloc(sizeof(double) * (size_t)(H * D));
    for (int64_t t = 0; t < n_q; ++t) {
        double sq = iq_scale ? (double)iq_scale[t] : 1.0;
        load_row(iq, dtype, t * H * D, H * D, sq, q);
        /* keys are independent: split them over threads */
        #pragma omp parallel
        {
            double *k = (double *)malloc(sizeof(double) * (size_t)D);
            #pragma omp for schedule(static)
            for (int64_t s = 0; s < n_k; ++s) {
                if (s > pos[t]) {
                    out[t * n_k + s] = -INFINITY;
                    continue;
                }
                double sk = ik_scale ? (double)ik_scale[s] : 1.0;
                load_row(ik, dtype, s * D, D, sk, k);
                double score = 0.0;
                for (int64_t h = 0; h < H; ++h) {
                    double dot = 0.0;
                    for (int64_t d = 0; d < D; ++d)
                        dot += q[h * D + d] * k[d];
                    double relu = dot > 0.0 ? dot : 0.0;
                    score += (double)iw[t * H + h] * relu;
                }
                out[t * n_k + s] = score;
            }
            free(k);
        }
    }
    free(q);
}

typedef struct { double score; int64_t index; } ora_pair;

/* Highest score first; among equal scores the lower index first.  -0.0 and
 * +0.0 compare equal, as numbers do. */
static int cmp_score_desc_index_asc(const void *a, const void *b)
{
    const ora_pair *x = (const ora_pair *)a, *y = (const ora_pair *)b;
    if (x->score > y->score) return -1;
    if (x->score < y->score) return 1;
    if (x->index < y->index) return -1;
    if (x->index > y->index) return 1;
    return 0;
}

static int cmp_i32_asc(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/*
 * Top-k selector [DD §1; V4 "从 O(N²) 到 O(N・k)"]: for each query row keep the
 * m = min(k, pos+1) highest-scoring visible keys.
 *   scores [n_q, n_k] fp64, pos [n_q]
 *   idx    [n_q, k]   int32: the kept keys in ascending position order, then -1
 *   kth    [n_q]      the m-th highest score (the weakest kept one), or NaN
 *                     for an empty row; may be NULL
 */
void ora_topk(int64_t n_q, int64_t n_k, const double *scores, const int64_t *pos,
              int64_t k, int32_t *idx, double *kth)
{
    #pragma omp parallel
    {
        ora_pair *row = (ora_pair *)malloc(sizeof(ora_pair) * (size_t)(n_k > 0 ? n_k : 1));
        #pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < n_q; ++t) {
            int64_t visible = pos[t] + 1;
            if (visible > n_k) visible = n_k;
            if (visible < 0) visible = 0;
            for (int64_t s = 0; s < visible; ++s) {
                row[s].score = scores[t * n_k + s];
                row[s].index = s;
            }
            qsort(row, (size_t)visible, sizeof(ora_pair), cmp_score_desc_index_asc);
            int64_t m = visible < k ? visible : k;
            int32_t *dst = idx + t * k;
            for (int64_t j = 0; j < m; ++j)
                dst[j] = (int32_t)row[j].index;
            qsort(dst, (size_t)m, sizeof(int32_t), cmp_i32_asc);
            for (int64_t j = m; j < k; ++j)
                dst[j] = -1;
            if (kth)
                kth[t] = m > 0 ? row[m - 1].score : NAN;
        }
        free(row);
    }
}

/*
 * Top-k with a structural backbone [SA: the sider.ai essay on DeepSeek Sparse
 * Attention ("sparse-attention-that-isn-t-sparse-thinking"), sections
 * "直覺：閃電索引器，而非割草機" and "DSA 可能如何選擇保留內容": keep a local window of
 * neighbours and always-connected global tokens, add salience-chosen far
 * tokens, attend over the union; V4 section "滑动窗口 KV Cache 与混合策略": the
 * most recent tokens kept in full, older ones chosen by importance].  Per
 * query row, with visible keys 0..pos:
 *   forced  F = the first `sinks` keys and the last `window` visible keys;
 *   C       = the visible keys outside F (sinks <= s <= pos - window);
 *   picks   = the m = min(k, |C|) highest-scoring keys of C (lower index first
 *             among equal scores);
 *   idx row = F together with the picks, ascending, then -1, width
 *             k + sinks + window.
 *   kth     = the m-th highest score among the picks, NaN when m = 0.
 * With sinks = window = 0 this is ora_topk.
 */
void ora_select_backbone(int64_t n_q, int64_t n_k, const double *scores, const int64_t *pos,
                         int64_t k, int64_t sinks, int64_t window, int32_t *idx, double *kth)
{
    const int64_t width = k + sinks + window;
    #pragma omp parallel
    {
        ora_pair *cand = (ora_pair *)malloc(sizeof(ora_pair) * (size_t)(n_k > 0 ? n_k : 1));
        #pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < n_q; ++t) {
            int64_t visible = pos[t] + 1;
            if (visible > n_k) visible = n_k;
            if (visible < 0) visible = 0;
            int32_t *dst = idx + t * width;
            int64_t n = 0;
            /* the forced keys */
            for (int64_t s = 0; s < visible; ++s)
                if (s < sinks || s >= visible - window)
                    dst[n++] = (int32_t)s;
            /* the candidates and their m best */
            int64_t nc = 0;
            for (int64_t s = 0; s < visible; ++s)
                if (!(s < sinks || s >= visible - window)) {
                    cand[nc].score = scores[t * n_k + s];
                    cand[nc].index = s;
                    ++nc;
                }
            qsort(cand, (size_t)nc, sizeof(ora_pair), cmp_score_desc_index_asc);
            int64_t m = nc < k ? nc : k;
            for (int64_t j = 0; j < m; ++j)
                dst[n++] = (int32_t)cand[j].index;
            qsort(dst, (size_t)n, sizeof(int32_t), cmp_i32_asc);
            for (int64_t j = n; j < width; ++j)
                dst[j] = -1;
            if (kth)
                kth[t] = m > 0 ? cand[m - 1].score : NAN;
        }
        free(cand);
    }
}

/*
 * Main attention over the selected rows only [DD §1: the main attention looks
 * at the selected subset; O(n*k)].  One sequence:
 *   q   [n_q, Hq, dqk]                      (dtype)
 *   k   [n_k, Hkv, dqk]                     (kv_dtype)
 *   v   [n_k, Hkv, dv]  or NULL when latent (kv_dtype): the value is then the
 *                       first dv entries of the key row (Hkv must be 1)
 *   k_scale, v_scale [n_k, Hkv] fp32 or NULL: an FP8 cache stores each
 *                       (token, kv head) row as codes times one scale; the
 *                       latent value uses its key row's scale
 *   idx [n_q, kk] int32; entries < 0 or > pos[t] or >= n_k are skipped
 *   out [n_q, Hq, dv] fp64, lse [n_q, Hq] fp64 (natural log; -inf and out = 0
 *   for a row with no valid entry)
 * Heads are grouped: query head h reads kv head h / (Hq / Hkv).
 */
void ora_sparse_attn(int64_t n_q, int64_t n_k, int64_t Hq, int64_t Hkv,
                     int64_t dqk, int64_t dv, int latent, int dtype, int kv_dtype,
                     const void *q, const void *k, const void *v,
                     const float *k_scale, const float *v_scale, double scale,
                     const int32_t *idx, int64_t kk, const int64_t *pos,
                     double *out, double *lse)
{
    int64_t group = Hq / Hkv;
    #pragma omp parallel
    {
        double *qh = (double *)malloc(sizeof(double) * (size_t)dqk);
        double *kr = (double *)malloc(sizeof(double) * (size_t)dqk);
        double *vr = (double *)malloc(sizeof(double) * (size_t)dv);
        double *z = (double *)malloc(sizeof(double) * (size_t)(kk > 0 ? kk : 1));
        int64_t *sel = (int64_t *)malloc(sizeof(int64_t) * (size_t)(kk > 0 ? kk : 1));
        #pragma omp for collapse(2) schedule(dynamic, 1)
        for (int64_t t = 0; t < n_q; ++t) {
            for (int64_t h = 0; h < Hq; ++h) {
                int64_t g = h / group;
                int64_t n_sel = 0;
                for (int64_t j = 0; j < kk; ++j) {
                    int64_t s = idx[t * kk + j];
                    if (s < 0 || s >= n_k || s > pos[t])
                        continue;
                    sel[n_sel++] = s;
                }
                double *o = out + (t * Hq + h) * dv;
                if (n_sel == 0) {
                    for (int64_t d = 0; d < dv; ++d) o[d] = 0.0;
                    lse[t * Hq + h] = -INFINITY;
                    continue;
                }
                load_row(q, dtype, (t * Hq + h) * dqk, dqk, 1.0, qh);
                double zmax = -INFINITY;
                for (int64_t j = 0; j < n_sel; ++j) {
                    load_row(k, kv_dtype, (sel[j] * Hkv + g) * dqk, dqk,
                             kv_row_scale(k_scale, sel[j] * Hkv + g), kr);
                    double dot = 0.0;
                    for (int64_t d = 0; d < dqk; ++d)
                        dot += qh[d] * kr[d];
                    z[j] = scale * dot;
                    if (z[j] > zmax) zmax = z[j];
                }
                double denom = 0.0;
                for (int64_t j = 0; j < n_sel; ++j)
                    denom += exp(z[j] - zmax);
                for (int64_t d = 0; d < dv; ++d) o[d] = 0.0;
                for (int64_t j = 0; j < n_sel; ++j) {
                    if (latent)
                        load_row(k, kv_dtype, (sel[j] * Hkv + g) * dqk, dv,
                                 kv_row_scale(k_scale, sel[j] * Hkv + g), vr);
                    else
                        load_row(v, kv_dtype, (sel[j] * Hkv + g) * dv, dv,
                                 kv_row_scale(v_scale, sel[j] * Hkv + g), vr);
                    double p = exp(z[j] - zmax) / denom;
                    for (int64_t d = 0; d < dv; ++d)
                        o[d] += p * vr[d];
                }
                lse[t * Hq + h] = zmax + log(denom);
            }
        }
        free(qh); free(kr); free(vr); free(z); free(sel);
    }
}

/*
 * Textbook dense causal attention (every key s <= pos[t]), used only to pin the
 * sparse routine: with k >= pos+1 the two must agree.  Same layouts as above.
 * Written separately on purpose: full score row, then max, then normalise.
 */
void ora_dense_causal_attn(int64_t n_q, int64_t n_k, int64_t Hq, int64_t Hkv,
                           int64_t dqk, int64_t dv, int latent, int dtype, int kv_dtype,
                           const void *q, const void *k, const void *v,
                           const float *k_scale, const float *v_scale, double scale,
                           const int64_t *pos, double *out, double *lse)
{
    int64_t group = Hq / Hkv;
    for (int64_t t = 0; t < n_q; ++t) {
        for (int64_t h = 0; h < Hq; ++h) {
            int64_t g = h / group;
            int64_t last = pos[t] < n_k - 1 ? pos[t] : n_k - 1;
            double *o = out + (t * Hq + h) * dv;
            for (int64_t d = 0; d < dv; ++d) o[d] = 0.0;
            if (last < 0) { lse[t * Hq + h] = -INFINITY; continue; }
            double *row = (double *)malloc(sizeof(double) * (size_t)(last + 1));
            double mx = -INFINITY;
            for (int64_t s = 0; s <= last; ++s) {
                double dot = 0.0;
                for (int64_t d = 0; d < dqk; ++d)
                    dot += load_elem(q, dtype, (t * Hq + h) * dqk + d) *
                           load_elem(k, kv_dtype, (s * Hkv + g) * dqk + d);
                row[s] = scale * dot * kv_row_scale(k_scale, s * Hkv + g);
                if (row[s] > mx) mx = row[s];
            }
            double sum = 0.0;
            for (int64_t s = 0; s <= last; ++s) {
                row[s] = exp(row[s] - mx);
                sum += row[s];
            }
            for (int64_t s = 0; s <= last; ++s) {
                for (int64_t d = 0; d < dv; ++d) {
                    double val = latent
                        ? load_elem(k, kv_dtype, (s * Hkv + g) * dqk + d) * kv_row_scale(k_scale, s * Hkv + g)
                        : load_elem(v, kv_dtype, (s * Hkv + g) * dv + d) * kv_row_scale(v_scale, s * Hkv + g);
                    o[d] += row[s] / sum * val;
                }
            }
            lse[t * Hq + h] = mx + log(sum);
            free(row);
        }
    }
}
