/*
 * prism_oracle.c -- plain CPU oracle for the Prism Attention decode hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  The product path
 * (token_level_sparse_prism_amd and its HIP kernels) never calls it, and
 * the two share no source, header, table or helper.
 *
 * What it follows.  "Prism Attention: Proposal-Refined Index Sharing
 * Mechanism for Efficient LLMs Inference" (paperpeel page of arXiv
 * 2610.22985):
 *   - Sec. 4 Overview and Sec. 4.1: an anchor (proposal) layer scores the
 *     whole context and emits an expanded candidate pool C_t^F; each
 *     following refined (shared) layer re-selects its own top-kappa inside
 *     that pool and attends to it.
 *   - Sec. 4.2: the proposal layer scores with a compressed key cache.  The
 *     page names INT2 and prints no scheme; this oracle implements the int8
 *     per-token absmax scheme fixed for this library (readings R1/R2 below)
 *     and, as a second key format, a 2-bit per-token scheme (reading R1'
 *     at orc_quantize_rows_int2).
 *   - Sec. 5.1 Implementation Details: pool size n = rho * kappa.
 *   - Sec. 1 and Sec. 2.1: token-level top-kappa sparse attention.
 * Every equation on the page is missing, so each step below states the
 * reading it takes:
 *   R2  keys: per-token symmetric absmax, scale = amax/127, round half to
 *       even, clamp to [-127, 127], an all-zero row gives scale 0 and codes 0.
 *   R3  query: the same quantizer with ONE absmax over the G query heads
 *       that share a KV head.
 *   R4  one pool and one index set per KV head; the G heads' scores are
 *       combined by SUM (default) or MAX.
 *   R5  query head h belongs to KV head h / G.
 *   R6  proposal score = float(int32 accumulator) * scale[t] (one fp32
 *       rounding), -0 mapped to +0; rank order = (score desc, index asc).
 *   R7  pool and index sets are written in ascending token order, padded
 *       with -1; effective sizes are min(kp, T_b) and min(kappa, |pool|).
 *   R8  refined scores are exact products of the stored values, summed in
 *       double.
 *   R10 attention = softmax(q.K / sqrt(D)) V over the selected tokens.
 *   R12 the cache holds T_b tokens; no mask beyond t < T_b.
 *
 * Precision.  Integer work is exact; refined scores and attention are in
 * double.  Non-finite inputs are rejected (return code ORC_ERR_NONFINITE).
 *
 * Pins.  tests/test_oracle_pins.py checks every function here against
 * brute force (repeated argmax), library routines (numpy integer / float64
 * matmul, torch scaled_dot_product_attention in float64), closed forms and
 * invariants.  Parity of the quantizer constants (R2, R3) and of the
 * aggregator (R4) against the authors' own choices is UNPINNED: the page
 * does not print them.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_ERR_ARG 1
#define ORC_ERR_NONFINITE 2
#define ORC_ERR_NOMEM 3

#define ORC_AGG_SUM 0
#define ORC_AGG_MAX 1

/* ------------------------------------------------------------------------ */
/* Step O1/O2: symmetric absmax int8 quantizer of one vector of n values.    */
/* Reading R2 (keys, per token) and R3 (query, per KV-head group).           */
/* ------------------------------------------------------------------------ */
static int quantize_vector(const float* x, int64_t n, int8_t* codes, float* scale_out)
{
    float amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        if (!isfinite(x[i])) return ORC_ERR_NONFINITE;
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
        for (int64_t i = 0; i < n; ++i) codes[i] = 0;
        *scale_out = 0.0f;
        return ORC_OK;
    }
    float scale = amax / 127.0f;  /* fp32, correctly rounded */
    float inv = 127.0f / amax;    /* fp32, correctly rounded */
    for (int64_t i = 0; i < n; ++i) {
        float y = x[i] * inv;     /* one fp32 product */
        float r = rintf(y);       /* round half to even (default mode) */
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        codes[i] = (int8_t)r;
    }
    *scale_out = scale;
    return ORC_OK;
}

/* O1 over a flat array of rows: K [n_rows][D] -> Kq [n_rows][D], scales [n_rows]. */
int orc_quantize_rows(const float* K, int64_t n_rows, int D, int8_t* Kq, float* scales)
{
    if (!K || !Kq || !scales || D <= 0 || n_rows < 0) return ORC_ERR_ARG;
    int err = ORC_OK;
#pragma omp parallel for schedule(static) reduction(max : err)
    for (int64_t r = 0; r < n_rows; ++r) {
        int e = quantize_vector(K + r * D, D, Kq + r * D, &scales[r]);
        if (e > err) err = e;
    }
    return err;
}

/* ------------------------------------------------------------------------ */
/* Step O1' (INT2 keys).  Sec. 4.2 says the proposal layer scores with a key  */
/* cache compressed to INT2 but prints no scheme.  Reading R1': per token,   */
/* the range [-amax, amax] is cut into four equal cells and each value is    */
/* coded by the centre of its cell:                                          */
/*   scale s = amax / 4 (exact);  u = K * (2 / amax) (one fp32 product,      */
/*   2/amax correctly rounded);  c = 2 * floor(u) + 1 clamped to [-3, 3],    */
/*   so c is in {-3, -1, +1, +3} and K is reconstructed as s * c.            */
/* A value on a cell boundary (u an integer) takes the upper cell.  An       */
/* all-zero row gives s = 0 and c = +1 everywhere (u = 0).  The codes are    */
/* returned one per element as signed levels; scoring them is step O3 with   */
/* these levels in place of the int8 codes.                                  */
/* ------------------------------------------------------------------------ */
static int quantize_vector_int2(const float* x, int64_t n, int8_t* codes, float* scale_out)
{
    float amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        if (!isfinite(x[i])) return ORC_ERR_NONFINITE;
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    float inv = amax > 0.0f ? 2.0f / amax : 0.0f; /* fp32, correctly rounded */
    for (int64_t i = 0; i < n; ++i) {
        float u = x[i] * inv;                     /* one fp32 product */
        float c = 2.0f * floorf(u) + 1.0f;        /* centre of the cell, in units of s */
        if (c > 3.0f) c = 3.0f;
        if (c < -3.0f) c = -3.0f;
        codes[i] = (int8_t)c;
    }
    *scale_out = amax * 0.25f;
    return ORC_OK;
}

/* O1' over a flat array of rows: K [n_rows][D] -> levels [n_rows][D] in {-3,-1,1,3}, scales. */
int orc_quantize_rows_int2(const float* K, int64_t n_rows, int D, int8_t* levels, float* scales)
{
    if (!K || !levels || !scales || D <= 0 || n_rows < 0) return ORC_ERR_ARG;
    int err = ORC_OK;
#pragma omp parallel for schedule(static) reduction(max : err)
    for (int64_t r = 0; r < n_rows; ++r) {
        int e = quantize_vector_int2(K + r * D, D, levels + r * D, &scales[r]);
        if (e > err) err = e;
    }
    return err;
}

/* O2: the group's G*D query values share one absmax.  Returns the codes
 * qi[G][D]; the query scale itself never enters the ranking (it multiplies
 * every score of the unit by the same positive number) and is returned only
 * for completeness. */
int orc_quantize_query(const float* q_group, int G, int D, int8_t* qi, float* scale_out)
{
    if (!q_group || !qi || G <= 0 || D <= 0) return ORC_ERR_ARG;
    float s = 0.0f;
    int e = quantize_vector(q_group, (int64_t)G * D, qi, &s);
    if (scale_out) *scale_out = s;
    return e;
}

/* ------------------------------------------------------------------------ */
/* Total orders used by the two selections (reading R6: score desc, index    */
/* asc).                                                                     */
/* ------------------------------------------------------------------------ */
typedef struct { float score; int32_t t; } orc_fitem;
typedef struct { double score; int32_t t; int32_t slot; } orc_ditem;

static int cmp_fitem(const void* pa, const void* pb)
{
    const orc_fitem* a = (const orc_fitem*)pa;
    const orc_fitem* b = (const orc_fitem*)pb;
    if (a->score > b->score) return -1;
    if (a->score < b->score) return 1;
    return (a->t < b->t) ? -1 : (a->t > b->t) ? 1 : 0;
}

static int cmp_ditem(const void* pa, const void* pb)
{
    const orc_ditem* a = (const orc_ditem*)pa;
    const orc_ditem* b = (const orc_ditem*)pb;
    if (a->score > b->score) return -1;
    if (a->score < b->score) return 1;
    return (a->t < b->t) ? -1 : (a->t > b->t) ? 1 : 0;
}

static int cmp_i32(const void* pa, const void* pb)
{
    int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
    return (a < b) ? -1 : (a > b) ? 1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Steps O3-O4 for one unit (b, g): quantized full-context scoring and the   */
/* top-kp candidate pool (Sec. 4.2; Sec. 4.1 pool C_t^F; n = rho*kappa in    */
/* Sec. 5.1).                                                                */
/*   q_group [G][D] fp32 (the G query heads of this KV head)                 */
/*   Kq [T_b][D] int8, scales [T_b] fp32 (this unit's rows, token-major)     */
/*   pool [kp] int32 out: ascending, -1 padded                               */
/*   scores [T_b] fp32 out (optional)                                        */
/* ------------------------------------------------------------------------ */
int orc_propose_unit(const float* q_group, int G, int D, const int8_t* Kq,
                     const float* scales, int64_t T_b, int64_t kp, int agg,
                     int32_t* pool, float* scores)
{
    if (!q_group || !pool || G <= 0 || D <= 0 || kp < 1 || T_b < 0) return ORC_ERR_ARG;
    if (T_b > 0 && (!Kq || !scales)) return ORC_ERR_ARG;
    if (agg != ORC_AGG_SUM && agg != ORC_AGG_MAX) return ORC_ERR_ARG;

    int8_t* qi = (int8_t*)malloc((size_t)G * D);
    orc_fitem* items = (orc_fitem*)malloc(sizeof(orc_fitem) * (size_t)(T_b > 0 ? T_b : 1));
    if (!qi || !items) { free(qi); free(items); return ORC_ERR_NOMEM; }
    int e = orc_quantize_query(q_group, G, D, qi, NULL);
    if (e != ORC_OK) { free(qi); free(items); return e; }

    for (int64_t t = 0; t < T_b; ++t) {
        const int8_t* krow = Kq + t * D;
        int64_t A = 0;
        for (int h = 0; h < G; ++h) {
            int64_t acc = 0; /* int32 suffices (|acc| <= D*127*127); int64 is exact too */
            for (int d = 0; d < D; ++d) acc += (int64_t)qi[h * D + d] * (int64_t)krow[d];
            if (agg == ORC_AGG_SUM) A += acc;
            else if (h == 0 || acc > A) A = acc;
        }
        float score = (float)A * scales[t]; /* int -> fp32 (exact below 2^24), one fp32 product */
        if (score == 0.0f) score = 0.0f;    /* canonical +0 */
        items[t].score = score;
        items[t].t = (int32_t)t;
        if (scores) scores[t] = score;
    }

    /* Exact top-kp by definition: full sort under the total order, take the prefix. */
    qsort(items, (size_t)T_b, sizeof(orc_fitem), cmp_fitem);
    int64_t n = T_b < kp ? T_b : kp;
    for (int64_t i = 0; i < n; ++i) pool[i] = items[i].t;
    qsort(pool, (size_t)n, sizeof(int32_t), cmp_i32);
    for (int64_t i = n; i < kp; ++i) pool[i] = -1;

    free(qi);
    free(items);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Step O7: softmax(z) V over an explicit list of tokens, for the G heads.   */
/*   logits [n][G] double (q.K, unscaled) for the listed tokens             */
/*   rows [n] token ids into V [.][D]                                        */
/*   out [G][D] double, lse [G] double                                       */
/* An empty list gives out = 0 and lse = -inf.                               */
/* ------------------------------------------------------------------------ */
static void attend_list(const double* logits, const int32_t* rows, int64_t n, int G, int D,
                        const float* V, double sm_scale, double* out, double* lse)
{
    for (int h = 0; h < G; ++h) {
        double* o = out + (int64_t)h * D;
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        if (n == 0) { lse[h] = -INFINITY; continue; }
        double m = -INFINITY;
        for (int64_t j = 0; j < n; ++j) {
            double z = logits[j * G + h] * sm_scale;
            if (z > m) m = z;
        }
        double wsum = 0.0;
        for (int64_t j = 0; j < n; ++j) {
            double w = exp(logits[j * G + h] * sm_scale - m);
            wsum += w;
            const float* v = V + (int64_t)rows[j] * D;
            for (int d = 0; d < D; ++d) o[d] += w * (double)v[d];
        }
        for (int d = 0; d < D; ++d) o[d] /= wsum;
        lse[h] = m + log(wsum);
    }
}

/* exact q.K for G heads of one token, in double (bf16/fp32 products are exact in double) */
static void exact_logits(const float* q_group, int G, int D, const float* krow, double* l)
{
    for (int h = 0; h < G; ++h) {
        double acc = 0.0;
        for (int d = 0; d < D; ++d) acc += (double)q_group[h * D + d] * (double)krow[d];
        l[h] = acc;
    }
}

static int check_finite(const float* x, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(x[i])) return ORC_ERR_NONFINITE;
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Steps O5-O7 for one unit at one refined layer (Sec. 4.1: the refined      */
/* layer re-selects its own top-kappa within the inherited pool; Sec. 5.3    */
/* notes this touches only the pool).                                        */
/*   K, V [T_b or more][D] fp32 rows of this unit                            */
/*   pool [kp] (entries outside [0, T_b) are ignored)                        */
/*   idx [kappa] out: ascending, -1 padded                                   */
/*   out [G][D], lse [G] out (double)                                        */
/*   S_out [kp] optional: group score per pool slot (NAN for empty slots)    */
/*   logits_out [kp][G] optional                                             */
/* ------------------------------------------------------------------------ */
int orc_refine_unit(const float* q_group, int G, int D, const float* K, const float* V,
                    int64_t T_b, const int32_t* pool, int64_t kp, int64_t kappa, int agg,
                    double sm_scale, int32_t* idx, double* out, double* lse,
                    double* S_out, double* logits_out)
{
    if (!q_group || !pool || !idx || !out || !lse || G <= 0 || D <= 0 || kp < 1 ||
        kappa < 1 || T_b < 0)
        return ORC_ERR_ARG;
    if (agg != ORC_AGG_SUM && agg != ORC_AGG_MAX) return ORC_ERR_ARG;
    if (check_finite(q_group, (int64_t)G * D)) return ORC_ERR_NONFINITE;

    orc_ditem* items = (orc_ditem*)malloc(sizeof(orc_ditem) * (size_t)kp);
    double* lg = (double*)malloc(sizeof(double) * (size_t)kp * G);
    double* sel_logits = (double*)malloc(sizeof(double) * (size_t)kp * G);
    int32_t* rows = (int32_t*)malloc(sizeof(int32_t) * (size_t)kp);
    if (!items || !lg || !sel_logits || !rows) {
        free(items); free(lg); free(sel_logits); free(rows);
        return ORC_ERR_NOMEM;
    }

    int64_t nvalid = 0;
    for (int64_t j = 0; j < kp; ++j) {
        int32_t t = pool[j];
        if (S_out) S_out[j] = NAN;
        if (t < 0 || t >= T_b) continue;
        const float* krow = K + (int64_t)t * D;
        if (check_finite(krow, D) || check_finite(V + (int64_t)t * D, D)) {
            free(items); free(lg); free(sel_logits); free(rows);
            return ORC_ERR_NONFINITE;
        }
        exact_logits(q_group, G, D, krow, lg + j * G);
        double S = 0.0;
        for (int h = 0; h < G; ++h) {
            double l = lg[j * G + h];
            if (agg == ORC_AGG_SUM) S += l;
            else if (h == 0 || l > S) S = l;
        }
        if (S_out) S_out[j] = S;
        items[nvalid].score = S;
        items[nvalid].t = t;
        items[nvalid].slot = (int32_t)j;
        ++nvalid;
    }
    if (logits_out)
        for (int64_t j = 0; j < kp; ++j)
            for (int h = 0; h < G; ++h)
                logits_out[j * G + h] = (pool[j] >= 0 && pool[j] < T_b) ? lg[j * G + h] : NAN;

    /* O6: exact top-kappa by definition (full sort, prefix), re-sorted ascending. */
    qsort(items, (size_t)nvalid, sizeof(orc_ditem), cmp_ditem);
    int64_t n = nvalid < kappa ? nvalid : kappa;
    for (int64_t i = 0; i < n; ++i) idx[i] = items[i].t;
    qsort(idx, (size_t)n, sizeof(int32_t), cmp_i32);
    for (int64_t i = n; i < kappa; ++i) idx[i] = -1;

    /* O7: attention over the selected tokens (ascending order; the sum is order-free in value up to rounding). */
    for (int64_t i = 0; i < n; ++i) {
        rows[i] = idx[i];
        exact_logits(q_group, G, D, K + (int64_t)idx[i] * D, sel_logits + i * G);
    }
    attend_list(sel_logits, rows, n, G, D, V, sm_scale, out, lse);

    free(items); free(lg); free(sel_logits); free(rows);
    return ORC_OK;
}

/* O7 alone, over a caller-given token list (entries < 0 or >= T_b skipped).
 * Used to evaluate attention on another selection (e.g. the GPU's). */
int orc_attend_unit(const float* q_group, int G, int D, const float* K, const float* V,
                    int64_t T_b, const int32_t* list, int64_t n_list, double sm_scale,
                    double* out, double* lse)
{
    if (!q_group || !out || !lse || G <= 0 || D <= 0 || n_list < 0) return ORC_ERR_ARG;
    double* lg = (double*)malloc(sizeof(double) * (size_t)(n_list > 0 ? n_list : 1) * G);
    int32_t* rows = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n_list > 0 ? n_list : 1));
    if (!lg || !rows) { free(lg); free(rows); return ORC_ERR_NOMEM; }
    int64_t n = 0;
    for (int64_t i = 0; i < n_list; ++i) {
        int32_t t = list[i];
        if (t < 0 || t >= T_b) continue;
        exact_logits(q_group, G, D, K + (int64_t)t * D, lg + n * G);
        rows[n++] = t;
    }
    attend_list(lg, rows, n, G, D, V, sm_scale, out, lse);
    free(lg); free(rows);
    return ORC_OK;
}

/* O8: dense attention over every t < T_b (the kappa = kp = T_b special case). */
int orc_dense_unit(const float* q_group, int G, int D, const float* K, const float* V,
                   int64_t T_b, double sm_scale, double* out, double* lse)
{
    if (!q_group || !out || !lse || G <= 0 || D <= 0 || T_b < 0) return ORC_ERR_ARG;
    int32_t* all = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T_b > 0 ? T_b : 1));
    if (!all) return ORC_ERR_NOMEM;
    for (int64_t t = 0; t < T_b; ++t) all[t] = (int32_t)t;
    int e = orc_attend_unit(q_group, G, D, K, V, T_b, all, T_b, sm_scale, out, lse);
    free(all);
    return e;
}

/* ------------------------------------------------------------------------ */
/* Batched drivers over all units (b, g), OpenMP over units.                 */
/* Layouts (row-major): q [B][Hq][D]; Kq, K, V [B][Hkv][T_max][D];           */
/* scales [B][Hkv][T_max]; pool [B][Hkv][kp]; idx [B][Hkv][kappa];           */
/* out [B][Hq][D]; lse [B][Hq].  seq_lens [B] or NULL (all T_max).           */
/* Query head h maps to KV head h / G (reading R5).                          */
/* ------------------------------------------------------------------------ */
static int64_t seq_len_of(const int32_t* seq_lens, int b, int64_t T_max)
{
    if (!seq_lens) return T_max;
    int64_t t = seq_lens[b];
    if (t < 0) t = 0;
    if (t > T_max) t = T_max;
    return t;
}

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int orc_propose(const float* q, int B, int Hq, int Hkv, int D, const int8_t* Kq,
                const float* scales, int64_t T_max, const int32_t* seq_lens, int64_t kp,
                int agg, int32_t* pool, float* scores, int nthreads)
{
    if (B < 0 || Hkv <= 0 || Hq <= 0 || Hq % Hkv != 0) return ORC_ERR_ARG;
    int G = Hq / Hkv;
    set_threads(nthreads);
    int err = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1) reduction(max : err)
    for (int64_t u = 0; u < (int64_t)B * Hkv; ++u) {
        int b = (int)(u / Hkv), g = (int)(u % Hkv);
        int64_t T_b = seq_len_of(seq_lens, b, T_max);
        const float* qg = q + ((int64_t)b * Hq + (int64_t)g * G) * D;
        int e = orc_propose_unit(qg, G, D, Kq + u * T_max * D, scales + u * T_max, T_b, kp,
                                 agg, pool + u * kp, scores ? scores + u * T_max : NULL);
        if (e > err) err = e;
    }
    return err;
}

int orc_refine(const float* q, int B, int Hq, int Hkv, int D, const float* K, const float* V,
               int64_t T_max, const int32_t* seq_lens, const int32_t* pool, int64_t kp,
               int64_t kappa, int agg, double sm_scale, int32_t* idx, double* out, double* lse,
               int nthreads)
{
    if (B < 0 || Hkv <= 0 || Hq <= 0 || Hq % Hkv != 0) return ORC_ERR_ARG;
    int G = Hq / Hkv;
    set_threads(nthreads);
    int err = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1) reduction(max : err)
    for (int64_t u = 0; u < (int64_t)B * Hkv; ++u) {
        int b = (int)(u / Hkv), g = (int)(u % Hkv);
        int64_t T_b = seq_len_of(seq_lens, b, T_max);
        int64_t hq0 = (int64_t)b * Hq + (int64_t)g * G;
        int e = orc_refine_unit(q + hq0 * D, G, D, K + u * T_max * D, V + u * T_max * D, T_b,
                                pool + u * kp, kp, kappa, agg, sm_scale, idx + u * kappa,
                                out + hq0 * D, lse + hq0, NULL, NULL);
        if (e > err) err = e;
    }
    return err;
}

int orc_dense(const float* q, int B, int Hq, int Hkv, int D, const float* K, const float* V,
              int64_t T_max, const int32_t* seq_lens, double sm_scale, double* out, double* lse,
              int nthreads)
{
    if (B < 0 || Hkv <= 0 || Hq <= 0 || Hq % Hkv != 0) return ORC_ERR_ARG;
    int G = Hq / Hkv;
    set_threads(nthreads);
    int err = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1) reduction(max : err)
    for (int64_t u = 0; u < (int64_t)B * Hkv; ++u) {
        int b = (int)(u / Hkv), g = (int)(u % Hkv);
        int64_t T_b = seq_len_of(seq_lens, b, T_max);
        int64_t hq0 = (int64_t)b * Hq + (int64_t)g * G;
        int e = orc_dense_unit(q + hq0 * D, G, D, K + u * T_max * D, V + u * T_max * D, T_b,
                               sm_scale, out + hq0 * D, lse + hq0);
        if (e > err) err = e;
    }
    return err;
}

int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
