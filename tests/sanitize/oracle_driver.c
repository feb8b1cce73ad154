/*
 * oracle_driver.c -- runs every entry point of the CPU oracle (oracle/prism_oracle.c) once on small
 * inputs: ragged and empty sequences, kp above T_b, ties, kappa = 1 and kappa = kp, both
 * aggregations, INT2 levels, the dense path.  Built with AddressSanitizer and
 * UndefinedBehaviorSanitizer by tests/test_sanitizers.py; exits non-zero when a call fails.
 * Test infrastructure only.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int orc_quantize_rows(const float* K, int64_t n_rows, int D, int8_t* Kq, float* scales);
int orc_quantize_rows_int2(const float* K, int64_t n_rows, int D, int8_t* levels, float* scales);
int orc_quantize_query(const float* q_group, int G, int D, int8_t* qi, float* scale_out);
int orc_propose_unit(const float* q_group, int G, int D, const int8_t* Kq, const float* scales, int64_t T_b,
                     int64_t kp, int agg, int32_t* pool, float* scores);
int orc_refine_unit(const float* q_group, int G, int D, const float* K, const float* V, int64_t T_b,
                    const int32_t* pool, int64_t kp, int64_t kappa, int agg, double sm_scale, int32_t* idx,
                    double* out, double* lse, double* S_out, double* logits_out);
int orc_attend_unit(const float* q_group, int G, int D, const float* K, const float* V, int64_t T_b,
                    const int32_t* list, int64_t n_list, double sm_scale, double* out, double* lse);
int orc_dense_unit(const float* q_group, int G, int D, const float* K, const float* V, int64_t T_b,
                   double sm_scale, double* out, double* lse);
int orc_propose(const float* q, int B, int Hq, int Hkv, int D, const int8_t* Kq, const float* scales,
                int64_t T_max, const int32_t* seq_lens, int64_t kp, int agg, int32_t* pool, float* scores,
                int nthreads);
int orc_refine(const float* q, int B, int Hq, int Hkv, int D, const float* K, const float* V, int64_t T_max,
               const int32_t* seq_lens, const int32_t* pool, int64_t kp, int64_t kappa, int agg, double sm_scale,
               int32_t* idx, double* out, double* lse, int nthreads);
int orc_dense(const float* q, int B, int Hq, int Hkv, int D, const float* K, const float* V, int64_t T_max,
              const int32_t* seq_lens, double sm_scale, double* out, double* lse, int nthreads);

static uint64_t g_state = 88172645463325252ull;
static float rnd(void) { /* xorshift64, uniform in [-1, 1) */
    g_state ^= g_state << 13; g_state ^= g_state >> 7; g_state ^= g_state << 17;
    return (float)((g_state >> 11) * (1.0 / 9007199254740992.0)) * 2.0f - 1.0f;
}

#define CHECK(call) do { int rc_ = (call); if (rc_ != 0) { fprintf(stderr, "%s -> %d\n", #call, rc_); return 1; } } while (0)

int main(void) {
    enum { B = 3, Hq = 8, Hkv = 2, D = 64, T = 300, KP = 120, KAPPA = 40 };
    const int G = Hq / Hkv;
    const int32_t lens[B] = {300, 77, 0};
    float* q = malloc(sizeof(float) * B * Hq * D);
    float* K = malloc(sizeof(float) * B * Hkv * T * D);
    float* V = malloc(sizeof(float) * B * Hkv * T * D);
    int8_t* Kq = malloc((size_t)B * Hkv * T * D);
    int8_t* lv = malloc((size_t)B * Hkv * T * D);
    float* sc = malloc(sizeof(float) * B * Hkv * T);
    int32_t* pool = malloc(sizeof(int32_t) * B * Hkv * KP);
    float* scores = malloc(sizeof(float) * B * Hkv * T);
    int32_t* idx = malloc(sizeof(int32_t) * B * Hkv * KP);  /* kappa up to kp below */
    double* out = malloc(sizeof(double) * B * Hq * D);
    double* lse = malloc(sizeof(double) * B * Hq);
    for (int i = 0; i < B * Hq * D; ++i) q[i] = rnd();
    for (int i = 0; i < B * Hkv * T * D; ++i) { K[i] = rnd(); V[i] = rnd(); }
    for (int d = 0; d < D; ++d) { K[5 * D + d] = 0.0f; K[9 * D + d] = K[8 * D + d]; }  /* zero row, tie */
    CHECK(orc_quantize_rows(K, (int64_t)B * Hkv * T, D, Kq, sc));
    CHECK(orc_quantize_rows_int2(K, (int64_t)B * Hkv * T, D, lv, sc));
    CHECK(orc_quantize_rows(K, (int64_t)B * Hkv * T, D, Kq, sc));
    int8_t qi[Hq * D];
    float qs;
    CHECK(orc_quantize_query(q, G, D, qi, &qs));
    for (int agg = 0; agg < 2; ++agg) {
        CHECK(orc_propose(q, B, Hq, Hkv, D, Kq, sc, T, lens, KP, agg, pool, scores, 2));
        CHECK(orc_propose(q, B, Hq, Hkv, D, lv, sc, T, lens, KP, agg, pool, NULL, 1));
        CHECK(orc_refine(q, B, Hq, Hkv, D, K, V, T, lens, pool, KP, KAPPA, agg, 0.125, idx, out, lse, 2));
        CHECK(orc_refine(q, B, Hq, Hkv, D, K, V, T, lens, pool, KP, 1, agg, 0.125, idx, out, lse, 1));
        CHECK(orc_refine(q, B, Hq, Hkv, D, K, V, T, lens, pool, KP, KP, agg, 0.125, idx, out, lse, 1));
    }
    {   /* one unit with kp above T_b, full outputs */
        int32_t pool1[400];
        float sc1[300];
        double S[400], lg[400 * 4], o1[4 * D], l1[4];
        int32_t id1[400];
        CHECK(orc_propose_unit(q, G, D, Kq, sc, 250, 400, 0, pool1, sc1));
        CHECK(orc_refine_unit(q, G, D, K, V, 250, pool1, 400, 400, 0, 0.125, id1, o1, l1, S, lg));
        CHECK(orc_attend_unit(q, G, D, K, V, 250, pool1, 400, 0.125, o1, l1));
        CHECK(orc_dense_unit(q, G, D, K, V, 250, 0.125, o1, l1));
    }
    CHECK(orc_dense(q, B, Hq, Hkv, D, K, V, T, lens, 0.125, out, lse, 2));
    free(q); free(K); free(V); free(Kq); free(lv); free(sc); free(pool); free(scores); free(idx); free(out); free(lse);
    printf("oracle driver ok\n");
    return 0;
}
