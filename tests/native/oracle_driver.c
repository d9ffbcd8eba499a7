/*
 * oracle_driver.c -- runs every entry point of oracle/tlsl_oracle.c on small
 * inputs (the DSA page's worked example of section 1.1, eq.(4)-(6), and a
 * seeded random case with empty, short and full rows) so that the oracle can
 * be built and exercised under ASan + UBSan by tests/test_sanitizers.py.
 * Prints "oracle driver ok" and exits 0 when the worked example comes out as
 * printed and every call accepts its arguments.  TEST INFRASTRUCTURE ONLY.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

double ora_decode_fp8_e4m3(uint8_t code);
double ora_decode_bf16(uint16_t bits);
int ora_topk_rows(const float *, const int64_t *, const int32_t *, int, int, int32_t *, float *);
int ora_index_prefill_rows(int, const void *, const float *, const void *, const float *, const float *, int,
                           int, int, int, int, const int64_t *, int, int32_t *, float *, float *, float *);
int ora_index_decode(int, const void *, const float *, const void *, const float *, const float *,
                     const int64_t *, int, int, int, const int32_t *, int, float *, float *);
int ora_sparse_attn_prefill_rows(int, const void *, const void *, const int32_t *, int, int, int, int, int,
                                 int, double, const int64_t *, int, double *, double *);
int ora_sparse_attn_decode(int, const void *, const void *, const int64_t *, const int32_t *, int, int, int,
                           int, int, double, const int32_t *, int, double *, double *);
int ora_sparse_attn_rows(int, const void *, const void *, const int32_t *, const int64_t *, int, int, int, int,
                         int, double, double *, double *);

static uint64_t rng = 88172645463325252ull;
static double urand(void) /* xorshift64, uniform in [-1, 1) */
{
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (double)(rng >> 11) / 4503599627370496.0 - 1.0;
}

int main(void)
{
    int fail = 0;
    /* worked example: query at t = 2, H^I = 2, d^I = 2 */
    float q[3 * 2 * 2] = {0}, k[3 * 2] = {2, -1, 1, 3, -1, 4}, w[3 * 2] = {0};
    q[8] = 1; q[9] = 0; q[10] = 0; q[11] = 1;
    w[4] = 0.75f; w[5] = 0.25f;
    int64_t row = 2;
    int32_t S[2];
    float Ss[2], sc[3], mg[3];
    fail |= ora_index_prefill_rows(0, q, NULL, k, NULL, w, 1, 3, 2, 2, 2, &row, 1, S, Ss, sc, mg) != 0;
    fail |= !(sc[0] == 1.5f && sc[1] == 1.5f && sc[2] == 1.0f && S[0] == 0 && S[1] == 1);
    /* eq.(5)-(6): logits 0.2, 1.2 over values (2,0), (0,3) */
    float kv[3 * 3] = {2, 0, 0.2f, 0, 3, 1.2f, 5, 5, 9};
    float qa[3 * 3] = {0, 0, 0, 0, 0, 0, 0, 0, 1};
    int32_t Sa[3 * 2] = {0, -1, 0, 1, 0, 1};
    double out[2], lse;
    fail |= ora_sparse_attn_prefill_rows(0, qa, kv, Sa, 1, 3, 1, 3, 2, 2, 1.0, &row, 1, out, &lse) != 0;
    fail |= !(fabs(out[0] - 0.538) < 5e-4 && fabs(out[1] - 2.193) < 5e-4);

    /* random case: B = 2, n = 40, H^I = 3, d^I = 8, k = 5, every row */
    enum { B = 2, N = 40, HI = 3, DI = 8, KK = 5, H = 2, DQK = 6, DV = 4 };
    float *qi = malloc(sizeof(float) * B * N * HI * DI), *ki = malloc(sizeof(float) * B * N * DI);
    float *wi = malloc(sizeof(float) * B * N * HI);
    for (int i = 0; i < B * N * HI * DI; ++i) qi[i] = (float)urand();
    for (int i = 0; i < B * N * DI; ++i) ki[i] = (float)urand();
    for (int i = 0; i < B * N * HI; ++i) wi[i] = (float)urand();
    int64_t rows[B * N];
    for (int i = 0; i < B * N; ++i) rows[i] = i;
    int32_t *Sp = malloc(sizeof(int32_t) * B * N * KK);
    float *Ssp = malloc(sizeof(float) * B * N * KK), *scp = malloc(sizeof(float) * B * N * N);
    float *mgp = malloc(sizeof(float) * B * N * N);
    fail |= ora_index_prefill_rows(0, qi, NULL, ki, NULL, wi, B, N, HI, DI, KK, rows, B * N, Sp, Ssp, scp, mgp) != 0;
    /* the same rows through topk_rows on the oracle's own scores */
    int64_t starts[B * N];
    int32_t lens[B * N];
    for (int i = 0; i < B * N; ++i) {
        starts[i] = (int64_t)i * N;
        lens[i] = (int32_t)(i % N) + 1;
    }
    int32_t *St = malloc(sizeof(int32_t) * B * N * KK);
    fail |= ora_topk_rows(scp, starts, lens, B * N, KK, St, NULL) != 0;
    for (int i = 0; i < B * N * KK; ++i) fail |= St[i] != Sp[i];
    /* decode: sequence lengths 0, 7, 33 */
    int64_t cu[4] = {0, 0, 7, 40};
    int32_t seqs[3] = {0, 1, 2};
    float dsc[40], dmg[40];
    fail |= ora_index_decode(0, qi, NULL, ki, NULL, wi, cu, 3, HI, DI, seqs, 3, dsc, dmg) != 0;
    /* attention: bf16 entries (zero bits are 0.0, others arbitrary finite) */
    uint16_t *qb = malloc(sizeof(uint16_t) * B * N * H * DQK), *kb = malloc(sizeof(uint16_t) * B * N * DQK);
    for (int i = 0; i < B * N * H * DQK; ++i) qb[i] = (uint16_t)(0x3f80 + (int)(urand() * 60));
    for (int i = 0; i < B * N * DQK; ++i) kb[i] = (uint16_t)(0x3f80 + (int)(urand() * 60));
    double *ob = malloc(sizeof(double) * B * N * H * DV), *lb = malloc(sizeof(double) * B * N * H);
    fail |= ora_sparse_attn_prefill_rows(1, qb, kb, Sp, B, N, H, DQK, DV, KK, 0.3, rows, B * N, ob, lb) != 0;
    int64_t lim[B * N];
    for (int i = 0; i < N; ++i) lim[i] = i;
    fail |= ora_sparse_attn_rows(1, qb, kb, Sp, lim, N, H, DQK, DV, KK, 0.3, ob, lb) != 0;
    int32_t Sd[3 * KK];
    for (int i = 0; i < 3 * KK; ++i) Sd[i] = i % 7 - 1;
    fail |= ora_sparse_attn_decode(1, qb, kb, cu, Sd, 3, H, DQK, DV, KK, 0.3, seqs, 3, ob, lb) != 0;
    for (int c = 0; c < 256; ++c) (void)ora_decode_fp8_e4m3((uint8_t)c);
    fail |= ora_decode_bf16(0x3f80) != 1.0;
    /* refusals: a row outside the batch, fp8 attention */
    int64_t bad = B * N;
    fail |= ora_index_prefill_rows(0, qi, NULL, ki, NULL, wi, B, N, HI, DI, KK, &bad, 1, Sp, NULL, NULL, NULL) == 0;
    fail |= ora_sparse_attn_rows(2, qb, kb, Sp, lim, 1, H, DQK, DV, KK, 0.3, ob, lb) == 0;
    free(qi); free(ki); free(wi); free(Sp); free(Ssp); free(scp); free(mgp); free(St);
    free(qb); free(kb); free(ob); free(lb);
    if (fail) {
        fprintf(stderr, "oracle driver: a check failed\n");
        return 1;
    }
    printf("oracle driver ok\n");
    return 0;
}
