/*
 * tlsl_oracle.c -- plain, slow, double-precision CPU oracle of the DSA
 * token-selection path.  TEST INFRASTRUCTURE ONLY: it is called by the tests,
 * by the smoke check and by the benchmark's CPU-baseline leg, never by the
 * library.  It shares no code, header or constant with the HIP library.
 *
 * Every function follows a definition on the DSA page ("2.2.1 DSA 与索引器:
 * 先召回 token, 再计算 Sparse MLA"):
 *   - the Lightning Indexer score, section 1.1 eq.(1);
 *   - the causal selection S_t = TopK({I[t,s] : 0 <= s <= t}, min(k, t+1)),
 *     section 1.1 eq.(2), 0-based positions, the current token included, the
 *     unused slots of a fixed-width row marked invalid (-1);
 *   - attention over the selected shared latent entries, section 1.1 eq.(3),
 *     in the weight-absorbed MQA form of section 2 ("KV cache, quantization
 *     and two states"): every head reads the same entry c_s, whose full width
 *     is the key and whose first Dv components are the value.
 *
 * Readings where the page is silent (they are the library's contract too):
 *   - ties in eq.(2) go to the lower position; -0.0 and +0.0 are equal;
 *   - a selected row is written in ascending position order, then -1s;
 *   - a score is accumulated in double and rounded once to fp32; selection
 *     compares those fp32 values;
 *   - fp8 is OCP e4m3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
 *     subnormals, S.1111.111 is NaN, no infinities); a token's value is its
 *     fp32 scale times the decoded code;
 *   - attention skips slots that are < 0 or beyond the causal limit and counts
 *     a repeated slot once per occurrence; a row without a valid slot gives
 *     o = 0 and lse = -inf.
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -shared -fPIC.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORA_F32 0
#define ORA_BF16 1
#define ORA_FP8 2

/* ---- storage formats -------------------------------------------------- */

/* OCP 8-bit floating point, E4M3 variant: value = (-1)^s * 2^(e-7) * 1.m for
 * e in 1..15, (-1)^s * 2^-6 * 0.m for e = 0; e = 15 with m = 7 is NaN. */
double ora_decode_fp8_e4m3(uint8_t code)
{
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32 word. */
double ora_decode_bf16(uint16_t bits)
{
    uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

static double load_elem(int dt, const void *base, int64_t idx)
{
    switch (dt) {
    case ORA_F32:
        return (double)((const float *)base)[idx];
    case ORA_BF16:
        return ora_decode_bf16(((const uint16_t *)base)[idx]);
    default:
        return ora_decode_fp8_e4m3(((const uint8_t *)base)[idx]);
    }
}

/* ---- eq.(1): Lightning Indexer score ---------------------------------- */

/* I = sum_j w[j] * ReLU(q_j . k) for one query (HI heads of DI values, already
 * dequantised) against one key.  Also returns the magnitude sum
 * sum_j |w[j]| * ReLU(q_j . k), used by tests to scale the score tolerance. */
static double indexer_score(const double *q, const double *w, const double *k,
                            int HI, int DI, double *mag)
{
    double total = 0.0, absum = 0.0;
    for (int j = 0; j < HI; ++j) {
        double dot = 0.0;
        for (int i = 0; i < DI; ++i)
            dot += q[(int64_t)j * DI + i] * k[i];
        double relu = dot > 0.0 ? dot : 0.0;
        total += w[j] * relu;
        absum += fabs(w[j]) * relu;
    }
    if (mag)
        *mag = absum;
    return total;
}

/* Dequantise one token's HI*DI query values (or DI key values). */
static void load_token(int dt, const void *base, const float *scale, int64_t token,
                       int64_t width, double *out)
{
    double s = (dt == ORA_FP8 && scale) ? (double)scale[token] : 1.0;
    for (int64_t i = 0; i < width; ++i)
        out[i] = s * load_elem(dt, base, token * width + i);
}

/* ---- eq.(2): causal top-k with the lower-position tie rule ------------ */

typedef struct {
    float score;
    int32_t pos;
} ora_cand;

/* (score descending, position ascending); the float comparison treats
 * -0.0 == +0.0. */
static int cmp_rank(const void *pa, const void *pb)
{
    const ora_cand *a = pa, *b = pb;
    if (a->score > b->score)
        return -1;
    if (a->score < b->score)
        return 1;
    return (a->pos > b->pos) - (a->pos < b->pos);
}

static int cmp_pos(const void *pa, const void *pb)
{
    const ora_cand *a = pa, *b = pb;
    return (a->pos > b->pos) - (a->pos < b->pos);
}

/* Select from len scores (positions 0..len-1) the min(k,len) best, write them
 * to S in ascending position, then -1; S_score gets the slot's score or -inf. */
static void select_row(const float *scores, int64_t len, int k, int32_t *S, float *S_score)
{
    int64_t K = len < k ? len : k;
    ora_cand *c = malloc(sizeof(ora_cand) * (size_t)(len > 0 ? len : 1));
    for (int64_t s = 0; s < len; ++s) {
        c[s].score = scores[s];
        c[s].pos = (int32_t)s;
    }
    qsort(c, (size_t)len, sizeof(ora_cand), cmp_rank);
    qsort(c, (size_t)K, sizeof(ora_cand), cmp_pos);
    for (int64_t i = 0; i < k; ++i) {
        S[i] = i < K ? c[i].pos : -1;
        if (S_score)
            S_score[i] = i < K ? c[i].score : -INFINITY;
    }
    free(c);
}

int ora_topk_rows(const float *scores, const int64_t *row_start, const int32_t *row_len,
                  int R, int k, int32_t *S, float *S_score)
{
    if (!scores || !row_start || !row_len || !S || R < 0 || k <= 0)
        return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < R; ++r)
        select_row(scores + row_start[r], row_len[r], k, S + (int64_t)r * k,
                   S_score ? S_score + (int64_t)r * k : NULL);
    return 0;
}

/* every listed row (sequence) must name one of the batch's rows */
static int rows_ok(const int64_t *rows, int nrows, int64_t limit)
{
    for (int r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= limit)
            return 0;
    return 1;
}

static int seqs_ok(const int32_t *seqs, int nseq, int B)
{
    for (int i = 0; i < nseq; ++i)
        if (seqs[i] < 0 || seqs[i] >= B)
            return 0;
    return 1;
}

/* Prefill: for each requested flattened row (b*n + t) compute I[t, 0..t]
 * (eq.1), select (eq.2).  Optional per-row outputs of width n: the fp32 scores
 * and magnitude sums of the causal part (entries beyond t are left as NaN). */
int ora_index_prefill_rows(int dt, const void *qI, const float *q_scale, const void *kI,
                           const float *k_scale, const float *wI, int B, int n, int HI,
                           int DI, int k, const int64_t *rows, int nrows, int32_t *S,
                           float *S_score, float *score_rows, float *mag_rows)
{
    if (!qI || !kI || !wI || !rows || !S || B <= 0 || n <= 0 || HI <= 0 || DI <= 0 || k <= 0)
        return -1;
    if (dt == ORA_FP8 && (!q_scale || !k_scale))
        return -1;
    if (!rows_ok(rows, nrows, (int64_t)B * n))
        return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < nrows; ++r) {
        int64_t row = rows[r];
        int b = (int)(row / n);
        int t = (int)(row % n);
        double *q = malloc(sizeof(double) * (size_t)HI * DI);
        double *w = malloc(sizeof(double) * (size_t)HI);
        double *kk = malloc(sizeof(double) * (size_t)DI);
        float *sc = malloc(sizeof(float) * (size_t)(t + 1));
        load_token(dt, qI, q_scale, row, (int64_t)HI * DI, q);
        for (int j = 0; j < HI; ++j)
            w[j] = (double)wI[row * HI + j];
        for (int s = 0; s <= t; ++s) {
            double mag;
            load_token(dt, kI, k_scale, (int64_t)b * n + s, DI, kk);
            sc[s] = (float)indexer_score(q, w, kk, HI, DI, &mag);
            if (score_rows)
                score_rows[(int64_t)r * n + s] = sc[s];
            if (mag_rows)
                mag_rows[(int64_t)r * n + s] = (float)mag;
        }
        if (score_rows)
            for (int s = t + 1; s < n; ++s)
                score_rows[(int64_t)r * n + s] = NAN;
        if (mag_rows)
            for (int s = t + 1; s < n; ++s)
                mag_rows[(int64_t)r * n + s] = NAN;
        select_row(sc, t + 1, k, S + (int64_t)r * k, S_score ? S_score + (int64_t)r * k : NULL);
        free(q);
        free(w);
        free(kk);
        free(sc);
    }
    return 0;
}

/* Decode: the newest token of sequence b (t = L_b - 1) scored against its
 * whole packed cache slice [cu[b], cu[b+1]).  Only the listed sequences are
 * computed; scores (and magnitude sums) are written at the cache offsets. */
int ora_index_decode(int dt, const void *qI, const float *q_scale, const void *kI,
                     const float *k_scale, const float *wI, const int64_t *cu, int B, int HI,
                     int DI, const int32_t *seqs, int nseq, float *scores, float *mags)
{
    if (!qI || !kI || !wI || !cu || !seqs || !scores || B <= 0 || HI <= 0 || DI <= 0)
        return -1;
    if (dt == ORA_FP8 && (!q_scale || !k_scale))
        return -1;
    if (!seqs_ok(seqs, nseq, B))
        return -1;
    for (int i = 0; i < nseq; ++i) {
        int b = seqs[i];
        if (b < 0 || b >= B)
            return -1;
        double *q = malloc(sizeof(double) * (size_t)HI * DI);
        double *w = malloc(sizeof(double) * (size_t)HI);
        load_token(dt, qI, q_scale, b, (int64_t)HI * DI, q);
        for (int j = 0; j < HI; ++j)
            w[j] = (double)wI[(int64_t)b * HI + j];
#pragma omp parallel
        {
            double *kk = malloc(sizeof(double) * (size_t)DI);
#pragma omp for schedule(static)
            for (int64_t s = cu[b]; s < cu[b + 1]; ++s) {
                double mag;
                load_token(dt, kI, k_scale, s, DI, kk);
                scores[s] = (float)indexer_score(q, w, kk, HI, DI, &mag);
                if (mags)
                    mags[s] = (float)mag;
            }
            free(kk);
        }
        free(q);
        free(w);
    }
    return 0;
}

/* ---- eq.(3): softmax attention over the selected shared entries -------- */

/* One query row: heads H, query q[H][Dqk] (dequantised), entries c[.][Dqk]
 * addressed through the slot list; valid slots are 0 <= s <= limit. */
static void attend_row(int dt, const double *q, const void *kv, int64_t kv_base,
                       const int32_t *slots, int k, int64_t limit, int H, int Dqk, int Dv,
                       double scale, double *out, double *lse)
{
    int nvalid = 0;
    for (int i = 0; i < k; ++i)
        if (slots[i] >= 0 && slots[i] <= limit)
            ++nvalid;
    if (nvalid == 0) {
        for (int h = 0; h < H; ++h) {
            for (int d = 0; d < Dv; ++d)
                out[(int64_t)h * Dv + d] = 0.0;
            if (lse)
                lse[h] = -INFINITY;
        }
        return;
    }
    double *c = malloc(sizeof(double) * (size_t)nvalid * Dqk);
    double *z = malloc(sizeof(double) * (size_t)nvalid);
    int v = 0;
    for (int i = 0; i < k; ++i) {
        if (slots[i] < 0 || slots[i] > limit)
            continue;
        for (int d = 0; d < Dqk; ++d)
            c[(int64_t)v * Dqk + d] = load_elem(dt, kv, (kv_base + slots[i]) * Dqk + d);
        ++v;
    }
    for (int h = 0; h < H; ++h) {
        const double *qh = q + (int64_t)h * Dqk;
        double m = -INFINITY;
        for (int i = 0; i < nvalid; ++i) {
            double dot = 0.0;
            for (int d = 0; d < Dqk; ++d)
                dot += qh[d] * c[(int64_t)i * Dqk + d];
            z[i] = scale * dot;
            if (z[i] > m)
                m = z[i];
        }
        double denom = 0.0;
        for (int i = 0; i < nvalid; ++i)
            denom += exp(z[i] - m);
        double *o = out + (int64_t)h * Dv;
        for (int d = 0; d < Dv; ++d)
            o[d] = 0.0;
        for (int i = 0; i < nvalid; ++i) {
            double p = exp(z[i] - m) / denom;
            for (int d = 0; d < Dv; ++d)
                o[d] += p * c[(int64_t)i * Dqk + d];
        }
        if (lse)
            lse[h] = m + log(denom);
    }
    free(c);
    free(z);
}

int ora_sparse_attn_prefill_rows(int dt, const void *q, const void *kv, const int32_t *S,
                                 int B, int n, int H, int Dqk, int Dv, int k, double scale,
                                 const int64_t *rows, int nrows, double *out, double *lse)
{
    if (!q || !kv || !S || !rows || !out || B <= 0 || n <= 0 || H <= 0 || Dv > Dqk || k <= 0)
        return -1;
    if (dt == ORA_FP8)
        return -1;
    if (!rows_ok(rows, nrows, (int64_t)B * n))
        return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < nrows; ++r) {
        int64_t row = rows[r];
        int64_t b = row / n, t = row % n;
        double *qq = malloc(sizeof(double) * (size_t)H * Dqk);
        for (int64_t i = 0; i < (int64_t)H * Dqk; ++i)
            qq[i] = load_elem(dt, q, row * H * Dqk + i);
        attend_row(dt, qq, kv, b * n, S + row * k, k, t, H, Dqk, Dv, scale,
                   out + (int64_t)r * H * Dv, lse ? lse + (int64_t)r * H : NULL);
        free(qq);
    }
    return 0;
}

int ora_sparse_attn_decode(int dt, const void *q, const void *kv, const int64_t *cu,
                           const int32_t *S, int B, int H, int Dqk, int Dv, int k, double scale,
                           const int32_t *seqs, int nseq, double *out, double *lse)
{
    if (!q || !kv || !cu || !S || !seqs || !out || B <= 0 || H <= 0 || Dv > Dqk || k <= 0)
        return -1;
    if (dt == ORA_FP8)
        return -1;
    if (!seqs_ok(seqs, nseq, B))
        return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < nseq; ++i) {
        int b = seqs[i];
        double *qq = malloc(sizeof(double) * (size_t)H * Dqk);
        for (int64_t j = 0; j < (int64_t)H * Dqk; ++j)
            qq[j] = load_elem(dt, q, (int64_t)b * H * Dqk + j);
        attend_row(dt, qq, kv, cu[b], S + (int64_t)b * k, k, cu[b + 1] - cu[b] - 1, H, Dqk,
                   Dv, scale, out + (int64_t)i * H * Dv, lse ? lse + (int64_t)i * H : NULL);
        free(qq);
    }
    return 0;
}

int ora_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
