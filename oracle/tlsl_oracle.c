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

/* The same attention for rows given one by one: query r (q_rows[r], H x Dqk)
 * attends over its slots S_rows[r] (k of them) into entries kv[0..], valid
 * slots 0 <= s <= limits[r].  For a prefill row t of batch row b this is
 * kv = that batch row's entries and limit t: the rows a test samples from a
 * large batch are evaluated without the whole query tensor. */
int ora_sparse_attn_rows(int dt, const void *q_rows, const void *kv, const int32_t *S_rows,
                         const int64_t *limits, int nrows, int H, int Dqk, int Dv, int k,
                         double scale, double *out, double *lse)
{
    if (!q_rows || !kv || !S_rows || !limits || !out || nrows < 0 || H <= 0 || Dv > Dqk || k <= 0)
        return -1;
    if (dt == ORA_FP8)
        return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < nrows; ++r) {
        double *qq = malloc(sizeof(double) * (size_t)H * Dqk);
        for (int64_t j = 0; j < (int64_t)H * Dqk; ++j)
            qq[j] = load_elem(dt, q_rows, (int64_t)r * H * Dqk + j);
        attend_row(dt, qq, kv, 0, S_rows + (int64_t)r * k, k, limits[r], H, Dqk, Dv, scale,
                   out + (int64_t)r * H * Dv, lse ? lse + (int64_t)r * H : NULL);
        free(qq);
    }
    return 0;
}

/* ---- eq.(8): sparse-stage indexer loss and its gradient ------------------
 *
 * DSA page, section 1.2 eq.(8) and the normalisation rule after it: the
 * indexer's loss on query t is KL(p_{t,S_t} || Softmax(I_{t,S_t})), both
 * distributions normalised over the selected set S_t; a teacher sub-vector cut
 * from a dense distribution is divided by its kept mass.  The indexer inputs
 * are leaves (detached), so the gradient flows into q^I, k^I and w^I only.
 *
 * For row t with slots S[t, 0..k) (a slot outside [0, t] is not part of S_t)
 * and teacher masses p[t, 0..k) (>= 0, normalised here over the valid slots):
 *   I_i = sum_j w_j ReLU(q_j . k_{S_i})                   eq.(1)
 *   P_i = p_i / sum_valid p                               kept-mass rule
 *   R_i = exp(I_i) / sum_valid exp(I)                     Softmax(I_{t,S_t})
 *   L_t = sum_valid P_i (log P_i - log R_i),  0 log 0 = 0  eq.(8)
 * and with g_i = R_i - P_i (dL_t/dI_i) and ReLU'(x) = [x > 0]:
 *   dL/dw_j  = sum_i g_i ReLU(q_j . k_{S_i})
 *   dL/dq_j  = sum_i g_i w_j [q_j . k_{S_i} > 0] k_{S_i}
 *   dL/dk_s += sum_{i: S_i = s} g_i sum_j w_j [q_j . k_s > 0] q_j
 * summed over the rows for dk.  A row with no valid slot, or whose teacher
 * has no mass on its valid slots, has L_t = 0 and no gradient.  Gradients
 * are with respect to the dequantised values (for fp8, q = scale * code).
 * All rows of the batch are computed; dk is accumulated in row order inside
 * each thread's block of rows, the blocks summed in thread order. */
/* Optional magnitude sums (NULL to skip), the sums of the absolute values of
 * the terms, with |g_i| replaced by R_i + P_i, used by tests to scale the
 * tolerance of a result computed in lower precision:
 *   loss_mag = sum_valid P_i (|log P_i| + |log R_i|)
 *   dq_mag   = sum_i (R_i + P_i) |w_j| [x > 0] |k_{S_i}|      (per j, d)
 *   dk_mag  += sum_{i: S_i = s} (R_i + P_i) sum_j |w_j| [x > 0] |q_j|
 *   dw_mag   = sum_i (R_i + P_i) ReLU(x)                     (per j)
 * and the kink bands: the same dq and dk terms, at full weight, for every x =
 * q_j . k_s within DI * 2^-24 * sum_d |q_jd k_sd| of zero -- there an fp32
 * accumulation of the dot product (in any order) may land on either side of
 * the ReLU's kink, so a result computed in fp32 may count the term or not:
 *   dq_kink  = sum_{i: |x| <= band} (R_i + P_i) |w_j| |k_{S_i}|
 *   dk_kink += sum_{i: S_i = s} (R_i + P_i) sum_{j: |x| <= band} |w_j| |q_j| */
int ora_indexer_kl_mag(int dt, const void *qI, const float *q_scale, const void *kI,
                       const float *k_scale, const float *wI, int B, int n, int HI, int DI, int k,
                       const int32_t *S, const float *p, double *loss, double *dq, double *dk,
                       double *dw, double *loss_mag, double *dq_mag, double *dk_mag,
                       double *dw_mag, double *dq_kink, double *dk_kink);

int ora_indexer_kl(int dt, const void *qI, const float *q_scale, const void *kI,
                   const float *k_scale, const float *wI, int B, int n, int HI, int DI, int k,
                   const int32_t *S, const float *p, double *loss, double *dq, double *dk,
                   double *dw)
{
    return ora_indexer_kl_mag(dt, qI, q_scale, kI, k_scale, wI, B, n, HI, DI, k, S, p, loss, dq, dk,
                              dw, NULL, NULL, NULL, NULL, NULL, NULL);
}

int ora_indexer_kl_mag(int dt, const void *qI, const float *q_scale, const void *kI,
                       const float *k_scale, const float *wI, int B, int n, int HI, int DI, int k,
                       const int32_t *S, const float *p, double *loss, double *dq, double *dk,
                       double *dw, double *loss_mag, double *dq_mag, double *dk_mag,
                       double *dw_mag, double *dq_kink, double *dk_kink)
{
    if (!qI || !kI || !wI || !S || !p || !loss || !dq || !dk || !dw || B <= 0 || n <= 0 ||
        HI <= 0 || DI <= 0 || k <= 0)
        return -1;
    if (dt == ORA_FP8 && (!q_scale || !k_scale))
        return -1;
    const int64_t rows = (int64_t)B * n;
    int nth = 1;
#ifdef _OPENMP
    nth = omp_get_max_threads();
#endif
    const int want_mag = loss_mag && dq_mag && dk_mag && dw_mag && dq_kink && dk_kink;
    double *dk_part = calloc((size_t)nth * rows * DI * (want_mag ? 3 : 1), sizeof(double));
    if (!dk_part)
        return -1;
#pragma omp parallel num_threads(nth)
    {
        int tid = 0;
#ifdef _OPENMP
        tid = omp_get_thread_num();
#endif
        double *mydk = dk_part + (size_t)tid * rows * DI;
        double *mydkm = want_mag ? dk_part + ((size_t)nth + tid) * rows * DI : NULL;
        double *mydkk = want_mag ? dk_part + ((size_t)2 * nth + tid) * rows * DI : NULL;
        double *band = malloc(sizeof(double) * (size_t)k * HI);
        double *R = malloc(sizeof(double) * (size_t)k), *Pn = malloc(sizeof(double) * (size_t)k);
        double *q = malloc(sizeof(double) * (size_t)HI * DI);
        double *w = malloc(sizeof(double) * (size_t)HI);
        double *keys = malloc(sizeof(double) * (size_t)k * DI);
        double *X = malloc(sizeof(double) * (size_t)k * HI);
        double *I = malloc(sizeof(double) * (size_t)k);
        double *g = malloc(sizeof(double) * (size_t)k);
        int *valid = malloc(sizeof(int) * (size_t)k);
#pragma omp for schedule(static)
        for (int64_t row = 0; row < rows; ++row) {
            int64_t b = row / n, t = row % n;
            double *dqr = dq + row * HI * DI, *dwr = dw + row * HI;
            for (int64_t i = 0; i < (int64_t)HI * DI; ++i)
                dqr[i] = 0.0;
            for (int j = 0; j < HI; ++j)
                dwr[j] = 0.0;
            loss[row] = 0.0;
            if (want_mag) {
                loss_mag[row] = 0.0;
                for (int64_t i = 0; i < (int64_t)HI * DI; ++i) {
                    dq_mag[row * HI * DI + i] = 0.0;
                    dq_kink[row * HI * DI + i] = 0.0;
                }
                for (int j = 0; j < HI; ++j)
                    dw_mag[row * HI + j] = 0.0;
            }
            const int32_t *Sr = S + row * k;
            const float *pr = p + row * k;
            load_token(dt, qI, q_scale, row, (int64_t)HI * DI, q);
            for (int j = 0; j < HI; ++j)
                w[j] = (double)wI[row * HI + j];
            /* eq.(1) on the valid slots, keeping every q_j . k dot product */
            double pmass = 0.0, imax = -INFINITY;
            int nvalid = 0;
            for (int i = 0; i < k; ++i) {
                valid[i] = Sr[i] >= 0 && Sr[i] <= t;
                if (!valid[i])
                    continue;
                ++nvalid;
                load_token(dt, kI, k_scale, b * n + Sr[i], DI, keys + (int64_t)i * DI);
                double sc = 0.0;
                for (int j = 0; j < HI; ++j) {
                    double dot = 0.0, adot = 0.0;
                    for (int d = 0; d < DI; ++d) {
                        dot += q[(int64_t)j * DI + d] * keys[(int64_t)i * DI + d];
                        adot += fabs(q[(int64_t)j * DI + d] * keys[(int64_t)i * DI + d]);
                    }
                    X[(int64_t)i * HI + j] = dot;
                    band[(int64_t)i * HI + j] = (double)DI * ldexp(1.0, -24) * adot;
                    sc += w[j] * (dot > 0.0 ? dot : 0.0);
                }
                I[i] = sc;
                pmass += (double)pr[i];
                if (sc > imax)
                    imax = sc;
            }
            if (nvalid == 0 || !(pmass > 0.0))
                continue;
            /* both distributions normalised over the valid slots */
            double z = 0.0;
            for (int i = 0; i < k; ++i)
                if (valid[i])
                    z += exp(I[i] - imax);
            const double logz = imax + log(z);
            double L = 0.0;
            for (int i = 0; i < k; ++i) {
                if (!valid[i]) {
                    g[i] = 0.0;
                    continue;
                }
                const double P = (double)pr[i] / pmass;
                const double logR = I[i] - logz;
                if (P > 0.0)
                    L += P * (log(P) - logR);
                g[i] = exp(logR) - P;
                R[i] = exp(logR);
                Pn[i] = P;
                if (want_mag && P > 0.0)
                    loss_mag[row] += P * (fabs(log(P)) + fabs(logR));
            }
            loss[row] = L;
            /* the chain rule through eq.(1) */
            for (int i = 0; i < k; ++i) {
                if (!valid[i])
                    continue;
                const double *ki = keys + (int64_t)i * DI;
                double *dks = mydk + (b * n + Sr[i]) * DI;
                for (int j = 0; j < HI; ++j) {
                    const double x = X[(int64_t)i * HI + j];
                    dwr[j] += g[i] * (x > 0.0 ? x : 0.0);
                    if (want_mag) {
                        dw_mag[row * HI + j] += (R[i] + Pn[i]) * (x > 0.0 ? x : 0.0);
                        if (fabs(x) <= band[(int64_t)i * HI + j]) {
                            const double cm = (R[i] + Pn[i]) * fabs(w[j]);
                            double *dkk = mydkk + (b * n + Sr[i]) * DI;
                            for (int d = 0; d < DI; ++d) {
                                dq_kink[row * HI * DI + (int64_t)j * DI + d] += cm * fabs(ki[d]);
                                dkk[d] += cm * fabs(q[(int64_t)j * DI + d]);
                            }
                        }
                    }
                    if (!(x > 0.0))
                        continue;
                    const double c = g[i] * w[j];
                    for (int d = 0; d < DI; ++d) {
                        dqr[(int64_t)j * DI + d] += c * ki[d];
                        dks[d] += c * q[(int64_t)j * DI + d];
                    }
                    if (want_mag) {
                        const double cm = (R[i] + Pn[i]) * fabs(w[j]);
                        double *dkm = mydkm + (b * n + Sr[i]) * DI;
                        for (int d = 0; d < DI; ++d) {
                            dq_mag[row * HI * DI + (int64_t)j * DI + d] += cm * fabs(ki[d]);
                            dkm[d] += cm * fabs(q[(int64_t)j * DI + d]);
                        }
                    }
                }
            }
        }
        free(q);
        free(w);
        free(keys);
        free(X);
        free(I);
        free(g);
        free(valid);
        free(R);
        free(Pn);
        free(band);
    }
    for (int64_t i = 0; i < rows * DI; ++i) {
        double acc = 0.0, accm = 0.0, acck = 0.0;
        for (int th = 0; th < nth; ++th) {
            acc += dk_part[(size_t)th * rows * DI + i];
            if (want_mag) {
                accm += dk_part[((size_t)nth + th) * rows * DI + i];
                acck += dk_part[((size_t)2 * nth + th) * rows * DI + i];
            }
        }
        dk[i] = acc;
        if (want_mag) {
            dk_mag[i] = accm;
            dk_kink[i] = acck;
        }
    }
    free(dk_part);
    return 0;
}

/* ---- coarse recall, then re-rank (DSA page, section 2, the paragraph on the
 * quantised key cache: recall a larger candidate set at FP8, then rank it with
 * a higher-precision indexer) ----------------------------------------------
 *
 * For each listed row (flattened b*n + t) the candidates are the valid entries
 * of C[r, 0..kc) (0 <= C <= t, each counted once); their scores are eq.(1) on
 * the fine inputs (dt_fine), and the min(k, #candidates) best by (score desc,
 * position asc) are written in ascending position order, then -1;
 * S_score holds each slot's fine score (-inf for padding). */
int ora_rerank_rows(int dt_fine, const void *qI, const void *kI, const float *wI, int B, int n,
                    int HI, int DI, const int64_t *rows, int nrows, const int32_t *C, int kc, int k,
                    int32_t *S, float *S_score)
{
    if (!qI || !kI || !wI || !rows || !C || !S || B <= 0 || n <= 0 || HI <= 0 || DI <= 0 || kc <= 0 ||
        k <= 0 || dt_fine == ORA_FP8)
        return -1;
    if (!rows_ok(rows, nrows, (int64_t)B * n))
        return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < nrows; ++r) {
        const int64_t row = rows[r], b = row / n, t = row % n;
        double *q = malloc(sizeof(double) * (size_t)HI * DI);
        double *w = malloc(sizeof(double) * (size_t)HI);
        double *kk = malloc(sizeof(double) * (size_t)DI);
        ora_cand *c = malloc(sizeof(ora_cand) * (size_t)kc);
        char *seen = calloc((size_t)t + 1, 1);
        load_token(dt_fine, qI, NULL, row, (int64_t)HI * DI, q);
        for (int j = 0; j < HI; ++j)
            w[j] = (double)wI[row * HI + j];
        int nc = 0;
        for (int i = 0; i < kc; ++i) {
            const int32_t s = C[(int64_t)r * kc + i];
            if (s < 0 || s > t || seen[s])
                continue;
            seen[s] = 1;
            load_token(dt_fine, kI, NULL, b * n + s, DI, kk);
            c[nc].score = (float)indexer_score(q, w, kk, HI, DI, NULL);
            c[nc].pos = s;
            ++nc;
        }
        const int K = nc < k ? nc : k;
        qsort(c, (size_t)nc, sizeof(ora_cand), cmp_rank);
        qsort(c, (size_t)K, sizeof(ora_cand), cmp_pos);
        for (int i = 0; i < k; ++i) {
            S[(int64_t)r * k + i] = i < K ? c[i].pos : -1;
            if (S_score)
                S_score[(int64_t)r * k + i] = i < K ? c[i].score : -INFINITY;
        }
        free(q);
        free(w);
        free(kk);
        free(c);
        free(seen);
    }
    return 0;
}

/* ---- selection-quality diagnostics (DSA page, sections 1.2 and 3.1) -----
 *
 * For row r, teacher masses a[0..L) (L = row_len[r], at row_start[r]) and a
 * selection S_r (k slots; entries outside [0, L) are not selected, a repeated
 * entry counts once):
 *   G       = TopK(a, min(m, L)) by the rule of eq.(2) (ties to the lower
 *             position)
 *   recall  = |G n S_r| / |G|                      eq.(9); eq.(14) is m = k
 *   mass    = sum_{s in S_r} a_s / sum_{s < L} a_s  eq.(15) with the teacher
 *             normalised over the row
 * recall is NaN when G is empty, mass when the row's total is not positive. */
int ora_selection_quality(const float *teacher, const int64_t *row_start, const int32_t *row_len,
                          int R, const int32_t *S, int k, int m, double *recall, double *mass)
{
    if (!teacher || !row_start || !row_len || !S || !recall || !mass || R < 0 || k <= 0 || m <= 0)
        return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < R; ++r) {
        const int64_t L = row_len[r] > 0 ? row_len[r] : 0;
        const float *a = teacher + row_start[r];
        const int32_t *Sr = S + (int64_t)r * k;
        char *in_s = calloc((size_t)(L > 0 ? L : 1), 1);
        for (int i = 0; i < k; ++i)
            if (Sr[i] >= 0 && Sr[i] < L)
                in_s[Sr[i]] = 1;
        double total = 0.0, covered = 0.0;
        for (int64_t s = 0; s < L; ++s) {
            total += (double)a[s];
            if (in_s[s])
                covered += (double)a[s];
        }
        mass[r] = total > 0.0 ? covered / total : NAN;
        int32_t *G = malloc(sizeof(int32_t) * (size_t)m);
        select_row(a, L, m, G, NULL);
        int64_t ng = 0, hit = 0;
        for (int i = 0; i < m; ++i) {
            if (G[i] < 0)
                continue;
            ++ng;
            hit += in_s[G[i]];
        }
        recall[r] = ng > 0 ? (double)hit / (double)ng : NAN;
        free(G);
        free(in_s);
    }
    return 0;
}

/* eq.(18): the cutoff margin s_(K) - s_(K+1) of each score row, K = min(k, L),
 * s_(1) >= s_(2) >= ... the row's scores in descending order; +inf when the
 * row has no (K+1)-th score (L <= k). */
int ora_cutoff_margin(const float *scores, const int64_t *row_start, const int32_t *row_len, int R,
                      int k, double *margin)
{
    if (!scores || !row_start || !row_len || !margin || R < 0 || k <= 0)
        return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < R; ++r) {
        const int64_t L = row_len[r] > 0 ? row_len[r] : 0;
        if (L <= k) {
            margin[r] = INFINITY;
            continue;
        }
        ora_cand *c = malloc(sizeof(ora_cand) * (size_t)L);
        for (int64_t s = 0; s < L; ++s) {
            c[s].score = scores[row_start[r] + s];
            c[s].pos = (int32_t)s;
        }
        qsort(c, (size_t)L, sizeof(ora_cand), cmp_rank);
        margin[r] = (double)c[k - 1].score - (double)c[k].score;
        free(c);
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
