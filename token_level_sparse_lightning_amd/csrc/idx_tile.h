// idx_tile.h -- the Lightning Indexer scoring tile (DSA page, section 1.1
// eq.(1)) shared by every kernel that computes indexer scores: the prefill
// and decode scans and the training step's recompute.  One fixed sequence of
// matrix-core products, ReLU, weighted head sum and lane-group reduction, so
// every caller gets bit-identical scores for the same query and key.
//
// fp8 inputs use the identity w ReLU(x) = (w x + w |x|) / 2.  The epilogue is
// one FMA with an |x| operand per (head, key) (no separate max), and the
// linear part sum_j (w_j / 2) q_j . k = qbar . k comes from one more
// matrix-core product per 16-key block: qbar is split into 8 fp8 rows with
// power-of-two scales (each split takes the residual of the previous ones,
// so the 8 together carry qbar to ~2^-24 of its largest element), and those
// rows, for up to two queries at once, are the A operand of the product.
#pragma once

#include "tlsl_device.h"

namespace tlsl {

// ---------------------------------------------------------------------------
// Scoring tile shared by every indexer kernel.
// ---------------------------------------------------------------------------
template <int DT, int HB, int DI>
struct Idx {
    using M = Mma<DT, DI>;
    static constexpr int NCH = M::NCH;
    static constexpr int ROWB = M::ROWB;

    // Query fragment of one token (HB blocks of 16 heads) and the lane's head
    // weights (rows 4g..4g+3 of each block), pre-multiplied by the token scale
    // (fp8: and by 1/2, the weight of the |x| part).
    __device__ __forceinline__ static void load_query(const unsigned char* q_tok, const float* w_tok,
                                                      float wmul, int HI, bool valid,
                                                      uint4 (&qf)[HB][NCH], float (&wv)[HB][4]) {
        const int l = lane_id(), g = l >> 4, c = l & 15;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
            const int h = 16 * hb + c;
            const bool ok = valid && h < HI;
            const uint4* src = reinterpret_cast<const uint4*>(q_tok + (size_t)(ok ? h : 0) * ROWB + g * (ROWB / 4));
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) qf[hb][ch] = ok ? src[ch] : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int hh = 16 * hb + 4 * g + r;
                wv[hb][r] = (valid && hh < HI) ? w_tok[hh] * wmul * (DT == kFP8 ? 0.5f : 1.f) : 0.f;
            }
        }
    }

    // Products of one query's head blocks with key block kb (accumulators
    // start at zero; the HB head blocks are independent accumulation chains,
    // interleaved step by step).
    __device__ __forceinline__ static void products(const uint4 (&qf)[HB][NCH], const uint4 (&kfb)[NCH],
                                                    v4f (&A)[HB]) {
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) A[hb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < M::STEPS; ++st)
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) A[hb] = M::step(qf[hb], kfb, st, A[hb]);
    }
    // ReLU, head weights and the lane's part of the head sum of one key block.
    __device__ __forceinline__ static float epilogue(const float (&wv)[HB][4], const v4f (&A)[HB]) {
        float p = 0.f;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int r = 0; r < 4; ++r) p = __builtin_fmaf(wv[hb][r], relu(A[hb][r]), p);
        return p;
    }

    // Scores of one query against a 64-key subtile whose key fragments are
    // kf[kb] (keys 16*kb + (l & 15)), in two parts: score_head() runs the
    // products of the four key blocks and the epilogues of the first three
    // (accumulators alternate between two sets, so the epilogue of key block
    // kb runs while the products of kb+1 are in flight) and leaves the last
    // block's products in `last`; score_tail() finishes.  score() is the two
    // back to back.  Lane l receives key l's score (before the key scale); the
    // operations and their order are fixed, so every caller gets bit-identical
    // scores.
    __device__ __forceinline__ static void score_head(const uint4 (&qf)[HB][NCH], const float (&wv)[HB][4],
                                                      const uint4 (&kf)[4][NCH], float (&part)[3],
                                                      v4f (&last)[HB]) {
        v4f acc[HB];
        products(qf, kf[0], acc);
        products(qf, kf[1], last);
        part[0] = epilogue(wv, acc);
        products(qf, kf[2], acc);
        part[1] = epilogue(wv, last);
        products(qf, kf[3], last);
        part[2] = epilogue(wv, acc);
    }
    __device__ __forceinline__ static float score_tail(const float (&wv)[HB][4], const float (&part)[3],
                                                       const v4f (&last)[HB]) {
        const float p[4] = {part[0], part[1], part[2], epilogue(wv, last)};
        return reduce_heads_64(p);
    }
    __device__ __forceinline__ static float score(const uint4 (&qf)[HB][NCH], const float (&wv)[HB][4],
                                                  const uint4 (&kf)[4][NCH]) {
        float part[3];
        v4f last[HB];
        score_head(qf, wv, kf, part, last);
        return score_tail(wv, part, last);
    }

    // The same scores with one accumulator set (fewer registers, more waves
    // per SIMD; for the bandwidth-bound scan).  Identical summation order, so
    // the results are bit-identical to score().
    __device__ __forceinline__ static float score_lean(const uint4 (&qf)[HB][NCH], const float (&wv)[HB][4],
                                                       const uint4 (&kf)[4][NCH]) {
        float part[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            v4f acc[HB];
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) acc[hb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < M::STEPS; ++st)
#pragma unroll
                for (int hb = 0; hb < HB; ++hb) acc[hb] = M::step(qf[hb], kf[kb], st, acc[hb]);
            float p = 0.f;
#pragma unroll
            for (int hb = 0; hb < HB; ++hb)
#pragma unroll
                for (int r = 0; r < 4; ++r) p = __builtin_fmaf(wv[hb][r], relu(acc[hb][r]), p);
            part[kb] = p;
        }
        return reduce_heads_64(part);
    }

    // ---- fp8: linear part of w ReLU(x) = (w x + w |x|) / 2 --------------------
    // Scratch of one query's linear-part rows (LDS): 8 split rows of DI fp8
    // codes, then their 8 scales.
    static constexpr int LIN_SPLITS = 8;
    static constexpr int LIN_SCRATCH = LIN_SPLITS * DI + LIN_SPLITS * 4;

    // qbar = sum_h (w_h wmul / 2) q_h of the query whose fragments are qf (as
    // load_query leaves them), and its splits, into scr.  Lane (g, c) first
    // sums its own heads 16 hb + c over its 32 dims (hb ascending), then the
    // 16 lanes of group g combine by recursive halving (partners 8, 4, 2, 1
    // apart), which leaves lane (g, c) with dims 32 g + 2 c and 32 g + 2 c + 1.
    // Split j: scale 2^e with the row's largest residual in [128, 256) times
    // 2^e, codes = fp8(residual / 2^e), residual -= codes * 2^e (exact).
    __device__ static void prep_lin(const uint4 (&qf)[HB][NCH], const float* w_tok, float wmul, int HI, bool valid,
                                    unsigned char* scr) {
        static_assert(DT == kFP8 && DI == 128, "the linear part is the fp8 path's (d^I = 128)");
        const int l = lane_id(), g = l >> 4, c = l & 15;
        float p[32];
#pragma unroll
        for (int d = 0; d < 32; ++d) p[d] = 0.f;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
            const int h = 16 * hb + c;
            const float wh = (valid && h < HI) ? w_tok[h] * wmul * 0.5f : 0.f;
#pragma unroll
            for (int ch = 0; ch < 2; ++ch) {
                const uint32_t u[4] = {qf[hb][ch].x, qf[hb][ch].y, qf[hb][ch].z, qf[hb][ch].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)u[e], false);
                    const v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)u[e], true);
                    const int d = 16 * ch + 4 * e;
                    p[d] = __builtin_fmaf(wh, lo[0], p[d]);
                    p[d + 1] = __builtin_fmaf(wh, lo[1], p[d + 1]);
                    p[d + 2] = __builtin_fmaf(wh, hi[0], p[d + 2]);
                    p[d + 3] = __builtin_fmaf(wh, hi[1], p[d + 3]);
                }
            }
        }
        // recursive halving over the 16 lanes of the group
#pragma unroll
        for (int half = 32, dist = 8; dist >= 1; half >>= 1, dist >>= 1) {
            const bool upper = (c & dist) != 0;  // keep the upper half of the live range
#pragma unroll
            for (int i = 0; i < half / 2; ++i) {
                const float give = upper ? p[i] : p[half / 2 + i];
                const float keep = upper ? p[half / 2 + i] : p[i];
                p[i] = keep + __shfl_xor(give, dist, 64);
            }
        }
        float r0 = p[0], r1 = p[1];
#pragma unroll
        for (int j = 0; j < LIN_SPLITS; ++j) {
            const float m = wave_max(fmaxf(fabsf(r0), fabsf(r1)));
            int code = 0;
            float sc = 0.f;
            if (m > 0.f) {
                int E;
                (void)frexpf(m, &E);
                const int sh = E - 8;  // m / 2^sh in [128, 256): inside the e4m3 range
                code = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(r0, -sh), ldexpf(r1, -sh), 0, false);
                const v2f back = __builtin_amdgcn_cvt_pk_f32_fp8(code, false);
                r0 -= ldexpf(back[0], sh);
                r1 -= ldexpf(back[1], sh);
                sc = ldexpf(1.f, sh);
            }
            *reinterpret_cast<uint16_t*>(scr + j * DI + 32 * g + 2 * c) = (uint16_t)(code & 0xffff);
            if (l == 0) reinterpret_cast<float*>(scr + LIN_SPLITS * DI)[j] = sc;
        }
    }

    // The A fragment of the linear-part product for the queries of slot 0
    // (scr0) and slot 1 (scr1, or null: rows of zeros): lane (g, c) holds row
    // c, i.e. split 2 (c >> 2) + (c & 1) of slot (c >> 1) & 1; output rows
    // 4 g + {0, 1} then belong to slot 0 (splits 2 g, 2 g + 1) and rows
    // 4 g + {2, 3} to slot 1.  ls[s] are the lane's two scales of slot s.
    __device__ __forceinline__ static void load_lin(const unsigned char* scr0, const unsigned char* scr1,
                                                    uint4 (&ql)[NCH], float (&ls)[2][2]) {
        const int l = lane_id(), g = l >> 4, c = l & 15;
        const int slot = (c >> 1) & 1, split = 2 * (c >> 2) + (c & 1);
        const unsigned char* scr = slot ? scr1 : scr0;
        if (scr) {
            const uint4* src = reinterpret_cast<const uint4*>(scr + split * DI + 32 * g);
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) ql[ch] = src[ch];
        } else {
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) ql[ch] = make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const unsigned char* sp = s ? scr1 : scr0;
            const float* scl = reinterpret_cast<const float*>((sp ? sp : scr0) + LIN_SPLITS * DI);
            ls[s][0] = sp ? scl[2 * g] : 0.f;
            ls[s][1] = sp ? scl[2 * g + 1] : 0.f;
        }
    }

    // Linear-part products of the four key blocks (rows as load_lin).
    __device__ __forceinline__ static void lin_products(const uint4 (&ql)[NCH], const uint4 (&kf)[4][NCH],
                                                        v4f (&lin)[4]) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            lin[kb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < M::STEPS; ++st) lin[kb] = M::step(ql, kf[kb], st, lin[kb]);
        }
    }
    // fp8 epilogue of one key block: the slot's two scaled linear rows, then
    // one FMA with |x| per head (wv holds w/2, times the query scale).
    __device__ __forceinline__ static float epilogue_lin(const float (&wv)[HB][4], const v4f (&A)[HB], float l0,
                                                         float l1, const float (&ls)[2]) {
        float p = ls[0] * l0;
        p = __builtin_fmaf(ls[1], l1, p);
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int r = 0; r < 4; ++r) p = __builtin_fmaf(wv[hb][r], fabsf(A[hb][r]), p);
        return p;
    }
    // score_head / score_tail / score / score_lean for fp8: the query in
    // linear-part slot SLOT (lin: lin_products of the subtile).
    template <int SLOT>
    __device__ __forceinline__ static void score_head_lin(const uint4 (&qf)[HB][NCH], const float (&wv)[HB][4],
                                                          const uint4 (&kf)[4][NCH], const v4f (&lin)[4],
                                                          const float (&ls)[2], float (&part)[3], v4f (&last)[HB]) {
        v4f acc[HB];
        products(qf, kf[0], acc);
        products(qf, kf[1], last);
        part[0] = epilogue_lin(wv, acc, lin[0][2 * SLOT], lin[0][2 * SLOT + 1], ls);
        products(qf, kf[2], acc);
        part[1] = epilogue_lin(wv, last, lin[1][2 * SLOT], lin[1][2 * SLOT + 1], ls);
        products(qf, kf[3], last);
        part[2] = epilogue_lin(wv, acc, lin[2][2 * SLOT], lin[2][2 * SLOT + 1], ls);
    }
    __device__ __forceinline__ static float score_tail_lin(const float (&wv)[HB][4], const float (&part)[3],
                                                           const v4f (&last)[HB], float l0, float l1,
                                                           const float (&ls)[2]) {
        const float p[4] = {part[0], part[1], part[2], epilogue_lin(wv, last, l0, l1, ls)};
        return reduce_heads_64(p);
    }
    template <int SLOT>
    __device__ __forceinline__ static float score_lin(const uint4 (&qf)[HB][NCH], const float (&wv)[HB][4],
                                                      const uint4 (&kf)[4][NCH], const v4f (&lin)[4],
                                                      const float (&ls)[2]) {
        float part[3];
        v4f last[HB];
        score_head_lin<SLOT>(qf, wv, kf, lin, ls, part, last);
        return score_tail_lin(wv, part, last, lin[3][2 * SLOT], lin[3][2 * SLOT + 1], ls);
    }
    // one accumulator set, slot 0 (the decode scan); same operations and order
    __device__ __forceinline__ static float score_lean_lin(const uint4 (&qf)[HB][NCH], const float (&wv)[HB][4],
                                                           const uint4 (&kf)[4][NCH], const uint4 (&ql)[NCH],
                                                           const float (&ls)[2]) {
        float part[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            v4f lin = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < M::STEPS; ++st) lin = M::step(ql, kf[kb], st, lin);
            v4f acc[HB];
            products(qf, kf[kb], acc);
            part[kb] = epilogue_lin(wv, acc, lin[0], lin[1], ls);
        }
        return reduce_heads_64(part);
    }

    // Key fragments of keys key0 + 16*kb + (l & 15), rows clamped to last,
    // straight from global memory.
    __device__ __forceinline__ static void load_keys_global(const unsigned char* kbase, int key0, int last,
                                                            uint4 (&kf)[4][NCH]) {
        const int l = lane_id(), g = l >> 4, c = l & 15;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const int key = min(key0 + 16 * kb + c, last);
            const uint4* src = reinterpret_cast<const uint4*>(kbase + (size_t)key * ROWB + g * (ROWB / 4));
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) kf[kb][ch] = src[ch];
        }
    }
};

}  // namespace tlsl
