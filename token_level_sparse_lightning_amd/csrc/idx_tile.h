// idx_tile.h -- the Lightning Indexer scoring tile (DSA page, section 1.1
// eq.(1)) shared by every kernel that computes indexer scores: the prefill
// and decode scans and the training step's recompute.  One fixed sequence of
// matrix-core products, ReLU, weighted head sum and lane-group reduction, so
// every caller gets bit-identical scores for the same query and key.
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
    // weights (rows 4g..4g+3 of each block), pre-multiplied by the token scale.
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
                wv[hb][r] = (valid && hh < HI) ? w_tok[hh] * wmul : 0.f;
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
