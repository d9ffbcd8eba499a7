// topk_common.h -- workgroup-level exact top-k of one score row with the
// lower-position tie rule (DSA page, section 1.1 eq.(2); section 2 notes radix
// top-k with variable-length rows).
#pragma once

#include "tlsl_device.h"

namespace tlsl {

constexpr int TK_LCAP = 8192;  // candidate keys gathered into LDS once a bin is this small

struct TopkSmem {
    uint32_t hist[2048];
    uint32_t lkeys[TK_LCAP];
    int scratch[64];
    int lcnt;
};

// Radix digits of the 32-bit score key, most significant first.
__device__ __forceinline__ int radix_shift(int p) { return p == 0 ? 21 : (p == 1 ? 10 : 0); }
__device__ __forceinline__ uint32_t radix_mask(int p) { return p == 2 ? 0x3ffu : 0x7ffu; }

// ---------------------------------------------------------------------------
// need-th largest (1 <= need <= number of keys) of the keys a workgroup of NT
// threads holds between them: each(f) calls f(key) for every key the calling
// thread holds (every key held by exactly one thread; the keys may sit in
// registers or in workgroup-visible memory) and is called up to five times.
// Returns the key T and *gt = number of keys above T.
//
// One histogram pass over the keys' own span [lo, hi] (2048 bins of 2^s keys)
// finds the bin holding the result; the few keys of that bin are then ranked
// against each other.  A bin with more than SEL_BLMAX keys (a span dominated
// by near-equal keys) falls back to three radix passes over the full key.
// exact = false stops after the histogram and returns the bin's lower edge, a
// lower bound of the need-th largest key (*gt is then not set); the bound is
// loose when the span is wide (2048 bins over keys of both signs).
// Ends with a barrier, so `sm` may be reused right away.
// ---------------------------------------------------------------------------
constexpr int SEL_BLMAX = 256;

struct SelectSmem {
    uint32_t hist[2048];
    uint32_t blist[SEL_BLMAX];
    int scratch[64];
    int bcnt, gsh;
    uint32_t tsh;
};

template <int NT, class Each>
__device__ uint32_t block_select_each(int need, Each each, SelectSmem& sm, int* gt_out, bool exact) {
    const int tid = threadIdx.x;
    uint32_t lo = 0xffffffffu, hi = 0u;
    each([&](uint32_t k) {
        lo = min(lo, k);
        hi = max(hi, k);
    });
    block_minmax_u32<NT>(&lo, &hi, sm.scratch);
    const uint32_t span = hi - lo;
    const int s = span < 2048u ? 0 : (32 - __clz(span)) - 11;
    for (int i = tid; i < 2048; i += NT) sm.hist[i] = 0;
    if (tid == 0) sm.bcnt = 0;
    __syncthreads();
    each([&](uint32_t k) { atomicAdd(&sm.hist[(k - lo) >> s], 1u); });
    __syncthreads();
    int above;
    const int d = block_find_bin<NT, 2048>(sm.hist, need, &above, sm.scratch);
    const uint32_t edge = lo + ((uint32_t)d << s);
    if (!exact) return edge;
    const int nb = (int)sm.hist[d];
    const int rank = need - above;  // inside bin d
    __syncthreads();  // every thread holds nb before the fallback clears hist
    uint32_t T;
    int gt;
    if (s == 0) {
        T = edge;
        gt = above;
    } else if (nb <= SEL_BLMAX) {
        each([&](uint32_t k) {
            if (((k - lo) >> s) == (uint32_t)d) sm.blist[atomicAdd(&sm.bcnt, 1)] = k;
        });
        __syncthreads();
        if (tid < nb) {
            const uint32_t kj = sm.blist[tid];
            int g = 0, e = 0;
            for (int m = 0; m < nb; ++m) {
                const uint32_t km = sm.blist[m];
                g += km > kj;
                e += km == kj;
            }
            if (g < rank && rank <= g + e) {  // equal keys write equal values
                sm.tsh = kj;
                sm.gsh = above + g;
            }
        }
        __syncthreads();
        T = sm.tsh;
        gt = sm.gsh;
    } else {
        uint32_t prefix = 0, pmask = 0;
        int left = need;
        gt = 0;
        for (int p = 0; p < 3; ++p) {
            const int sh = radix_shift(p);
            const uint32_t dm = radix_mask(p);
            for (int i = tid; i < 2048; i += NT) sm.hist[i] = 0;
            __syncthreads();
            each([&](uint32_t k) {
                if ((k & pmask) == prefix) atomicAdd(&sm.hist[(k >> sh) & dm], 1u);
            });
            __syncthreads();
            int ab;
            const int dd = block_find_bin<NT, 2048>(sm.hist, left, &ab, sm.scratch);
            gt += ab;
            left -= ab;
            prefix |= (uint32_t)dd << sh;
            pmask |= dm << sh;
        }
        T = prefix;
    }
    __syncthreads();
    *gt_out = gt;
    return T;
}

// Keys in workgroup-visible memory: key_of(i, &valid) for i < cnt, read by
// thread i % NT.
template <int NT, class KeyFn>
__device__ uint32_t block_select_adaptive(int cnt, int need, KeyFn key_of, SelectSmem& sm, int* gt_out,
                                          bool exact = true) {
    const auto each = [&](auto&& f) {
        for (int i = threadIdx.x; i < cnt; i += NT) {
            bool ok;
            const uint32_t k = key_of(i, &ok);
            if (ok) f(k);
        }
    };
    return block_select_each<NT>(need, each, sm, gt_out, exact);
}

// Exact selection of the K = min(k, L) best of sc[0..L) ordered by (score desc,
// position asc).  Writes S[0..k): the selected positions ascending, then -1;
// Ss (optional): each slot's score, -inf for unused slots.  All NT threads of
// the workgroup call it; `sc` must be visible to the whole workgroup.
//
// Method: three radix passes over the score key (11, 11, 10 bits) find the
// K-th largest key T and the count gt of keys above it; once the candidate
// bin holds at most TK_LCAP keys the remaining passes run on an LDS copy.
// A final in-order pass keeps every key > T and the first K - gt keys == T
// (lowest positions first).
template <int NT>
__device__ void block_topk_row(const float* __restrict__ sc, int L, int k, int32_t* __restrict__ S,
                               float* __restrict__ Ss, TopkSmem& sm) {
    const int tid = threadIdx.x;
    const int K = min(k, L);
    if (L <= k) {
        for (int i = tid; i < k; i += NT) {
            S[i] = i < L ? i : -1;
            if (Ss) Ss[i] = i < L ? sc[i] : -INFINITY;
        }
        return;
    }
    uint32_t prefix = 0, pmask = 0;
    int need = K, gt = 0, lcnt = 0;
    bool in_lds = false;
    for (int p = 0; p < 3; ++p) {
        const int sh = radix_shift(p);
        const uint32_t dm = radix_mask(p);
        for (int i = tid; i < 2048; i += NT) sm.hist[i] = 0;
        __syncthreads();
        if (!in_lds) {
            for (int i = tid; i < L; i += NT) {
                uint32_t key = score_key(sc[i]);
                if ((key & pmask) == prefix) atomicAdd(&sm.hist[(key >> sh) & dm], 1u);
            }
        } else {
            for (int i = tid; i < lcnt; i += NT) {
                uint32_t key = sm.lkeys[i];
                if ((key & pmask) == prefix) atomicAdd(&sm.hist[(key >> sh) & dm], 1u);
            }
        }
        __syncthreads();
        int above;
        const int d = block_find_bin<NT, 2048>(sm.hist, need, &above, sm.scratch);
        const int cd = (int)sm.hist[d];
        gt += above;
        need -= above;
        prefix |= (uint32_t)d << sh;
        pmask |= dm << sh;
        if (p < 2 && !in_lds && cd <= TK_LCAP) {
            if (tid == 0) sm.lcnt = 0;
            __syncthreads();
            for (int i = tid; i < L; i += NT) {
                uint32_t key = score_key(sc[i]);
                if ((key & pmask) == prefix) sm.lkeys[atomicAdd(&sm.lcnt, 1)] = key;
            }
            __syncthreads();
            lcnt = sm.lcnt;
            in_lds = true;
        }
        __syncthreads();
    }
    const uint32_t T = prefix;
    const int need_ties = K - gt;
    int run_sel = 0, run_tie = 0;
    for (int base = 0; base < L && run_sel < K; base += NT) {
        const int i = base + tid;
        const bool v = i < L;
        const float s = v ? sc[i] : 0.f;
        const uint32_t key = v ? score_key(s) : 0u;
        const bool isgt = v && key > T, istie = v && key == T;
        int rt, rdum, tt, tdum;
        block_scan2<NT>(istie, false, &rt, &rdum, &tt, &tdum, sm.scratch);
        const bool sel = isgt || (istie && run_tie + rt < need_ties);
        int rs, ts;
        block_scan2<NT>(sel, false, &rs, &rdum, &ts, &tdum, sm.scratch);
        if (sel) {
            S[run_sel + rs] = i;
            if (Ss) Ss[run_sel + rs] = s;
        }
        run_sel += ts;
        run_tie += tt;
    }
    for (int i = K + tid; i < k; i += NT) {
        S[i] = -1;
        if (Ss) Ss[i] = -INFINITY;
    }
}

}  // namespace tlsl
