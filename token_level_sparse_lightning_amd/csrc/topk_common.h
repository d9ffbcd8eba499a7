// topk_common.h -- workgroup-level exact top-k of one score row with the
// lower-position tie rule (DSA page, section 1.1 eq.(2); section 2 notes radix
// top-k with variable-length rows).
#pragma once

#include "tlsl_device.h"

namespace tlsl {

constexpr int TK_LCAP = 8192;          // candidate keys gathered into LDS once a bin is this small
constexpr int TK_BITMAP_WORDS = 4096;  // rows up to 131072 positions use the bitmap path

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
// by near-equal keys) becomes the range of a further level, tightened to its
// keys' min and max (at most three more levels; a bin of equal keys ends at
// once).  exact = false stops after the first histogram and returns the bin's
// lower edge, a lower bound of the need-th largest key (*gt is then not set);
// the bound is loose when the span is wide (2048 bins over keys of both
// signs).  Ends with a barrier, so `sm` may be reused right away.
// ---------------------------------------------------------------------------
constexpr int SEL_BLMAX = 256;

struct SelectSmem {
    uint32_t hist[2048];
    uint32_t blist[SEL_BLMAX];
    int scratch[64];
    int bcnt, gsh;
    uint32_t tsh;
};

// Shared memory of block_topk_row: the radix path's histogram and LDS key
// copy, or the bitmap path's select state and position bitmap.
struct TopkSmem {
    union {
        struct {
            uint32_t hist[2048];
            uint32_t lkeys[TK_LCAP];
            int scratch[64];
            int lcnt;
        } r;
        struct {
            SelectSmem sel;
            uint32_t bitmap[TK_BITMAP_WORDS];
            int nties;
        } b;
    };
};

// Exclusive scan of an int over the workgroup; scratch >= NT/64 + 1 ints.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* total, int* scratch) {
    constexpr int NW = NT / 64;
    const int w = threadIdx.x >> 6, l = lane_id();
    const int incl = wave_incl_scan(v);
    if (l == 63) scratch[w] = incl;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int c = scratch[i];
        if (i < w) base += c;
        tot += c;
    }
    __syncthreads();
    *total = tot;
    return base + incl - v;
}

// RUNS: count a run of keys falling in one bin with one atomic (for key sets
// with long runs of equal keys, e.g. a row of ties); otherwise one atomic per
// key, with no per-key branch.
template <int NT, bool RUNS = true, class Each>
__device__ uint32_t block_select_each(int need, Each each, SelectSmem& sm, int* gt_out, bool exact) {
    const int tid = threadIdx.x;
    uint32_t lo = 0xffffffffu, hi = 0u;
    each([&](uint32_t k) {
        lo = min(lo, k);
        hi = max(hi, k);
    });
    block_minmax_u32<NT>(&lo, &hi, sm.scratch);
    // Level by level: a histogram of the keys inside [lo, hi] over 2048 bins
    // of 2^s keys finds the bin d holding the need-th largest; a bin of at
    // most SEL_BLMAX keys is ranked directly, a larger one becomes the next
    // level's range (tightened to its keys' own min and max, so a bin of equal
    // keys ends the search at once).  Each level shrinks the span by 2^11.
    int gt = 0;  // keys above the current range
    uint32_t T = 0u;
    for (int level = 0;; ++level) {
        const uint32_t span = hi - lo;
        const int s = span < 2048u ? 0 : (32 - __clz(span)) - 11;
        for (int i = tid; i < 2048; i += NT) sm.hist[i] = 0;
        if (tid == 0) sm.bcnt = 0;
        __syncthreads();
        if (!RUNS && level == 0) {
            // every key lies in [lo, hi]
            each([&](uint32_t k) { atomicAdd(&sm.hist[(k - lo) >> s], 1u); });
        } else if (!RUNS) {
            each([&](uint32_t k) {
                if (k >= lo && k <= hi) atomicAdd(&sm.hist[(k - lo) >> s], 1u);
            });
        } else {
            // run-length counts: a thread adds a run of keys in one bin with
            // one atomic (a bin of many equal keys would otherwise serialise
            // every key of it on one LDS word)
            int cur = -1;
            uint32_t run = 0u;
            each([&](uint32_t k) {
                if (k >= lo && k <= hi) {
                    const int b = (int)((k - lo) >> s);
                    if (b != cur) {
                        if (run) atomicAdd(&sm.hist[cur], run);
                        cur = b;
                        run = 0u;
                    }
                    ++run;
                }
            });
            if (run) atomicAdd(&sm.hist[cur], run);
        }
        __syncthreads();
        int above;
        const int d = block_find_bin<NT, 2048>(sm.hist, need, &above, sm.scratch);
        const uint32_t edge = lo + ((uint32_t)d << s);
        if (!exact) return edge;  // a lower bound of the need-th largest key
        const int nb = (int)sm.hist[d];
        const int rank = need - above;  // inside bin d
        __syncthreads();  // every thread holds nb before hist is cleared again
        if (s == 0) {
            T = edge;
            gt += above;
            break;
        }
        const uint32_t bmask = ((uint32_t)1 << s) - 1u;
        const uint32_t bhi = edge > 0xffffffffu - bmask ? 0xffffffffu : edge + bmask;  // bin d's last key
        if (nb <= SEL_BLMAX) {
            each([&](uint32_t k) {
                if (k >= edge && k <= bhi) sm.blist[atomicAdd(&sm.bcnt, 1)] = k;
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
                    sm.gsh = g;
                }
            }
            __syncthreads();
            T = sm.tsh;
            gt += above + sm.gsh;
            break;
        }
        // next level: the keys of bin d, between their own min and max
        gt += above;
        need = rank;
        uint32_t nlo = 0xffffffffu, nhi = 0u;
        each([&](uint32_t k) {
            if (k >= edge && k <= bhi) {
                nlo = min(nlo, k);
                nhi = max(nhi, k);
            }
        });
        block_minmax_u32<NT>(&nlo, &nhi, sm.scratch);
        lo = nlo;
        hi = nhi;
    }
    __syncthreads();
    *gt_out = gt;
    return T;
}

// ---------------------------------------------------------------------------
// Exact top-K of `cnt` candidates held in registers, written in candidate
// order.  Candidate i (0 <= i < cnt) is item i / NT of thread i % NT, with its
// order-preserving score key and its position; candidates are in ascending
// position order, so "the lower position wins a tie" is "the earlier
// candidate wins".  Writes the K = min(k, ...) selected positions to S[0..K)
// (ascending), their scores to Ss (optional), then -1 / -inf up to S[topk).
// All NT threads call it; requires K <= cnt.
//
// The K-th largest key T comes from the register-visiting select; every key
// above T and the first K - gt keys equal to T are selected.  Per (item,
// wave) group the counts of both kinds, scanned in candidate order by the
// first wave, and each lane's rank inside its wave's ballot give every
// selected candidate its slot.
// ---------------------------------------------------------------------------
template <int NT, int SEG>
__device__ void select_ordered(const uint32_t (&key)[SEG], const int (&pos)[SEG], int cnt, int K, int topk,
                               int32_t* __restrict__ Srow, float* __restrict__ Ssrow, SelectSmem& sel,
                               int (&gcnt)[2][SEG * (NT / 64)]) {
    constexpr int NW = NT / 64;
    constexpr int NE = SEG * NW;  // (item, wave) groups, in candidate order
    const int tid = threadIdx.x, w = tid >> 6;
    // every candidate is kept when there are exactly K of them
    const bool all = cnt == K;
    uint32_t T = 0u;  // key of the K-th largest candidate
    int gt = cnt;     // candidates with a key above T
    if (!all) {
        const auto each = [&](auto&& f) {
#pragma unroll
            for (int u = 0; u < SEG; ++u)
                if (tid + u * NT < cnt) f(key[u]);
        };
        T = block_select_each<NT, false>(K, each, sel, &gt, true);
    }
    const int need_ties = K - gt;
#pragma unroll
    for (int u = 0; u < SEG; ++u) {
        const bool ok = tid + u * NT < cnt;
        const uint64_t mg = ballot(ok && (all || key[u] > T));
        const uint64_t mt = ballot(ok && !all && key[u] == T);
        if (lane_id() == 0) {
            gcnt[0][u * NW + w] = __popcll(mg);
            gcnt[1][u * NW + w] = __popcll(mt);
        }
    }
    __syncthreads();
    if (w == 0) {
        // exclusive scan of the NE group counts by the first wave
        constexpr int PER = (NE + 63) / 64;
        const int l = lane_id();
        int cg[PER], ct[PER], sg = 0, st = 0;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int e = l * PER + j;
            cg[j] = e < NE ? gcnt[0][e] : 0;
            ct[j] = e < NE ? gcnt[1][e] : 0;
            sg += cg[j];
            st += ct[j];
        }
        int eg = wave_incl_scan(sg) - sg, et = wave_incl_scan(st) - st;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int e = l * PER + j;
            if (e < NE) {
                gcnt[0][e] = eg;
                gcnt[1][e] = et;
            }
            eg += cg[j];
            et += ct[j];
        }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < SEG; ++u) {
        if (u * NT >= cnt) break;
        const bool ok = tid + u * NT < cnt;
        const bool isg = ok && (all || key[u] > T);
        const bool ist = ok && !all && key[u] == T;
        const uint64_t mg = ballot(isg), mt = ballot(ist);
        const int rg = gcnt[0][u * NW + w] + rank_below(mg);  // keys above T before this one
        const int rt = gcnt[1][u * NW + w] + rank_below(mt);  // keys equal to T before this one
        if (isg || (ist && rt < need_ties)) {
            const int slot = rg + min(rt, need_ties);
            Srow[slot] = pos[u];
            if (Ssrow) Ssrow[slot] = key_score(key[u]);
        }
    }
    for (int i = K + tid; i < topk; i += NT) {
        Srow[i] = -1;
        if (Ssrow) Ssrow[i] = -INFINITY;
    }
}

// Keys in workgroup-visible memory: key_of(i, &valid) for i < cnt, read by
// thread i % NT.
template <int NT, bool RUNS = true, class KeyFn>
__device__ uint32_t block_select_adaptive(int cnt, int need, KeyFn key_of, SelectSmem& sm, int* gt_out,
                                          bool exact = true) {
    // eight keys per thread in flight (the keys may come from global memory)
    const auto each = [&](auto&& f) {
        int i = threadIdx.x;
        for (; i + 7 * NT < cnt; i += 8 * NT) {
            uint32_t kk[8];
            bool ok[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) kk[u] = key_of(i + u * NT, &ok[u]);
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (ok[u]) f(kk[u]);
        }
        for (; i < cnt; i += NT) {
            bool ok;
            const uint32_t k = key_of(i, &ok);
            if (ok) f(k);
        }
    };
    return block_select_each<NT, RUNS>(need, each, sm, gt_out, exact);
}

// Exact selection of the K = min(k, L) best of sc[0..L) ordered by (score desc,
// position asc).  Writes S[0..k): the selected positions ascending, then -1;
// Ss (optional): each slot's score, -inf for unused slots.  All NT threads of
// the workgroup call it; `sc` must be visible to the whole workgroup.
//
// Radix path (rows longer than the bitmap): three radix passes over the score
// key (11, 11, 10 bits) find the K-th largest key T and the count gt of keys
// above it; once the candidate bin holds at most TK_LCAP keys the remaining
// passes run on an LDS copy.  A final in-order pass keeps every key > T and
// the first K - gt keys == T (lowest positions first).
template <int NT>
__device__ void block_topk_row_radix(const float* __restrict__ sc, int L, int k, int32_t* __restrict__ S,
                                     float* __restrict__ Ss, TopkSmem& smu) {
    auto& sm = smu.r;
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


// Bitmap path (rows of at most TK_BITMAP_WORDS * 32 positions): the K-th
// largest key T by the span select over the row's own key range (a few bins
// of near-equal keys instead of the radix passes' crowded top digits); when
// more keys tie at T than slots remain, the lowest positions among them by a
// second select over inverted positions; every kept position sets its bit in
// a position bitmap, and a prefix popcount over the bitmap gives each its
// slot, in ascending position order.
template <int NT>
__device__ void block_topk_row(const float* __restrict__ sc, int L, int k, int32_t* __restrict__ S,
                               float* __restrict__ Ss, TopkSmem& smu) {
    const int tid = threadIdx.x;
    const int K = min(k, L);
    const int nwords = (L + 31) / 32;
    if (L <= k || nwords > TK_BITMAP_WORDS) {
        block_topk_row_radix<NT>(sc, L, k, S, Ss, smu);
        return;
    }
    auto& sm = smu.b;
    for (int i = tid; i < nwords; i += NT) sm.bitmap[i] = 0u;
    if (tid == 0) sm.nties = 0;
    __syncthreads();
    int gt;
    const uint32_t T = block_select_adaptive<NT>(
        L, K, [&](int i, bool* ok) { *ok = true; return score_key(sc[i]); }, sm.sel, &gt);
    const int need_ties = K - gt;
    // row visits with eight loads per thread in flight
    const auto visit = [&](auto&& f) {
        int i = tid;
        for (; i + 7 * NT < L; i += 8 * NT) {
            uint32_t kk[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) kk[u] = score_key(sc[i + u * NT]);
#pragma unroll
            for (int u = 0; u < 8; ++u) f(i + u * NT, kk[u]);
        }
        for (; i < L; i += NT) f(i, score_key(sc[i]));
    };
    int nt_local = 0;
    visit([&](int, uint32_t key) { nt_local += key == T; });
    nt_local = wave_sum(nt_local);
    if (lane_id() == 0 && nt_local) atomicAdd(&sm.nties, nt_local);
    __syncthreads();
    // ties at T: keep the need_ties lowest positions, i.e. the largest
    // inverted positions; when every tie is kept no selection is needed
    uint32_t inv_cut = 0u;
    if (sm.nties > need_ties) {
        int tgt;
        inv_cut = block_select_adaptive<NT>(
            L, need_ties, [&](int i, bool* ok) { *ok = score_key(sc[i]) == T; return ~(uint32_t)i; }, sm.sel, &tgt);
    }
    visit([&](int i, uint32_t key) {
        if (key > T || (key == T && ~(uint32_t)i >= inv_cut)) atomicOr(&sm.bitmap[i >> 5], 1u << (i & 31));
    });
    __syncthreads();
    // ordered output: each thread owns a contiguous run of bitmap words
    const int per = (nwords + NT - 1) / NT;
    const int w0 = min(nwords, tid * per), w1 = min(nwords, w0 + per);
    int mine = 0;
    for (int wd = w0; wd < w1; ++wd) mine += __popc(sm.bitmap[wd]);
    int total;
    int o = block_excl_scan<NT>(mine, &total, sm.sel.scratch);
    for (int wd = w0; wd < w1; ++wd) {
        uint32_t bits = sm.bitmap[wd];
        while (bits) {
            const int b = __builtin_ctz(bits);
            bits &= bits - 1;
            const int p = wd * 32 + b;
            S[o] = p;
            if (Ss) Ss[o] = sc[p];
            ++o;
        }
    }
    for (int i = K + tid; i < k; i += NT) {
        S[i] = -1;
        if (Ss) Ss[i] = -INFINITY;
    }
    __syncthreads();  // the caller may reuse the shared memory right away
}

}  // namespace tlsl
