// indexer.hip -- Lightning Indexer scoring and causal top-k on gfx950.
//
// The score of the DSA page, section 1.1 eq.(1), is a contraction over the
// indexer dimension followed by ReLU and a weighted sum over the indexer heads.
// It runs on the matrix cores as a 16x16 tile per (16 heads x 16 keys) block:
// heads on the M side, keys on the N side, dI on the reduction side.  ReLU, the
// weights and the head sum stay in registers (the epilogue), so no score
// matrix is stored.
//
// Prefill (eq.(2) for every row of a B x n batch) runs in three stages:
//  1. prefill_score: a workgroup owns 4*QW consecutive queries.  It first
//     scores them against every STRIDE-th key ("sample pass") and takes, per
//     query, a high order statistic of the sample as a conservative score
//     threshold.  It then walks all causal key tiles from the diagonal down,
//     appends every (score, position) that reaches the threshold to the
//     query's candidate buffer (descending position order) and counts them.
//  2. prefill_finalize: one workgroup per row reads the buffer once into
//     registers, selects the exact top-k (histogram select over the
//     register-held keys) and writes S in ascending position order.
//     A row whose buffer missed (fewer candidates than min(k, t+1): the sample
//     threshold overshot) or overflowed goes on a fallback list.
//  3. prefill_fallback: rescores the listed rows in full (spread over the
//     whole grid) and selects from them.
// The result does not depend on the threshold: every key that can be in the
// top-k reaches the buffer, or the row is recomputed.
//
// Decode (index_decode) scores the newest query of each sequence against its
// whole packed key cache with the same tile code, so a decode row equals the
// prefill row at the same length bit for bit.
#include <math.h>

#include <algorithm>

#include "idx_tile.h"
#include "tlsl_device.h"
#include "tlsl_internal.h"
#include "topk_common.h"

namespace tlsl {

// LDS image of a 64-key subtile.  Rows of 128 or 256 bytes are padded by 64 or
// 32 bytes and their 16-byte chunks are permuted within the row by XOR with the
// row's index in its 16-row block (the same for every key block, so a lane's
// fragment offsets are fixed): measured on gfx950, the fragment reads of this
// layout (lane (g,c) reads row c, chunk g*NCH + ch) take ~5.8 cycles per wave
// instruction against ~8.6 for rows padded by 16 bytes.  Other row sizes keep
// the 16-byte padding.
template <int DT, int DI>
struct KTile {
    static constexpr int ROWB = DI * ElemBytes<DT>::v;
    static constexpr bool SWZ = ROWB == 128 || ROWB == 256;
    static constexpr int STRIDE = ROWB + (ROWB == 256 ? 32 : (ROWB == 128 ? 64 : 16));
    static constexpr int BYTES = 64 * STRIDE;
    static constexpr int CPR = ROWB / 16;       // 16-B chunks per row
    static constexpr int CHUNKS = 64 * CPR;     // per subtile
    // byte offset of chunk k of row r
    __device__ __forceinline__ static int pos(int r, int k) {
        return r * STRIDE + 16 * (SWZ ? ((k ^ (r & 15)) & (CPR - 1)) : k);
    }
};

// four waves per workgroup, two workgroups per compute unit (two waves per
// SIMD): the two workgroups of a CU do not wait at each other's barriers or
// sample passes (against one eight-wave workgroup: 3% faster at n=131072)
constexpr int PF_WAVES = 4;
constexpr int PF_NT = PF_WAVES * 64;
constexpr int PF_RBUF = 512;      // per-query LDS buffer of sample scores
constexpr float PF_SIGMA = 4.0f;  // safety margin of the sample threshold, in standard deviations
// LDS scratch of one wave for the fp8 linear-part rows (the largest
// Idx<kFP8, HB, 128>::LIN_SCRATCH); other input types need none
constexpr int LIN_SCR = 8 * 128 + 8 * 4;
template <int DT>
constexpr int lin_scr_bytes() { return DT == kFP8 ? LIN_SCR : 16; }

struct PrefillArgs {
    const unsigned char* q;
    const float* q_scale;
    const unsigned char* k;
    const float* k_scale;
    const float* w;
    int B, n, HI, topk, cap, stride, tiles;
    uint2* buf;      // [B*n][cap] (score bits, position)
    int* cnt;        // [B*n] candidates found (may exceed cap)
    int* fb_count;   // fallback list length (zeroed here)
};

// r-th largest value (1-based) of vals[0..cnt) in LDS, owned by one wave, and
// the count of values strictly above it.
__device__ float wave_kth_largest(const float* vals, int cnt, int r, uint32_t* hist, int* gt_out) {
    const int l = lane_id();
    uint32_t prefix = 0, pmask = 0;
    int need = r, gt = 0;
    for (int sh = 24; sh >= 0; sh -= 8) {
        for (int i = l; i < 256; i += 64) hist[i] = 0;
        wave_lds_fence();
        for (int i = l; i < cnt; i += 64) {
            const uint32_t key = score_key(vals[i]);
            if ((key & pmask) == prefix) atomicAdd(&hist[(key >> sh) & 255u], 1u);
        }
        wave_lds_fence();
        int above;
        const int d = wave_find_bin<256>(hist, need, &above);
        gt += above;
        need -= above;
        prefix |= (uint32_t)d << sh;
        pmask |= 255u << sh;
        wave_lds_fence();
    }
    *gt_out = gt;
    return key_score(prefix);
}

// Number of sample values the threshold keeps for query t: the expected count
// of sample keys inside the final top-K plus PF_SIGMA standard deviations.
// Returns 0 when no useful threshold exists.
__device__ __forceinline__ int sample_rank(int t, int topk, int stride) {
    const int ns = t / stride + 1;
    const int K = min(topk, t + 1);
    const float mu = (float)ns * (float)K / (float)(t + 1);
    const int r = (int)ceilf(mu + PF_SIGMA * sqrtf(mu)) + 2;
    return (r < ns && r <= PF_RBUF - 64) ? r : 0;
}

template <int DT, int HB, int DI, int QW>
__global__ __launch_bounds__(PF_NT, 2) void prefill_score_kernel(PrefillArgs a) {
    using I = Idx<DT, HB, DI>;
    using KT = KTile<DT, DI>;
    constexpr int NCH = I::NCH;
    constexpr int TQ = PF_WAVES * QW;
    __shared__ __align__(16) unsigned char ktile[2][KT::BYTES];
    __shared__ float rbuf[TQ][PF_RBUF];
    __shared__ uint32_t whist[PF_WAVES][256];

    // the wave index is uniform across the wave: in a scalar register, every
    // per-query quantity derived from it is scalar too
    // the wave index is uniform across the wave: in a scalar register, every
    // per-query quantity derived from it is scalar too
    const int tid = threadIdx.x, wv_id = __builtin_amdgcn_readfirstlane(tid >> 6), l = lane_id(), g = l >> 4, c = l & 15;
    const int b = blockIdx.x % a.B;
    const int tile = a.tiles - 1 - blockIdx.x / a.B;  // heaviest tiles first
    const int t0 = tile * TQ;
    const int t_last = min(t0 + TQ, a.n) - 1;
    if (blockIdx.x == 0 && tid == 0) *a.fb_count = 0;

    const size_t tok0 = (size_t)b * a.n;
    const unsigned char* kb_base = a.k + tok0 * KT::ROWB;

    int tq[QW];
    bool qv[QW];
    uint4 qf[QW][HB][NCH];
    float wv[QW][HB][4];
#pragma unroll
    for (int i = 0; i < QW; ++i) {
        tq[i] = t0 + wv_id * QW + i;
        qv[i] = tq[i] < a.n;
        const size_t row = tok0 + (qv[i] ? tq[i] : 0);
        const float wmul = (DT == kFP8) ? a.q_scale[row] : 1.f;
        I::load_query(a.q + row * (size_t)a.HI * KT::ROWB, a.w + row * a.HI, wmul, a.HI, qv[i], qf[i], wv[i]);
    }
    // fp8: the linear-part rows of the wave's queries (slot i = query i), built
    // in the queries' sample buffers, which are free until the sample pass
    uint4 ql[NCH];
    float ls[2][2];
    if constexpr (DT == kFP8) {
        static_assert(I::LIN_SCRATCH <= PF_RBUF * (int)sizeof(float), "linear-part scratch fits a sample buffer");
#pragma unroll
        for (int i = 0; i < QW; ++i) {
            const size_t row = tok0 + (qv[i] ? tq[i] : 0);
            I::prep_lin(qf[i], a.w + row * a.HI, a.q_scale[row], a.HI, qv[i],
                        reinterpret_cast<unsigned char*>(rbuf[wv_id * QW + i]));
        }
        wave_lds_fence();
        I::load_lin(reinterpret_cast<const unsigned char*>(rbuf[wv_id * QW]),
                    QW > 1 ? reinterpret_cast<const unsigned char*>(rbuf[wv_id * QW + QW - 1]) : nullptr, ql, ls);
        wave_lds_fence();
    }
    // scores of query i for a subtile whose key fragments are kfx (fp8: lin
    // holds the subtile's linear-part products)
    auto score_q = [&](int i, const uint4 (&kfx)[4][NCH], const v4f (&lin)[4]) -> float {
        if constexpr (DT == kFP8) {
            if (i == 0) return I::template score_lin<0>(qf[0], wv[0], kfx, lin, ls[0]);
            return I::template score_lin<1>(qf[QW - 1], wv[QW - 1], kfx, lin, ls[1]);
        } else {
            return I::score(qf[i], wv[i], kfx);
        }
    };

    // cooperative copy of 64 key rows (row r <- key key_of(r), clamped) into LDS
    auto copy_rows = [&](unsigned char* dst, int key0, int kstep) {
        for (int ch = tid; ch < KT::CHUNKS; ch += PF_NT) {
            const int r = ch / KT::CPR, off = (ch % KT::CPR) * 16;
            const int key = min(key0 + r * kstep, a.n - 1);
            *reinterpret_cast<uint4*>(dst + KT::pos(r, off / 16)) =
                *reinterpret_cast<const uint4*>(kb_base + (size_t)key * KT::ROWB + off);
        }
    };
    auto frag_from_lds = [&](const unsigned char* src, uint4 (&kf)[4][NCH]) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch)
                kf[kb][ch] = *reinterpret_cast<const uint4*>(src + KT::pos(16 * kb + c, g * NCH + ch));
        }
    };

    // ---- sample pass: conservative per-query threshold ----------------------
    float theta[QW];
    int rneed[QW];
    bool any_pre = false;
#pragma unroll
    for (int i = 0; i < QW; ++i) {
        theta[i] = -INFINITY;
        rneed[i] = (qv[i] && tq[i] + 1 > a.cap) ? sample_rank(tq[i], a.topk, a.stride) : 0;
        any_pre |= rneed[i] > 0;
    }
    if (__syncthreads_or(any_pre)) {
        int rc[QW];
        float rth[QW];
#pragma unroll
        for (int i = 0; i < QW; ++i) { rc[i] = 0; rth[i] = -INFINITY; }
        const int nsamp = t_last / a.stride + 1;
        const int nss = (nsamp + 63) / 64;  // sample subtiles
        __syncthreads();
        copy_rows(ktile[0], 0, a.stride);
        __syncthreads();
        for (int js = 0; js < nss; ++js) {
            const int cur = js & 1;
            // the next sample subtile: loaded into registers now, stored to the
            // other LDS buffer after this one is scored
            constexpr int SPER = (KT::CHUNKS + PF_NT - 1) / PF_NT;
            static_assert(SPER >= 1 && SPER <= 4, "prefetch holds one to four chunks per thread");
            auto sp_load = [&](int u) {
                const int ch = min(tid + u * PF_NT, KT::CHUNKS - 1);
                const int r = ch / KT::CPR, off = (ch % KT::CPR) * 16;
                const int key = min(((js + 1) * 64 + r) * a.stride, a.n - 1);
                return *reinterpret_cast<const uint4*>(kb_base + (size_t)key * KT::ROWB + off);
            };
            uint4 spv[SPER];
#pragma unroll
            for (int u = 0; u < SPER; ++u) spv[u] = sp_load(u);
            asm volatile("" ::: "memory");
            uint4 kf[4][NCH];
            frag_from_lds(ktile[cur], kf);
            const int s = (js * 64 + l) * a.stride;
            const float ks = (DT == kFP8) ? a.k_scale[tok0 + min(s, a.n - 1)] : 1.f;
            v4f slin[4];
            if constexpr (DT == kFP8) I::lin_products(ql, kf, slin);
#pragma unroll
            for (int i = 0; i < QW; ++i) {
                if (rneed[i] == 0 || js * 64 * a.stride > tq[i]) continue;
                float sc = score_q(i, kf, slin);
                if (DT == kFP8) sc *= ks;
                const bool ok = s <= tq[i] && sc >= rth[i];
                const uint64_t m = ballot(ok);
                float* rb = rbuf[wv_id * QW + i];
                if (ok) rb[rc[i] + rank_below(m)] = sc;
                rc[i] += __popcll(m);
                if (rc[i] > PF_RBUF - 64) {
                    // keep the rneed largest values, raise the sample threshold
                    wave_lds_fence();
                    int gt;
                    const float v = wave_kth_largest(rb, rc[i], rneed[i], whist[wv_id], &gt);
                    float vals[PF_RBUF / 64];
#pragma unroll
                    for (int j = 0; j < PF_RBUF / 64; ++j) vals[j] = (l + 64 * j < rc[i]) ? rb[l + 64 * j] : -INFINITY;
                    wave_lds_fence();
                    int outc = 0;
#pragma unroll
                    for (int j = 0; j < PF_RBUF / 64; ++j) {
                        const bool keep = (l + 64 * j < rc[i]) && vals[j] > v;
                        const uint64_t mk = ballot(keep);
                        if (keep) rb[outc + rank_below(mk)] = vals[j];
                        outc += __popcll(mk);
                    }
                    for (int j = outc + l; j < rneed[i]; j += 64) rb[j] = v;
                    wave_lds_fence();
                    rc[i] = rneed[i];
                    rth[i] = v;
                }
            }
            asm volatile("" ::: "memory");
            {
                auto sp_store = [&](int u, const uint4& v) {
                    const int ch = tid + u * PF_NT;
                    if (ch < KT::CHUNKS) {
                        const int r = ch / KT::CPR, off = (ch % KT::CPR) * 16;
                        *reinterpret_cast<uint4*>(ktile[cur ^ 1] + KT::pos(r, off / 16)) = v;
                    }
                };
#pragma unroll
                for (int u = 0; u < SPER; ++u) sp_store(u, spv[u]);
            }
            __syncthreads();
        }
#pragma unroll
        for (int i = 0; i < QW; ++i) {
            if (rneed[i] > 0 && rc[i] >= rneed[i]) {
                wave_lds_fence();
                int gt;
                theta[i] = wave_kth_largest(rbuf[wv_id * QW + i], rc[i], rneed[i], whist[wv_id], &gt);
            }
        }
    }

    // ---- main pass: every causal key, diagonal first -----------------------
    // The last query of each subtile is finished one iteration late: its final
    // epilogue, head sum, threshold test and append run after the next
    // barrier, once the next subtile's fragment loads are issued, so that this
    // dependent tail overlaps the LDS latency instead of idling the matrix
    // cores before the barrier.  Appends stay in descending position order.
    int cntq[QW];
#pragma unroll
    for (int i = 0; i < QW; ++i) cntq[i] = 0;
    // threshold test and ordered append slot of query i's scores sc at positions s
    auto select = [&](int i, float sc, int s, bool& st, size_t& idx, uint2& val) {
        const bool ok = s <= tq[i] && sc >= theta[i];
        const uint64_t m = ballot(ok);
        const int slot = cntq[i] + rank_above(m);
        st = ok && slot < a.cap;
        idx = (tok0 + tq[i]) * (size_t)a.cap + slot;
        val = make_uint2(__float_as_uint(sc), (uint32_t)s);
        cntq[i] += __popcll(m);
    };
    float tpart[3];
    v4f tlast[HB];
    float tl0 = 0.f, tl1 = 0.f;  // fp8: the deferred query's linear rows of its last key block
    float tks = 1.f;
    int ts = 0;
    bool tpend = false;
    const int nsub = t_last / 64 + 1;
    __syncthreads();
    copy_rows(ktile[0], (nsub - 1) * 64, 1);
    __syncthreads();
    for (int it = 0; it < nsub; ++it) {
        const int j = nsub - 1 - it;
        const int cur = it & 1;
        // prefetch the next subtile into registers
        // (issued unconditionally from clamped rows, pinned ahead of the compute
        // and stored to LDS after it, so the loads stay in flight meanwhile)
        constexpr int PER = (KT::CHUNKS + PF_NT - 1) / PF_NT;
        static_assert(PER >= 1 && PER <= 4, "prefetch holds one to four chunks per thread");
        auto pf_load = [&](int u) {
            const int ch = min(tid + u * PF_NT, KT::CHUNKS - 1);
            const int r = ch / KT::CPR, off = (ch % KT::CPR) * 16;
            return *reinterpret_cast<const uint4*>(kb_base + (size_t)max((j - 1) * 64 + r, 0) * KT::ROWB + off);
        };
        uint4 pre[PER];
#pragma unroll
        for (int u = 0; u < PER; ++u) pre[u] = pf_load(u);
        asm volatile("" ::: "memory");
        uint4 kf[4][NCH];
        frag_from_lds(ktile[cur], kf);
        // the fragment loads stay ahead of the previous subtile's tail
        __builtin_amdgcn_sched_barrier(0);
        // candidate appends are held until the prefetched subtile is in LDS:
        // a store issued between the prefetch loads and their use would make
        // the wait for the loads wait for the store as well
        bool tst = false;
        size_t tidx = 0;
        uint2 tval = make_uint2(0, 0);
        if (tpend) {
            float sc;
            if constexpr (DT == kFP8) sc = I::score_tail_lin(wv[QW - 1], tpart, tlast, tl0, tl1, ls[QW - 1]);
            else sc = I::score_tail(wv[QW - 1], tpart, tlast);
            if (DT == kFP8) sc *= tks;
            select(QW - 1, sc, ts, tst, tidx, tval);
        }
        tpend = false;
        const int s = j * 64 + l;
        const float ks = (DT == kFP8) ? a.k_scale[tok0 + min(s, a.n - 1)] : 1.f;
        bool cst[QW];
        size_t cidx[QW];
        uint2 cval[QW];
        v4f lin[4];
        if constexpr (DT == kFP8) I::lin_products(ql, kf, lin);
#pragma unroll
        for (int i = 0; i < QW; ++i) {
            cst[i] = false;
            if (!qv[i] || j * 64 > tq[i]) continue;
            if (i < QW - 1) {
                float sc = score_q(i, kf, lin);
                if (DT == kFP8) sc *= ks;
                select(i, sc, s, cst[i], cidx[i], cval[i]);
            } else {
                if constexpr (DT == kFP8) {
                    I::template score_head_lin<QW - 1>(qf[i], wv[i], kf, lin, ls[QW - 1], tpart, tlast);
                    tl0 = lin[3][2 * (QW - 1)];
                    tl1 = lin[3][2 * (QW - 1) + 1];
                } else {
                    I::score_head(qf[i], wv[i], kf, tpart, tlast);
                }
                ts = s;
                tks = ks;
                tpend = true;
            }
        }
        asm volatile("" ::: "memory");
        {
            // stored on the last trip too (into the idle buffer, never read):
            // every path then retires the prefetch loads here
            auto pf_store = [&](int u, const uint4& v) {
                const int ch = tid + u * PF_NT;
                if (ch < KT::CHUNKS) {
                    const int r = ch / KT::CPR, off = (ch % KT::CPR) * 16;
                    *reinterpret_cast<uint4*>(ktile[cur ^ 1] + KT::pos(r, off / 16)) = v;
                }
            };
#pragma unroll
            for (int u = 0; u < PER; ++u) pf_store(u, pre[u]);
        }
        if (tst) a.buf[tidx] = tval;
#pragma unroll
        for (int i = 0; i < QW; ++i)
            if (cst[i]) a.buf[cidx[i]] = cval[i];
        __syncthreads();
    }
    if (tpend) {
        bool tst;
        size_t tidx;
        uint2 tval;
        float sc;
        if constexpr (DT == kFP8) sc = I::score_tail_lin(wv[QW - 1], tpart, tlast, tl0, tl1, ls[QW - 1]);
        else sc = I::score_tail(wv[QW - 1], tpart, tlast);
        if (DT == kFP8) sc *= tks;
        select(QW - 1, sc, ts, tst, tidx, tval);
        if (tst) a.buf[tidx] = tval;
    }
    if (l == 0) {
#pragma unroll
        for (int i = 0; i < QW; ++i)
            if (qv[i]) a.cnt[tok0 + tq[i]] = cntq[i];
    }
}

// ---------------------------------------------------------------------------
// Stage 2: exact selection from a row's candidate buffer.
// ---------------------------------------------------------------------------
constexpr int FIN_NT = 256;  // four waves per row: more rows in flight per CU than with eight

struct FinalizeArgs {
    const uint2* buf;
    const int* cnt;
    int n, topk, cap;
    int32_t* S;
    float* Ss;
    int* fb_count;
    int* fb_list;
};

template <int CAPMAX>
__global__ __launch_bounds__(FIN_NT) void prefill_finalize_kernel(FinalizeArgs a) {
    // Candidate i of a row, in ascending position order (buffer entry cnt-1-i:
    // the buffer holds descending positions), is held in registers by thread
    // i % FIN_NT as its (i / FIN_NT)-th item: one coalesced read of the buffer
    // gives both the score keys for the selection and the positions for S.
    constexpr int SEG = (CAPMAX + FIN_NT - 1) / FIN_NT;
    __shared__ SelectSmem sel;
    __shared__ int gcnt[2][SEG * (FIN_NT / 64)];
    const int tid = threadIdx.x;
    const int row = blockIdx.x;
    const int t = row % a.n;
    const int K = min(a.topk, t + 1);
    const int cnt = a.cnt[row];
    if (cnt < K || cnt > a.cap) {
        if (tid == 0) a.fb_list[atomicAdd(a.fb_count, 1)] = row;
        return;
    }
    const uint2* src = a.buf + (size_t)row * a.cap;
    // all loads issued before any is used (indices clamped, so always in
    // bounds; items past the count are never read back)
    uint2 e[SEG];
#pragma unroll
    for (int u = 0; u < SEG; ++u) e[u] = src[max(cnt - 1 - (tid + u * FIN_NT), 0)];
    uint32_t key[SEG];
    int pos[SEG];
#pragma unroll
    for (int u = 0; u < SEG; ++u) {
        key[u] = score_key(__uint_as_float(e[u].x));
        pos[u] = (int)e[u].y;
    }
    select_ordered<FIN_NT, SEG>(key, pos, cnt, K, a.topk, a.S + (size_t)row * a.topk,
                                a.Ss ? a.Ss + (size_t)row * a.topk : nullptr, sel, gcnt);
}

// ---------------------------------------------------------------------------
// Stage 3: rows whose buffer missed or overflowed are rescored in full.
// ---------------------------------------------------------------------------
constexpr int FB_NT = 512;

struct FallbackArgs {
    const unsigned char* q;
    const float* q_scale;
    const unsigned char* k;
    const float* k_scale;
    const float* w;
    int n, HI, topk;
    const int* fb_count;
    const int* fb_list;
    float* scratch;  // [fallback workgroups][n]
    int32_t* S;
    float* Ss;
};

// Scores of fallback row `row` for the 64-key subtiles j = j0, j0 + jstep, ...
// below j1, into sc[0..t] (one wave per subtile; the same tile code as the
// main pass, so the scores are bit-identical to it).
template <int DT, int HB, int DI>
__device__ __forceinline__ void fallback_rescore(const FallbackArgs& a, int row, int j0, int j1, int jstep,
                                                 float* sc, unsigned char* lscr) {
    using I = Idx<DT, HB, DI>;
    constexpr int NCH = I::NCH;
    const int l = lane_id();
    const int t = row % a.n;
    const size_t tok0 = (size_t)row - t;
    uint4 qf[HB][NCH];
    float wv[HB][4];
    const float wmul = (DT == kFP8) ? a.q_scale[row] : 1.f;
    I::load_query(a.q + (size_t)row * a.HI * I::ROWB, a.w + (size_t)row * a.HI, wmul, a.HI, true, qf, wv);
    // fp8: the row's linear-part rows in slot 0 (lscr: the wave's LDS scratch)
    uint4 ql[NCH];
    float ls[2][2];
    if constexpr (DT == kFP8) {
        I::prep_lin(qf, a.w + (size_t)row * a.HI, wmul, a.HI, true, lscr);
        wave_lds_fence();
        I::load_lin(lscr, nullptr, ql, ls);
        wave_lds_fence();
    }
    const unsigned char* kb_base = a.k + tok0 * I::ROWB;
    for (int j = j0; j < j1 && j * 64 <= t; j += jstep) {
        uint4 kf[4][NCH];
        I::load_keys_global(kb_base, j * 64, t, kf);
        float s;
        if constexpr (DT == kFP8) {
            v4f lin[4];
            I::lin_products(ql, kf, lin);
            s = I::template score_lin<0>(qf, wv, kf, lin, ls[0]);
        } else {
            s = I::score(qf, wv, kf);
        }
        const int key = j * 64 + l;
        if (DT == kFP8) s *= a.k_scale[tok0 + min(key, t)];
        if (key <= t) sc[key] = s;
    }
}

// Stage 3a: the first gridDim(3b) entries of the fallback list are rescored
// in parallel: work items (entry i, chunk of FBS_CHUNK keys) spread over the
// whole grid; entry i's scores go to scratch row i.  (A rare miss would
// otherwise rescore a whole row on one compute unit.)
constexpr int FBS_NT = 512;
constexpr int FBS_CHUNK = 4096;
constexpr int FBS_BLOCKS = 256;

template <int DT, int HB, int DI>
__global__ __launch_bounds__(FBS_NT) void prefill_fallback_score_kernel(FallbackArgs a, int fb_rows) {
    const int nfb = min(*a.fb_count, fb_rows);
    const int nch = (a.n + FBS_CHUNK - 1) / FBS_CHUNK;
    const int w = threadIdx.x >> 6;
    __shared__ __align__(16) unsigned char lscr[FBS_NT / 64][lin_scr_bytes<DT>()];
    for (int item = blockIdx.x; item < nfb * nch; item += gridDim.x) {
        const int i = item / nch, c = item - i * nch;
        const int row = a.fb_list[i];
        constexpr int SUB = FBS_CHUNK / 64;
        fallback_rescore<DT, HB, DI>(a, row, c * SUB + w, (c + 1) * SUB, FBS_NT / 64, a.scratch + (size_t)i * a.n,
                                     lscr[w]);
    }
}

// Stage 3b: each fallback row is selected from its full score row; entries
// past the first gridDim.x (not rescored by stage 3a) are rescored here.
template <int DT, int HB, int DI>
__global__ __launch_bounds__(FB_NT) void prefill_fallback_kernel(FallbackArgs a) {
    __shared__ TopkSmem sm;
    __shared__ __align__(16) unsigned char lscr[FB_NT / 64][lin_scr_bytes<DT>()];
    const int nfb = *a.fb_count;
    const int w = threadIdx.x >> 6;
    float* sc = a.scratch + (size_t)blockIdx.x * a.n;
    for (int it = blockIdx.x; it < nfb; it += gridDim.x) {
        const int row = a.fb_list[it];
        const int t = row % a.n;
        if (it >= (int)gridDim.x) fallback_rescore<DT, HB, DI>(a, row, w, 1 << 30, FB_NT / 64, sc, lscr[w]);
        __threadfence();
        __syncthreads();
        __threadfence();
        block_topk_row<FB_NT>(sc, t + 1, a.topk, a.S + (size_t)row * a.topk,
                              a.Ss ? a.Ss + (size_t)row * a.topk : nullptr, sm);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Decode scan: one query per sequence against its packed key cache.
// ---------------------------------------------------------------------------
constexpr int DEC_NT = 256;
constexpr int DEC_CHUNK = 4096;  // keys per workgroup

template <int DT, int HB, int DI>
__global__ __launch_bounds__(DEC_NT) void decode_score_kernel(const unsigned char* q, const float* q_scale,
                                                              const unsigned char* kc, const float* k_scale,
                                                              const float* w, const int64_t* cu, int HI,
                                                              float* scores) {
    using I = Idx<DT, HB, DI>;
    constexpr int NCH = I::NCH;
    const int b = blockIdx.x;
    const int64_t start = cu[b];
    const int L = (int)(cu[b + 1] - start);
    if ((int64_t)blockIdx.y * DEC_CHUNK >= L) return;
    const int wv_id = threadIdx.x >> 6, l = lane_id();
    __shared__ __align__(16) unsigned char lscr[DEC_NT / 64][lin_scr_bytes<DT>()];
    uint4 qf[HB][NCH];
    float wv[HB][4];
    const float wmul = (DT == kFP8) ? q_scale[b] : 1.f;
    I::load_query(q + (size_t)b * HI * I::ROWB, w + (size_t)b * HI, wmul, HI, true, qf, wv);
    uint4 ql[NCH];
    float ls[2][2];
    if constexpr (DT == kFP8) {
        I::prep_lin(qf, w + (size_t)b * HI, wmul, HI, true, lscr[wv_id]);
        wave_lds_fence();
        I::load_lin(lscr[wv_id], nullptr, ql, ls);
    }
    auto score_sub = [&](const uint4 (&kfx)[4][NCH]) -> float {
        if constexpr (DT == kFP8) {
            v4f lin[4];
            I::lin_products(ql, kfx, lin);
            return I::template score_lin<0>(qf, wv, kfx, lin, ls[0]);
        } else {
            return I::score(qf, wv, kfx);
        }
    };
    const unsigned char* kb_base = kc + (size_t)start * I::ROWB;
    constexpr int STEP = 64 * (DEC_NT / 64);
    // chunks blockIdx.y, + gridDim.y, ...: a sequence longer than the launch
    // was sized for (max_len) is still scored in full
    for (int64_t base64 = (int64_t)blockIdx.y * DEC_CHUNK; base64 < L; base64 += (int64_t)gridDim.y * DEC_CHUNK) {
        const int base = (int)base64;
        const int end = min(L, base + DEC_CHUNK);
        // two subtiles in flight per wave: the next one loads while this one is scored
        uint4 kf[2][4][NCH];
        int j0 = base + 64 * wv_id;
        if (j0 < end) I::load_keys_global(kb_base, j0, L - 1, kf[0]);
        for (; j0 < end; j0 += 2 * STEP) {
            const int j1 = j0 + STEP;
            if (j1 < end) I::load_keys_global(kb_base, j1, L - 1, kf[1]);
            {
                float s = score_sub(kf[0]);
                const int key = j0 + l;
                if (DT == kFP8) s *= k_scale[start + min(key, L - 1)];
                if (key < L) scores[start + key] = s;
            }
            if (j1 >= end) break;
            if (j1 + STEP < end) I::load_keys_global(kb_base, j1 + STEP, L - 1, kf[0]);
            {
                float s = score_sub(kf[1]);
                const int key = j1 + l;
                if (DT == kFP8) s *= k_scale[start + min(key, L - 1)];
                if (key < L) scores[start + key] = s;
            }
        }
    }
}

// Balanced decode scan: the batch is cut into sequence-aligned 64-key
// subtiles; workgroup i takes an equal contiguous range of them (the subtile
// prefix over the sequences is rebuilt in LDS by every workgroup), its waves
// interleave over the range, and each wave keeps the next subtile's keys in
// flight while it scores the current one.  Every workgroup has the same amount
// of work and no workgroup is launched for keys past a sequence's end.  One
// eight-wave workgroup per CU (two waves per SIMD): each CU then walks one
// contiguous range, twice as long as with two four-wave workgroups, with
// half as many sequence boundaries and the whole range staged in LDS
// (measured 153 -> 147 us at 64 sequences, identical scores).
constexpr int DEC2_NT = 512;
constexpr int DEC2_MAXB = 4096;
// Dynamic LDS: the subtile prefix and sequence starts of the batch, then the
// staged scores -- the workgroup's whole range when it fits (written by the
// workgroup at the end, mostly with 16-byte stores), else a stage per wave
// (written at the end of each sequence run or when full).  Stored per subtile
// in between the key loads, the 256-byte score stores cost 22 of 135 us at
// 64 sequences; staged, about half of that.
// dynamic LDS per workgroup: with the static part (the fp8 linear-part
// scratch, 8.4 KB for eight waves) within the CU's 160 KB
constexpr size_t DEC2_LDS_BUDGET = 150 * 1024;
__host__ __device__ constexpr size_t dec2_off_sstart(int B) { return ((size_t)(B + 1) * 4 + 7) & ~(size_t)7; }
__host__ __device__ constexpr size_t dec2_off_stage(int B) {
    return (dec2_off_sstart(B) + (size_t)(B + 1) * 8 + 15) & ~(size_t)15;
}

__device__ __forceinline__ int find_seq(const int* pre, int B, int g) {
    int lo = 0, hi = B;  // pre[lo] <= g < pre[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (pre[mid] <= g) lo = mid;
        else hi = mid;
    }
    return lo;
}

template <int DT, int HB, int DI>
__global__ __launch_bounds__(DEC2_NT) void decode_scan_kernel(const unsigned char* q, const float* q_scale,
                                                              const unsigned char* kc, const float* k_scale,
                                                              const float* w, const int64_t* cu, int B, int HI,
                                                              float* scores, int scap, int stage_sub) {
    using I = Idx<DT, HB, DI>;
    constexpr int NCH = I::NCH;
    constexpr int NWV = DEC2_NT / 64;
    extern __shared__ __align__(16) unsigned char dsm[];
    int* pre = reinterpret_cast<int*>(dsm);
    int64_t* sstart = reinterpret_cast<int64_t*>(dsm + dec2_off_sstart(B));
    __shared__ int scratch[16];
    // (wave index as a scalar: the subtile loop is then uniform, and the
    // compiler adds no wait for all loads at its head)
    const int tid = threadIdx.x, wv_id = __builtin_amdgcn_readfirstlane(tid >> 6), l = lane_id();
    // scap > 0: each wave stages up to scap subtiles; scap == 0: the range of
    // the workgroup is staged (subtile g at (g - g0) * 64; stage_sub subtiles
    // at most, which covers the range whenever max_len bounds the lengths as
    // required; past it scores are stored directly) and written by the
    // workgroup at the end with 16-byte stores
    float* const stage = reinterpret_cast<float*>(dsm + dec2_off_stage(B));
    float* sb = stage + (size_t)wv_id * scap * 64;
    // subtile prefix over the sequences, and the sequence starts
    int carry = 0;
    for (int b0 = 0; b0 < B; b0 += DEC2_NT) {
        const int b = b0 + tid;
        if (b <= B) sstart[b] = cu[b];
        const int ns = b < B ? (int)((cu[b + 1] - cu[b] + 63) >> 6) : 0;
        int incl = wave_incl_scan(ns);
        if (l == 63) scratch[wv_id] = incl;
        __syncthreads();
        int wbase = carry, tot = 0;
        for (int i = 0; i < NWV; ++i) {
            if (i < wv_id) wbase += scratch[i];
            tot += scratch[i];
        }
        if (b < B) pre[b] = wbase + incl - ns;
        carry += tot;
        __syncthreads();
    }
    // (the loop above writes sstart[B] only when B is not a multiple of
    // DEC2_NT; the end of the last sequence is set here for every B)
    if (tid == 0) {
        pre[B] = carry;
        sstart[B] = cu[B];
    }
    __syncthreads();
    const int total = carry;
    const int per = (total + gridDim.x - 1) / gridDim.x;
    const int g0 = blockIdx.x * per, g1 = min(total, g0 + per);

    uint4 qf[HB][NCH];
    float wv[HB][4];
    uint4 ql[NCH];  // fp8: linear-part rows of the segment's query (slot 0)
    float ls[2][2];
    __shared__ __align__(16) unsigned char lscr[NWV][lin_scr_bytes<DT>()];
    uint4 kf[2][4][NCH];
    float ksc[2];
    // the wave's subtiles are g0+wv_id, +NWV, ...; they are walked one sequence
    // (segment) at a time so that the inner loop has straight-line loads.  A
    // subtile's keys and key scales are loaded one step before its scores:
    // both are loop-carried, so the compiler cannot sink the scale load next
    // to a store.  Loads past the segment end are clamped to its last key (in
    // bounds, unused).  Scores go to the wave's stage in LDS and out at the
    // end of the segment (or when the stage is full).
    int g = g0 + wv_id;
    while (g < g1) {
        const int b = find_seq(pre, B, g);
        const int seg_end = min(g1, pre[b + 1]);
        const int64_t start = sstart[b];
        const int L = (int)(sstart[b + 1] - start);
        const unsigned char* kbase = kc + (size_t)start * I::ROWB;
        const float wmul = (DT == kFP8) ? q_scale[b] : 1.f;
        I::load_query(q + (size_t)b * HI * I::ROWB, w + (size_t)b * HI, wmul, HI, true, qf, wv);
        if constexpr (DT == kFP8) {
            wave_lds_fence();  // the previous segment's reads of the scratch are done
            I::prep_lin(qf, w + (size_t)b * HI, wmul, HI, true, lscr[wv_id]);
            wave_lds_fence();
            I::load_lin(lscr[wv_id], nullptr, ql, ls);
        }
        int key0 = (g - pre[b]) * 64;
        auto fetch = [&](int k0, uint4 (&kf_)[4][NCH], float& ks_) {
            I::load_keys_global(kbase, min(k0, L - 1), L - 1, kf_);
            ks_ = DT == kFP8 ? k_scale[start + min(k0 + l, L - 1)] : 1.f;
        };
        fetch(key0, kf[0], ksc[0]);
        int nst = 0, st_key0 = key0;  // staged subtiles and the first one's key
        auto flush = [&] {
            for (int k = 0; k < nst; ++k) {
                const int key = st_key0 + 64 * NWV * k + l;
                if (key < L) scores[start + key] = sb[64 * k + l];
            }
            nst = 0;
        };
        auto step = [&](const uint4 (&cur)[4][NCH], float ks, uint4 (&ahead)[4][NCH], float& ks_ahead) {
            fetch(key0 + 64 * NWV, ahead, ks_ahead);
            float s;
            if constexpr (DT == kFP8) s = I::score_lean_lin(qf, wv, cur, ql, ls[0]) * ks;
            else s = I::score_lean(qf, wv, cur) * ks;
            if (scap == 0) {
                if (g - g0 < stage_sub) stage[(size_t)(g - g0) * 64 + l] = s;
                else if (key0 + l < L) scores[start + key0 + l] = s;
            } else {
                if (nst == 0) st_key0 = key0;
                sb[64 * nst + l] = s;
                if (++nst == scap) flush();
            }
            g += NWV;
            key0 += 64 * NWV;
            return g < seg_end;
        };
        for (;;) {
            if (!step(kf[0], ksc[0], kf[1], ksc[1])) break;
            if (!step(kf[1], ksc[1], kf[0], ksc[0])) break;
        }
        if (scap > 0) flush();
    }
    if (scap == 0 && g0 < g1) {
        // the workgroup's staged range, one contiguous run per sequence: a
        // head of up to 3 scores to the next 16-byte boundary, 16-byte
        // stores, a tail
        __syncthreads();
        for (int b = find_seq(pre, B, g0); b < B && pre[b] < g1; ++b) {
            const int gs = max(g0, pre[b]), ge = min(min(g1, g0 + stage_sub), pre[b + 1]);
            if (gs >= ge) continue;
            const int64_t start = sstart[b];
            const int L = (int)(sstart[b + 1] - start);
            const int kfirst = (gs - pre[b]) * 64;
            const int n = min(L, (ge - pre[b]) * 64) - kfirst;
            const float* src = stage + (size_t)(gs - g0) * 64;
            float* dst = scores + start + kfirst;
            const int head = min(n, (int)((4 - ((start + kfirst) & 3)) & 3));
            if (tid < head) dst[tid] = src[tid];
            const int m = (n - head) >> 2;
            float4* d4 = reinterpret_cast<float4*>(dst + head);
            for (int i = tid; i < m; i += DEC2_NT) {
                const float* v = src + head + 4 * i;
                d4[i] = make_float4(v[0], v[1], v[2], v[3]);
            }
            const int t0 = head + 4 * m;
            if (t0 + tid < n) dst[t0 + tid] = src[t0 + tid];
        }
    }
}

// ---------------------------------------------------------------------------
// Host launchers.
// ---------------------------------------------------------------------------
// Compute units of the current device (queried once per device).
int device_cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

static int head_blocks(int HI) { return HI <= 16 ? 1 : (HI <= 32 ? 2 : 4); }
static int queries_per_wave(const IndexerShape& s) {
    const int eb = s.dt == kF32 ? 4 : (s.dt == kBF16 ? 2 : 1);
    const int nch = s.DI * eb / 64;
    return nch * head_blocks(s.HI) <= 8 ? 2 : 1;
}
template <int DT, int HB, int DI>
static hipError_t launch_prefill_t(const PrefillArgs& pa, const FinalizeArgs& fa, const FallbackArgs& fb,
                                   int qw, int rows, int cap, int fb_blocks, hipStream_t st) {
    // two queries per wave only where the fragments of both fit in registers
    // (the rule of queries_per_wave); the other form is not instantiated
    constexpr int QW = Mma<DT, DI>::NCH * HB <= 8 ? 2 : 1;
    if (qw != QW) return hipErrorInvalidValue;
    TLSL_TIMED_LAUNCH("prefill_score_kernel", st,
                      hipLaunchKernelGGL((prefill_score_kernel<DT, HB, DI, QW>), dim3(pa.tiles * pa.B), dim3(PF_NT), 0,
                                         st, pa));
    if (cap <= 1024)
        TLSL_TIMED_LAUNCH("prefill_finalize_kernel", st,
                          hipLaunchKernelGGL((prefill_finalize_kernel<1024>), dim3(rows), dim3(FIN_NT), 0, st, fa));
    else if (cap <= 4352)
        TLSL_TIMED_LAUNCH("prefill_finalize_kernel", st,
                          hipLaunchKernelGGL((prefill_finalize_kernel<4352>), dim3(rows), dim3(FIN_NT), 0, st, fa));
    else
        TLSL_TIMED_LAUNCH("prefill_finalize_kernel", st,
                          hipLaunchKernelGGL((prefill_finalize_kernel<8448>), dim3(rows), dim3(FIN_NT), 0, st, fa));
    TLSL_TIMED_LAUNCH("prefill_fallback_score_kernel", st,
                      hipLaunchKernelGGL((prefill_fallback_score_kernel<DT, HB, DI>), dim3(FBS_BLOCKS), dim3(FBS_NT), 0,
                                         st, fb, fb_blocks));
    TLSL_TIMED_LAUNCH("prefill_fallback_kernel", st,
                      hipLaunchKernelGGL((prefill_fallback_kernel<DT, HB, DI>), dim3(fb_blocks), dim3(FB_NT), 0, st, fb));
    return hipGetLastError();
}

template <int DT, int DI>
static hipError_t launch_prefill_hb(int hb, const PrefillArgs& pa, const FinalizeArgs& fa, const FallbackArgs& fb,
                                    int qw, int rows, int cap, int fbb, hipStream_t st) {
    if (hb == 1) return launch_prefill_t<DT, 1, DI>(pa, fa, fb, qw, rows, cap, fbb, st);
    if (hb == 2) return launch_prefill_t<DT, 2, DI>(pa, fa, fb, qw, rows, cap, fbb, st);
    return launch_prefill_t<DT, 4, DI>(pa, fa, fb, qw, rows, cap, fbb, st);
}

hipError_t launch_index_prefill(const IndexerShape& s, const void* q, const float* q_scale, const void* k,
                                const float* k_scale, const float* w, int B, int n, int topk, int32_t* S,
                                float* S_score, void* ws, const PrefillPlan& plan, hipStream_t st) {
    unsigned char* wsb = static_cast<unsigned char*>(ws);
    const int qw = queries_per_wave(s);
    const int tq = PF_WAVES * qw;
    PrefillArgs pa;
    pa.q = static_cast<const unsigned char*>(q);
    pa.q_scale = q_scale;
    pa.k = static_cast<const unsigned char*>(k);
    pa.k_scale = k_scale;
    pa.w = w;
    pa.B = B;
    pa.n = n;
    pa.HI = s.HI;
    pa.topk = topk;
    pa.cap = plan.cap;
    pa.stride = plan.stride;
    pa.tiles = (n + tq - 1) / tq;
    pa.buf = reinterpret_cast<uint2*>(wsb + plan.off_buf);
    pa.cnt = reinterpret_cast<int*>(wsb + plan.off_cnt);
    pa.fb_count = reinterpret_cast<int*>(wsb + plan.off_fbcount);
    FinalizeArgs fa;
    fa.buf = pa.buf;
    fa.cnt = pa.cnt;
    fa.n = n;
    fa.topk = topk;
    fa.cap = plan.cap;
    fa.S = S;
    fa.Ss = S_score;
    fa.fb_count = pa.fb_count;
    fa.fb_list = reinterpret_cast<int*>(wsb + plan.off_fblist);
    FallbackArgs fb;
    fb.q = pa.q;
    fb.q_scale = q_scale;
    fb.k = pa.k;
    fb.k_scale = k_scale;
    fb.w = w;
    fb.n = n;
    fb.HI = s.HI;
    fb.topk = topk;
    fb.fb_count = pa.fb_count;
    fb.fb_list = fa.fb_list;
    fb.scratch = reinterpret_cast<float*>(wsb + plan.off_fbscratch);
    fb.S = S;
    fb.Ss = S_score;
    const int hb = head_blocks(s.HI);
    const int rows = B * n;
    if (s.dt == kFP8) return launch_prefill_hb<kFP8, 128>(hb, pa, fa, fb, qw, rows, plan.cap, plan.fb_blocks, st);
    if (s.dt == kBF16) {
        if (s.DI == 32) return launch_prefill_hb<kBF16, 32>(hb, pa, fa, fb, qw, rows, plan.cap, plan.fb_blocks, st);
        if (s.DI == 64) return launch_prefill_hb<kBF16, 64>(hb, pa, fa, fb, qw, rows, plan.cap, plan.fb_blocks, st);
        return launch_prefill_hb<kBF16, 128>(hb, pa, fa, fb, qw, rows, plan.cap, plan.fb_blocks, st);
    }
    if (s.DI == 32) return launch_prefill_hb<kF32, 32>(hb, pa, fa, fb, qw, rows, plan.cap, plan.fb_blocks, st);
    return launch_prefill_hb<kF32, 64>(hb, pa, fa, fb, qw, rows, plan.cap, plan.fb_blocks, st);
}

template <int DT, int HB, int DI>
static hipError_t launch_decode_t(const void* q, const float* q_scale, const void* kc, const float* k_scale,
                                  const float* w, const int64_t* cu, int B, int HI, int max_len, float* scores,
                                  hipStream_t st) {
    if (B <= DEC2_MAXB) {
        // resident workgroups per CU (one with the LDS budget above; at most
        // two), each with an equal share of the batch's subtiles; the stage
        // holds a workgroup's whole share when it fits, else a share per wave
        // (flushed when full)
        constexpr int NWV = DEC2_NT / 64;
        const int64_t nsub_max = (int64_t)B * ((max_len + 63) / 64);
        // resident workgroups per CU, queried once per device and instantiation
        static int occ[64] = {0};
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
        int nb = occ[dev];
        if (nb == 0) {
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_scan_kernel<DT, HB, DI>, DEC2_NT,
                                                             DEC2_LDS_BUDGET) != hipSuccess ||
                nb < 1)
                nb = 1;
            occ[dev] = nb;
        }
        const int grid = (int)std::min<int64_t>((int64_t)device_cu_count() * std::min(nb, 2), std::max<int64_t>(1, nsub_max));
        const int64_t per_max = (nsub_max + grid - 1) / grid;  // >= every workgroup's share
        const int64_t pw_max = (per_max + NWV - 1) / NWV;
        const size_t base = dec2_off_stage(B);
        const bool wg_stage = base + (size_t)per_max * 256 <= DEC2_LDS_BUDGET;
        const int scap =
            wg_stage ? 0 : (int)std::max<int64_t>(1, std::min<int64_t>(pw_max, (DEC2_LDS_BUDGET - base) / (NWV * 256)));
        const size_t dyn = wg_stage ? base + (size_t)per_max * 256 : base + (size_t)NWV * scap * 256;
        TLSL_TIMED_LAUNCH("decode_scan_kernel", st,
                          hipLaunchKernelGGL((decode_scan_kernel<DT, HB, DI>), dim3(grid), dim3(DEC2_NT), dyn, st,
                                             static_cast<const unsigned char*>(q), q_scale,
                                             static_cast<const unsigned char*>(kc), k_scale, w, cu, B, HI, scores,
                                             scap, (int)(wg_stage ? per_max : 0)));
        return hipGetLastError();
    }
    // one workgroup column per sequence (x), chunks of DEC_CHUNK keys (y)
    dim3 grid(B, std::min((max_len + DEC_CHUNK - 1) / DEC_CHUNK, 65535));
    TLSL_TIMED_LAUNCH("decode_score_kernel", st,
                      hipLaunchKernelGGL((decode_score_kernel<DT, HB, DI>), grid, dim3(DEC_NT), 0, st,
                                         static_cast<const unsigned char*>(q), q_scale,
                                         static_cast<const unsigned char*>(kc), k_scale, w, cu, HI, scores));
    return hipGetLastError();
}

template <int DT, int DI>
static hipError_t launch_decode_hb(int hb, const void* q, const float* qs, const void* kc, const float* ks,
                                   const float* w, const int64_t* cu, int B, int HI, int ml, float* sc,
                                   hipStream_t st) {
    if (hb == 1) return launch_decode_t<DT, 1, DI>(q, qs, kc, ks, w, cu, B, HI, ml, sc, st);
    if (hb == 2) return launch_decode_t<DT, 2, DI>(q, qs, kc, ks, w, cu, B, HI, ml, sc, st);
    return launch_decode_t<DT, 4, DI>(q, qs, kc, ks, w, cu, B, HI, ml, sc, st);
}

hipError_t launch_index_decode(const IndexerShape& s, const void* q, const float* q_scale, const void* kc,
                               const float* k_scale, const float* w, const int64_t* cu, int B, int max_len,
                               float* scores, hipStream_t st) {
    const int hb = head_blocks(s.HI);
    if (s.dt == kFP8) return launch_decode_hb<kFP8, 128>(hb, q, q_scale, kc, k_scale, w, cu, B, s.HI, max_len, scores, st);
    if (s.dt == kBF16) {
        if (s.DI == 32) return launch_decode_hb<kBF16, 32>(hb, q, q_scale, kc, k_scale, w, cu, B, s.HI, max_len, scores, st);
        if (s.DI == 64) return launch_decode_hb<kBF16, 64>(hb, q, q_scale, kc, k_scale, w, cu, B, s.HI, max_len, scores, st);
        return launch_decode_hb<kBF16, 128>(hb, q, q_scale, kc, k_scale, w, cu, B, s.HI, max_len, scores, st);
    }
    if (s.DI == 32) return launch_decode_hb<kF32, 32>(hb, q, q_scale, kc, k_scale, w, cu, B, s.HI, max_len, scores, st);
    return launch_decode_hb<kF32, 64>(hb, q, q_scale, kc, k_scale, w, cu, B, s.HI, max_len, scores, st);
}

}  // namespace tlsl
