// topk.hip -- topk_select: exact top-k of explicit variable-length score rows
// (DSA page, section 1.1 eq.(2); section 2 on radix top-k over rows given by
// sequence lengths, avoiding a full sort).
//
// One workgroup per row, in one launch:
//  1. the r-th largest of a strided sample of the row (r = expected sample
//     hits inside the top-k plus 4 standard deviations) -- a conservative
//     threshold;
//  2. every (score, position) of the row at or above it is appended to LDS
//     (16-byte loads, one LDS counter increment per wave and load);
//  3. an exact radix select among those candidates, ties resolved to the
//     lowest positions, and the selected positions written in ascending order
//     through a position bitmap.
// A row whose candidates miss (the sample threshold overshot) or overflow is
// selected from its full score row instead (topk_common.h).  The result never
// depends on the threshold, only the work does.
#include <math.h>

#include "tlsl_device.h"
#include "tlsl_internal.h"
#include "topk_common.h"

namespace tlsl {

constexpr int TR_NT = 1024;              // workgroup (one row)
constexpr int TT_SAMPLE_MAX = 8192;      // sample values held in LDS
constexpr int TSEL_CAPMAX = 8448;        // candidates held in LDS, max
constexpr int TSEL_BITMAP_WORDS = 4096;  // rows up to 131072 use the bitmap output
constexpr int TR_BATCH = 8;              // 16-byte loads in flight per thread
constexpr float TSEL_SIGMA = 4.0f;

struct TopkArgs {
    const float* scores;
    const int64_t* row_start;
    const int32_t* row_len;
    int k, cap;
    int32_t* S;
    float* Ss;
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

__device__ __forceinline__ int sample_stride(int L) { return max(16, (L + TT_SAMPLE_MAX - 1) / TT_SAMPLE_MAX); }

struct TopkRowSmem {
    uint32_t keys[TSEL_CAPMAX];  // the sample's keys, then the candidates' keys
    uint32_t pos[TSEL_CAPMAX];
    uint32_t bitmap[TSEL_BITMAP_WORDS];
    SelectSmem sel;
    int cnt, nties;
};

union TopkRowShared {
    TopkRowSmem f;
    TopkSmem g;
};

__global__ __launch_bounds__(TR_NT) void topk_row_kernel(TopkArgs a) {
    __shared__ TopkRowShared sh;
    TopkRowSmem& s = sh.f;
    const int r = blockIdx.x, tid = threadIdx.x, l = lane_id();
    const int L = max(a.row_len[r], 0);
    const int K = min(a.k, L);
    const float* sc = a.scores + a.row_start[r];
    int32_t* Srow = a.S + (size_t)r * a.k;
    float* Ssrow = a.Ss ? a.Ss + (size_t)r * a.k : nullptr;
    if (L <= a.k) {
        for (int i = tid; i < a.k; i += TR_NT) {
            Srow[i] = i < L ? i : -1;
            if (Ssrow) Ssrow[i] = i < L ? sc[i] : -INFINITY;
        }
        return;
    }
    const int nwords = (L + 31) / 32;
    // ---- 1. sample threshold (rows within the candidate capacity keep all) --
    float theta = -INFINITY;
    {
        const int stride = sample_stride(L);
        const int ns = (L - 1) / stride + 1;
        const float mu = (float)ns * (float)K / (float)L;
        const int need = (int)ceilf(mu + TSEL_SIGMA * sqrtf(mu)) + 2;
        if (L > a.cap && need < ns) {
            batched_copy<TR_NT, 16>(ns, [&](int j) { return sc[(size_t)j * stride]; },
                                    [&](int j, float v) { s.keys[j] = score_key(v); });
            __syncthreads();
            int gt;
            const uint32_t T = block_select_adaptive<TR_NT>(
                ns, need, [&](int i, bool* ok) { *ok = true; return s.keys[i]; }, s.sel, &gt);
            theta = key_score(T);
        }
    }
    // ---- 2. candidates: every score >= theta, appended to LDS ---------------
    // 16-byte loads from the first 16-byte boundary of the row (the head
    // before it and the tail after the last whole float4, fewer than 4 scores
    // each, go to the first threads with the first batch); per batch each
    // thread counts its hits, one workgroup scan gives every thread its slots
    {
        const int head = min(L, (int)(((16 - ((uintptr_t)sc & 15)) & 15) / 4));
        const float4* v4 = reinterpret_cast<const float4*>(sc + head);
        const int n4 = (L - head) / 4;
        const int tail0 = head + 4 * n4;
        int base = 0;
        for (int b0 = 0; b0 == 0 || b0 < n4; b0 += TR_NT * TR_BATCH) {
            float4 v[TR_BATCH];
#pragma unroll
            for (int u = 0; u < TR_BATCH; ++u) {
                const int i = b0 + u * TR_NT + tid;
                v[u] = i < n4 ? v4[i] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
            }
            // the scalar extras: thread t < 4 takes head score t and tail score t
            float xh = -INFINITY, xt = -INFINITY;
            if (b0 == 0 && tid < 4) {
                if (tid < head) xh = sc[tid];
                if (tail0 + tid < L) xt = sc[tail0 + tid];
            }
            int mine = (xh >= theta) + (xt >= theta);
#pragma unroll
            for (int u = 0; u < TR_BATCH; ++u)
                mine += (v[u].x >= theta) + (v[u].y >= theta) + (v[u].z >= theta) + (v[u].w >= theta);
            int total;
            int o = base + block_excl_scan<TR_NT>(mine, &total, s.sel.scratch);
            auto put = [&](float x, int p) {
                if (x >= theta) {
                    if (o < TSEL_CAPMAX) {
                        s.keys[o] = score_key(x);
                        s.pos[o] = (uint32_t)p;
                    }
                    ++o;
                }
            };
            put(xh, tid);
            put(xt, tail0 + tid);
#pragma unroll
            for (int u = 0; u < TR_BATCH; ++u) {
                const int p = head + 4 * (b0 + u * TR_NT + tid);
                put(v[u].x, p);
                put(v[u].y, p + 1);
                put(v[u].z, p + 2);
                put(v[u].w, p + 3);
            }
            base += total;
        }
        if (tid == 0) s.cnt = base;
    }
    __syncthreads();
    const int cnt = s.cnt;
    if (cnt < K || cnt > min(a.cap, TSEL_CAPMAX) || nwords > TSEL_BITMAP_WORDS) {
        __syncthreads();  // every thread has read cnt before the union is reused
        block_topk_row<TR_NT>(sc, L, a.k, Srow, Ssrow, sh.g);
        return;
    }
    // ---- 3. exact selection among the candidates ---------------------------
    for (int i = tid; i < nwords; i += TR_NT) s.bitmap[i] = 0u;
    if (tid == 0) s.nties = 0;
    __syncthreads();
    int gt;
    const uint32_t T = block_select_adaptive<TR_NT>(cnt, K, [&](int i, bool* ok) { *ok = true; return s.keys[i]; },
                                                    s.sel, &gt);
    // ties at T: keep the (K - gt) lowest positions, i.e. the largest inverted
    // positions; when every tie is kept no selection is needed
    const int need_ties = K - gt;
    int nt_local = 0;
    for (int i = tid; i < cnt; i += TR_NT) nt_local += s.keys[i] == T;
    nt_local = wave_sum(nt_local);
    if (l == 0 && nt_local) atomicAdd(&s.nties, nt_local);
    __syncthreads();
    uint32_t inv_cut = 0u;
    if (s.nties > need_ties) {
        int tgt;
        inv_cut = block_select_adaptive<TR_NT>(
            cnt, need_ties, [&](int i, bool* ok) { *ok = s.keys[i] == T; return ~s.pos[i]; }, s.sel, &tgt);
    }
    for (int i = tid; i < cnt; i += TR_NT) {
        const uint32_t key = s.keys[i];
        if (key > T || (key == T && ~s.pos[i] >= inv_cut)) atomicOr(&s.bitmap[s.pos[i] >> 5], 1u << (s.pos[i] & 31));
    }
    __syncthreads();
    // ordered output: each thread owns a contiguous run of bitmap words
    const int per = (nwords + TR_NT - 1) / TR_NT;
    const int w0 = min(nwords, tid * per), w1 = min(nwords, w0 + per);
    int mine = 0;
    for (int wd = w0; wd < w1; ++wd) mine += __popc(s.bitmap[wd]);
    int total;
    int o = block_excl_scan<TR_NT>(mine, &total, s.sel.scratch);
    for (int wd = w0; wd < w1; ++wd) {
        uint32_t bits = s.bitmap[wd];
        while (bits) {
            const int b = __builtin_ctz(bits);
            bits &= bits - 1;
            const int p = wd * 32 + b;
            Srow[o] = p;
            if (Ssrow) Ssrow[o] = sc[p];
            ++o;
        }
    }
    for (int i = K + tid; i < a.k; i += TR_NT) {
        Srow[i] = -1;
        if (Ssrow) Ssrow[i] = -INFINITY;
    }
}

static int topk_cap(int k) { return std::min(TSEL_CAPMAX, (int)((2 * (size_t)k + 256 + 255) / 256 * 256)); }

size_t topk_ws_bytes(int, int, int) { return 256; }  // none needed; never empty (a NULL workspace is a size query)

hipError_t launch_topk_select(const float* scores, const int64_t* row_start, const int32_t* row_len, int R, int k,
                              int max_len, int32_t* S, float* S_score, void* ws, hipStream_t st) {
    (void)max_len;
    (void)ws;
    TopkArgs a;
    a.scores = scores;
    a.row_start = row_start;
    a.row_len = row_len;
    a.k = k;
    a.cap = topk_cap(k);
    a.S = S;
    a.Ss = S_score;
    TLSL_TIMED_LAUNCH("topk_row_kernel", st, hipLaunchKernelGGL(topk_row_kernel, dim3(R), dim3(TR_NT), 0, st, a));
    return hipGetLastError();
}

}  // namespace tlsl
