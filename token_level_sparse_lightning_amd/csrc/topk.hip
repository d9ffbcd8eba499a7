// topk.hip -- topk_select: exact top-k of explicit variable-length score rows
// (DSA page, section 1.1 eq.(2); section 2 on radix top-k over rows given by
// sequence lengths, avoiding a full sort).
//
// Three launches, every one spread over many workgroups:
//  1. topk_threshold: per row, the r-th largest of a strided sample of the
//     row (r = expected sample hits inside the top-k plus 4 standard
//     deviations) -- a conservative threshold.
//  2. topk_filter: workgroups over (row chunk) append every (score, position)
//     at or above the row's threshold to the row's candidate buffer.
//  3. topk_final: per row, an exact radix select among the candidates in LDS,
//     ties resolved to the lowest positions, and the selected positions
//     written in ascending order through a position bitmap.  A row whose
//     candidates miss (the sample threshold overshot) or overflow is selected
//     from its full score row instead (topk_common.h).
// The result never depends on the threshold, only the work does.
#include <math.h>

#include <algorithm>
#include <mutex>

#include "../../include/tlsl.h"
#include "tlsl_device.h"
#include "tlsl_internal.h"
#include "topk_common.h"

namespace tlsl {

constexpr int TT_NT = 1024;             // threshold workgroup
constexpr int TT_SAMPLE_MAX = 4096;     // sample values per row (held in registers)
constexpr int TF_NT = 256;              // filter workgroup
constexpr int TF_PER = 8;               // scores per filter thread (more workgroups in flight than with 16)
constexpr int TF_CHUNK = TF_NT * TF_PER;
constexpr int TFIN_NT = 1024;           // final workgroup
constexpr int TSEL_CAPMAX = 8448;       // candidate buffer entries per row, max
constexpr int TSEL_BITMAP_WORDS = 4096; // rows up to 131072 use the bitmap output
constexpr int TSEL_CNT_STRIDE = kTopkCntStride;  // one 128-byte line per row counter
constexpr float TSEL_SIGMA = 4.0f;

struct TopkArgs {
    const float* scores;
    const int64_t* row_start;
    const int32_t* row_len;
    int k, cap;
    float* theta;   // [R]
    int* cnt;       // [R]
    uint2* buf;     // [R][cap]
    int32_t* S;
    float* Ss;
};

__device__ __forceinline__ int sample_stride(int L) { return max(16, (L + TT_SAMPLE_MAX - 1) / TT_SAMPLE_MAX); }

__global__ __launch_bounds__(TT_NT) void topk_threshold_kernel(TopkArgs a) {
    // sample j of the row is held in registers by thread j % TT_NT
    constexpr int SEG = TT_SAMPLE_MAX / TT_NT;
    __shared__ SelectSmem sel;
    const int r = blockIdx.x, tid = threadIdx.x;
    const int L = max(a.row_len[r], 0);
    if (tid == 0) a.cnt[r * TSEL_CNT_STRIDE] = 0;
    const int K = min(a.k, L);
    const int stride = sample_stride(L);
    const int ns = L > 0 ? (L - 1) / stride + 1 : 0;
    const float mu = L > 0 ? (float)ns * (float)K / (float)L : 0.f;
    const int need = (int)ceilf(mu + TSEL_SIGMA * sqrtf(mu)) + 2;
    if (L <= a.cap || need >= ns) {
        if (tid == 0) a.theta[r] = -INFINITY;
        return;
    }
    const float* sc = a.scores + a.row_start[r];
    // every load issued before any is used (indices clamped, so always in
    // bounds; samples past ns are never visited)
    float v[SEG];
#pragma unroll
    for (int u = 0; u < SEG; ++u) v[u] = sc[(size_t)min(tid + u * TT_NT, ns - 1) * stride];
    uint32_t key[SEG];
#pragma unroll
    for (int u = 0; u < SEG; ++u) key[u] = score_key(v[u]);
    const auto each = [&](auto&& f) {
#pragma unroll
        for (int u = 0; u < SEG; ++u)
            if (tid + u * TT_NT < ns) f(key[u]);
    };
    int gt;
    const uint32_t T = block_select_each<TT_NT>(need, each, sel, &gt, true);
    if (tid == 0) a.theta[r] = key_score(T);
}

__global__ __launch_bounds__(TF_NT) void topk_filter_kernel(TopkArgs a) {
    const int r = blockIdx.y;
    const int L = max(a.row_len[r], 0);
    __shared__ int wsum[TF_NT / 64 + 1];
    const float th = a.theta[r];
    const float* sc = a.scores + a.row_start[r];
    uint2* out = a.buf + (size_t)r * a.cap;
    const int w = threadIdx.x >> 6;
    // chunks blockIdx.x, + gridDim.x, ...: a row longer than the launch was
    // sized for (max_len) is still filtered in full
    for (int64_t base64 = (int64_t)blockIdx.x * TF_CHUNK; base64 < L; base64 += (int64_t)gridDim.x * TF_CHUNK) {
        const int base = (int)base64;  // idx below stays < L + TF_CHUNK; rows hold < 2^31 - TF_CHUNK scores
        float v[TF_PER];
#pragma unroll
        for (int i = 0; i < TF_PER; ++i) {
            const int idx = base + i * TF_NT + threadIdx.x;
            v[i] = idx < L ? sc[idx] : -INFINITY;
        }
        // count first, then reserve the workgroup's slots with a single atomic
        uint64_t m[TF_PER];
        int mine = 0;
#pragma unroll
        for (int i = 0; i < TF_PER; ++i) {
            const int idx = base + i * TF_NT + threadIdx.x;
            m[i] = ballot(idx < L && v[i] >= th);
            mine += __popcll(m[i]);
        }
        if (lane_id() == 0) wsum[w] = mine;
        __syncthreads();
        if (threadIdx.x == 0) {
            int tot = 0;
            for (int i = 0; i < TF_NT / 64; ++i) tot += wsum[i];
            wsum[TF_NT / 64] = tot > 0 ? atomicAdd(&a.cnt[r * TSEL_CNT_STRIDE], tot) : 0;
        }
        __syncthreads();
        int slot = wsum[TF_NT / 64];
        for (int i = 0; i < w; ++i) slot += wsum[i];
#pragma unroll
        for (int i = 0; i < TF_PER; ++i) {
            const int idx = base + i * TF_NT + threadIdx.x;
            const bool ok = (m[i] >> lane_id()) & 1ull;
            const int s = slot + rank_below(m[i]);
            if (ok && s < a.cap) out[s] = make_uint2(__float_as_uint(v[i]), (uint32_t)idx);
            slot += __popcll(m[i]);
        }
        __syncthreads();  // wsum is reused by the next chunk
    }
}

struct TopkFinalSmem {
    uint32_t keys[TSEL_CAPMAX];
    uint32_t pos[TSEL_CAPMAX];
    uint32_t bitmap[TSEL_BITMAP_WORDS];
    SelectSmem sel;
    int nties;
};

union TopkFinalShared {
    TopkFinalSmem f;
    TopkSmem g;
};

__global__ __launch_bounds__(TFIN_NT) void topk_final_kernel(TopkArgs a) {
    __shared__ TopkFinalShared sh;
    const int r = blockIdx.x, tid = threadIdx.x;
    const int L = max(a.row_len[r], 0);
    const int K = min(a.k, L);
    const float* sc = a.scores + a.row_start[r];
    int32_t* Srow = a.S + (size_t)r * a.k;
    float* Ssrow = a.Ss ? a.Ss + (size_t)r * a.k : nullptr;
    const int cnt = a.cnt[r * TSEL_CNT_STRIDE];
    const int nwords = (L + 31) / 32;
    if (L > a.k && (cnt < K || cnt > a.cap || nwords > TSEL_BITMAP_WORDS)) {
        block_topk_row<TFIN_NT>(sc, L, a.k, Srow, Ssrow, sh.g);
        return;
    }
    if (L <= a.k) {
        for (int i = tid; i < a.k; i += TFIN_NT) {
            Srow[i] = i < L ? i : -1;
            if (Ssrow) Ssrow[i] = i < L ? sc[i] : -INFINITY;
        }
        return;
    }
    TopkFinalSmem& s = sh.f;
    const uint2* src = a.buf + (size_t)r * a.cap;
    if (cnt > 0)
        batched_copy<TFIN_NT, 8>(cnt, [&](int i) { return src[i]; }, [&](int i, uint2 e) {
            s.keys[i] = score_key(__uint_as_float(e.x));
            s.pos[i] = e.y;
        });
    for (int i = tid; i < nwords; i += TFIN_NT) s.bitmap[i] = 0u;
    if (tid == 0) s.nties = 0;
    __syncthreads();
    int gt;
    // the filtered candidates (a row whose ties overflow them takes the
    // full-row path above): one atomic per key
    const uint32_t T = block_select_adaptive<TFIN_NT, false>(
        cnt, K, [&](int i, bool* ok) { *ok = true; return s.keys[i]; }, s.sel, &gt);
    // ties at T: keep the (K - gt) lowest positions, i.e. the largest inverted
    // positions; when every tie is kept no selection is needed
    const int need_ties = K - gt;
    int nt_local = 0;
    for (int i = tid; i < cnt; i += TFIN_NT) nt_local += s.keys[i] == T;
    nt_local = wave_sum(nt_local);
    if (lane_id() == 0 && nt_local) atomicAdd(&s.nties, nt_local);
    __syncthreads();
    uint32_t inv_cut = 0u;
    if (s.nties > need_ties) {
        int tgt;
        inv_cut = block_select_adaptive<TFIN_NT, false>(
            cnt, need_ties, [&](int i, bool* ok) { *ok = s.keys[i] == T; return ~s.pos[i]; }, s.sel, &tgt);
    }
    for (int i = tid; i < cnt; i += TFIN_NT) {
        const uint32_t key = s.keys[i];
        if (key > T || (key == T && ~s.pos[i] >= inv_cut)) atomicOr(&s.bitmap[s.pos[i] >> 5], 1u << (s.pos[i] & 31));
    }
    __syncthreads();
    // ordered output: each thread owns a contiguous run of bitmap words
    const int per = (nwords + TFIN_NT - 1) / TFIN_NT;
    const int w0 = min(nwords, tid * per), w1 = min(nwords, w0 + per);
    int mine = 0;
    for (int wd = w0; wd < w1; ++wd) mine += __popc(s.bitmap[wd]);
    int total;
    int o = block_excl_scan<TFIN_NT>(mine, &total, s.sel.scratch);
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
    for (int i = K + tid; i < a.k; i += TFIN_NT) {
        Srow[i] = -1;
        if (Ssrow) Ssrow[i] = -INFINITY;
    }
}

hipError_t launch_topk_select(const float* scores, const int64_t* row_start, const int32_t* row_len, int R, int k,
                              int max_len, int32_t* S, float* S_score, void* ws, hipStream_t st) {
    unsigned char* w = static_cast<unsigned char*>(ws);
    TopkArgs a;
    a.scores = scores;
    a.row_start = row_start;
    a.row_len = row_len;
    a.k = k;
    const TopkLayout lay = topk_layout(R, k);
    a.cap = lay.cap;
    a.theta = reinterpret_cast<float*>(w + lay.off_theta);
    a.cnt = reinterpret_cast<int*>(w + lay.off_cnt);
    a.buf = reinterpret_cast<uint2*>(w + lay.off_buf);
    a.S = S;
    a.Ss = S_score;
    TLSL_TIMED_LAUNCH("topk_threshold_kernel", st, hipLaunchKernelGGL(topk_threshold_kernel, dim3(R), dim3(TT_NT), 0, st, a));
    const int chunks = max_len > 0 ? std::min((max_len + TF_CHUNK - 1) / TF_CHUNK, 65535) : 1;
    TLSL_TIMED_LAUNCH("topk_filter_kernel", st,
                      hipLaunchKernelGGL(topk_filter_kernel, dim3(chunks, R), dim3(TF_NT), 0, st, a));
    TLSL_TIMED_LAUNCH("topk_final_kernel", st, hipLaunchKernelGGL(topk_final_kernel, dim3(R), dim3(TFIN_NT), 0, st, a));
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Allocation-free variant: topk_select_noalloc runs the same three kernels
// with their workspace in this file-scope device array (one per device, held
// until the process ends).  Every byte of it that the kernels read is written
// earlier in the same call (the threshold kernel sets each row's threshold
// and zeroes its counter, the filter fills the candidate buffers up to that
// counter), so nothing needs clearing between calls; calls that overlap on
// one device share the array and race.  Host code never uses the array's name
// as an address: it takes the device address with hipGetSymbolAddress, once
// per device with that device current, and passes that pointer.
static __device__ __align__(256) unsigned char scratch[TLSL_NOALLOC_SCRATCH_BYTES];

hipError_t topk_noalloc_scratch(void** out) {
    static std::mutex mu;
    static void* addr[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}

}  // namespace tlsl
