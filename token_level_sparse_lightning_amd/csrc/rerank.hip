// rerank.hip -- coarse recall, then re-rank, on gfx950 (DSA page, section 2,
// the paragraph on the quantised key cache: the FP8 indexer recalls a larger
// candidate set, a higher-precision indexer ranks it).
//
// index_prefill on the fp8 inputs with budget k' gives each row's candidates
// C_t (ascending positions, then -1).  rerank_kernel, one workgroup per row:
//  0. the row's candidate positions are staged in LDS, so that no gather
//     waits for a position loaded from global memory just before it;
//  1. each wave scores 64 candidates at a time with the fine (bf16) query and
//     the candidates' fine keys, gathered straight from global memory, through
//     the indexer's scoring tile (idx_tile.h: the same instructions as
//     index_prefill, so all-history candidates reproduce the plain bf16
//     selection bit for bit);
//  2. the candidates' score keys and positions are held in registers and the
//     exact top-K is written in position order by the same register-visiting
//     select as the prefill finalize (topk_common.h: select_ordered).
#include "idx_tile.h"
#include "tlsl_device.h"
#include "tlsl_internal.h"
#include "topk_common.h"

namespace tlsl {

constexpr int RR_NT = 256;

struct RerankArgs {
    const unsigned char* q;  // fine [rows][HI][DI]
    const unsigned char* k;  // fine [B*n][DI]
    const float* w;          // [rows][HI]
    const int32_t* C;        // [rows][kc] candidates (index_prefill's layout)
    int n, HI, topk, kc;
    int32_t* S;
    float* Ss;
};

template <int DT, int HB, int DI, int CAPMAX>
__global__ __launch_bounds__(RR_NT) void rerank_kernel(RerankArgs a) {
    using I = Idx<DT, HB, DI>;
    constexpr int NCH = I::NCH;
    constexpr int SEG = CAPMAX / RR_NT;
    __shared__ float sc[CAPMAX];
    __shared__ int cpos[CAPMAX];  // the row's candidate positions
    __shared__ SelectSmem sel;
    __shared__ int gcnt[2][SEG * (RR_NT / 64)];
    const int tid = threadIdx.x, l = lane_id(), g = l >> 4, c = l & 15;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int row = blockIdx.x;
    const int t = row % a.n;
    const size_t tok0 = (size_t)row - t;
    // index_prefill writes min(kc, t+1) ascending positions, then -1
    const int nc = min(a.kc, t + 1);
    const int32_t* Crow = a.C + (size_t)row * a.kc;
    const unsigned char* kbase = a.k + tok0 * I::ROWB;
    for (int i = tid; i < nc; i += RR_NT) cpos[i] = Crow[i];
    __syncthreads();
    {
        uint4 qf[HB][NCH];
        float wvv[HB][4];
        I::load_query(a.q + (size_t)row * a.HI * I::ROWB, a.w + (size_t)row * a.HI, 1.f, a.HI, true, qf, wvv);
        // the wave's subtiles j = wv, wv + 4, ...; the next one's keys are
        // gathered while this one is scored (two register sets, alternating)
        auto gather = [&](int j, uint4 (&kf)[4][NCH]) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int i = min(64 * j + 16 * kb + c, nc - 1);  // past the end: a valid, unused key
                const uint4* src =
                    reinterpret_cast<const uint4*>(kbase + (size_t)cpos[i] * I::ROWB + g * (I::ROWB / 4));
#pragma unroll
                for (int ch = 0; ch < NCH; ++ch) kf[kb][ch] = src[ch];
            }
        };
        constexpr int STEP = RR_NT / 64;
        uint4 kfa[4][NCH], kfb[4][NCH];
        int j = wv;
        if (64 * j < nc) gather(j, kfa);
        while (64 * j < nc) {
            if (64 * (j + STEP) < nc) gather(j + STEP, kfb);
            float s = I::score(qf, wvv, kfa);
            if (64 * j + l < nc) sc[64 * j + l] = s;
            j += STEP;
            if (64 * j >= nc) break;
            if (64 * (j + STEP) < nc) gather(j + STEP, kfa);
            s = I::score(qf, wvv, kfb);
            if (64 * j + l < nc) sc[64 * j + l] = s;
            j += STEP;
        }
    }
    __syncthreads();
    uint32_t key[SEG];
    int pos[SEG];
#pragma unroll
    for (int u = 0; u < SEG; ++u) {
        const int i = tid + u * RR_NT;
        key[u] = i < nc ? score_key(sc[i]) : 0u;
        pos[u] = i < nc ? cpos[i] : -1;
    }
    select_ordered<RR_NT, SEG>(key, pos, nc, min(a.topk, nc), a.topk, a.S + (size_t)row * a.topk,
                               a.Ss ? a.Ss + (size_t)row * a.topk : nullptr, sel, gcnt);
}

template <int HB>
static hipError_t launch_rerank_hb(const RerankArgs& ra, int rows, hipStream_t st) {
    if (ra.kc <= 1024)
        TLSL_TIMED_LAUNCH("rerank_kernel", st,
                          hipLaunchKernelGGL((rerank_kernel<kBF16, HB, 128, 1024>), dim3(rows), dim3(RR_NT), 0, st, ra));
    else
        TLSL_TIMED_LAUNCH("rerank_kernel", st,
                          hipLaunchKernelGGL((rerank_kernel<kBF16, HB, 128, 4096>), dim3(rows), dim3(RR_NT), 0, st, ra));
    return hipGetLastError();
}

hipError_t launch_index_prefill_rerank(const IndexerShape& coarse, const void* q8, const float* q_scale,
                                       const void* k8, const float* k_scale, const void* qf, const void* kf,
                                       const float* w, int B, int n, int topk, int kc, int32_t* S, float* S_score,
                                       int32_t* C, void* ws, const PrefillPlan& plan, hipStream_t st) {
    // coarse recall: the fp8 indexer with budget kc
    hipError_t e = launch_index_prefill(coarse, q8, q_scale, k8, k_scale, w, B, n, kc, C, nullptr, ws, plan, st);
    if (e != hipSuccess) return e;
    RerankArgs ra;
    ra.q = static_cast<const unsigned char*>(qf);
    ra.k = static_cast<const unsigned char*>(kf);
    ra.w = w;
    ra.C = C;
    ra.n = n;
    ra.HI = coarse.HI;
    ra.topk = topk;
    ra.kc = kc;
    ra.S = S;
    ra.Ss = S_score;
    const int hb = coarse.HI <= 16 ? 1 : (coarse.HI <= 32 ? 2 : 4);
    if (hb == 1) return launch_rerank_hb<1>(ra, B * n, st);
    if (hb == 2) return launch_rerank_hb<2>(ra, B * n, st);
    return launch_rerank_hb<4>(ra, B * n, st);
}

}  // namespace tlsl
