// diag.hip -- selection-quality diagnostics on gfx950 (DSA page, section 1.2
// eq.(9) and section 3.1 eq.(14), (15), (18)): how much of a teacher
// distribution a selection covers, and how close each row's selection is to
// its cutoff.
//
//  * selection_quality: G = TopK(teacher, min(m, L)) by the selection rule of
//    eq.(2) (topk_select on the teacher rows), then per row
//      recall = |G n S| / |G|                         eq.(9) (eq.(14): m = k)
//      mass   = sum_{s in S} a_s / sum_{s < L} a_s     eq.(15)
//    one workgroup per row: the row total and the covered mass accumulate in
//    fp64 in a fixed order; G's positions are looked up in the (ascending)
//    selection by binary search.
//  * cutoff_margin: Delta_k = s_(K) - s_(K+1) (eq.(18)), from the top-(K+1)
//    of the row (topk_select with k + 1): the two smallest of those K+1
//    scores; +inf when the row has no (K+1)-th score.
#include <math.h>

#include <algorithm>

#include "tlsl_device.h"
#include "tlsl_internal.h"

namespace tlsl {

constexpr int DG_NT = 256;

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    return v;
}

__global__ __launch_bounds__(DG_NT) void selection_quality_kernel(const float* teacher, const int64_t* row_start,
                                                                  const int32_t* row_len, const int32_t* S, int k,
                                                                  const int32_t* G, int m, float* recall,
                                                                  float* mass) {
    __shared__ double red[2][DG_NT / 64];
    __shared__ int ired[DG_NT / 64][2];
    const int r = blockIdx.x, tid = threadIdx.x, w = tid >> 6;
    const int L = max(row_len[r], 0);
    const float* a = teacher + row_start[r];
    const int32_t* Sr = S + (size_t)r * k;
    const int32_t* Gr = G + (size_t)r * m;
    // valid prefix of the selection (ascending positions, then -1)
    int ks = 0;
    {
        int lo = 0, hi = k;  // first slot that is < 0
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (Sr[mid] >= 0) lo = mid + 1;
            else hi = mid;
        }
        ks = lo;
    }
    double tot = 0.0, cov = 0.0;
    {
        // eight loads per thread in flight, added in a fixed order
        int s = tid;
        for (; s + 7 * DG_NT < L; s += 8 * DG_NT) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = a[s + u * DG_NT];
#pragma unroll
            for (int u = 0; u < 8; ++u) tot += (double)v[u];
        }
        for (; s < L; s += DG_NT) tot += (double)a[s];
    }
    for (int i = tid; i < ks; i += DG_NT) {
        const int s = Sr[i];
        if (s < L) cov += (double)a[s];
    }
    int ng = 0, hit = 0;
    for (int i = tid; i < m; i += DG_NT) {
        const int gpos = Gr[i];
        if (gpos < 0) continue;
        ++ng;
        int lo = 0, hi = ks;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (Sr[mid] < gpos) lo = mid + 1;
            else hi = mid;
        }
        hit += lo < ks && Sr[lo] == gpos;
    }
    tot = wave_sum_f64(tot);
    cov = wave_sum_f64(cov);
    ng = wave_sum(ng);
    hit = wave_sum(hit);
    if (lane_id() == 0) {
        red[0][w] = tot;
        red[1][w] = cov;
        ired[w][0] = ng;
        ired[w][1] = hit;
    }
    __syncthreads();
    if (tid == 0) {
        double T = 0.0, C = 0.0;
        int NG = 0, HIT = 0;
        for (int i = 0; i < DG_NT / 64; ++i) {
            T += red[0][i];
            C += red[1][i];
            NG += ired[i][0];
            HIT += ired[i][1];
        }
        mass[r] = T > 0.0 ? (float)(C / T) : NAN;
        recall[r] = NG > 0 ? (float)HIT / (float)NG : NAN;
    }
}

// one wave per row: the two smallest of the row's top-(k+1) scores
__global__ __launch_bounds__(DG_NT) void cutoff_margin_kernel(const float* Ss, const int32_t* row_len, int R, int k,
                                                              float* margin) {
    const int r = blockIdx.x * (DG_NT / 64) + (threadIdx.x >> 6);
    if (r >= R) return;
    const int L = max(row_len[r], 0);
    if (L <= k) {
        if (lane_id() == 0) margin[r] = INFINITY;
        return;
    }
    const float* row = Ss + (size_t)r * (k + 1);
    float mn = INFINITY;
    for (int i = lane_id(); i <= k; i += 64) mn = fminf(mn, row[i]);
    mn = wave_min(mn);
    int nmin = 0;
    float second = INFINITY;
    for (int i = lane_id(); i <= k; i += 64) {
        const float v = row[i];
        if (v == mn) ++nmin;
        else second = fminf(second, v);
    }
    nmin = wave_sum(nmin);
    second = wave_min(second);
    if (lane_id() == 0) margin[r] = nmin >= 2 ? 0.f : second - mn;
}

hipError_t launch_selection_quality(const float* teacher, const int64_t* row_start, const int32_t* row_len, int R,
                                    const int32_t* S, int k, int m, int max_len, float* recall, float* mass, void* ws,
                                    hipStream_t st) {
    // the teacher's top-m, then the per-row counts and sums
    unsigned char* w = static_cast<unsigned char*>(ws);
    int32_t* G = reinterpret_cast<int32_t*>(w);
    const size_t g_bytes = ((size_t)R * m * sizeof(int32_t) + 255) & ~(size_t)255;
    hipError_t e = launch_topk_select(teacher, row_start, row_len, R, m, max_len, G, nullptr, w + g_bytes, st);
    if (e != hipSuccess) return e;
    TLSL_TIMED_LAUNCH("selection_quality_kernel", st,
                      hipLaunchKernelGGL(selection_quality_kernel, dim3(R), dim3(DG_NT), 0, st, teacher, row_start,
                                         row_len, S, k, G, m, recall, mass));
    return hipGetLastError();
}

hipError_t launch_cutoff_margin(const float* scores, const int64_t* row_start, const int32_t* row_len, int R, int k,
                                int max_len, float* margin, void* ws, hipStream_t st) {
    unsigned char* w = static_cast<unsigned char*>(ws);
    const size_t sel = ((size_t)R * (k + 1) * sizeof(int32_t) + 255) & ~(size_t)255;
    int32_t* S1 = reinterpret_cast<int32_t*>(w);
    float* Ss1 = reinterpret_cast<float*>(w + sel);
    hipError_t e = launch_topk_select(scores, row_start, row_len, R, k + 1, max_len, S1, Ss1, w + 2 * sel, st);
    if (e != hipSuccess) return e;
    TLSL_TIMED_LAUNCH("cutoff_margin_kernel", st,
                      hipLaunchKernelGGL(cutoff_margin_kernel, dim3((R + DG_NT / 64 - 1) / (DG_NT / 64)), dim3(DG_NT),
                                         0, st, Ss1, row_len, R, k, margin));
    return hipGetLastError();
}

}  // namespace tlsl
