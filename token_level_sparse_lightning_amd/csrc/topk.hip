// topk.hip -- topk_select: exact top-k of explicit variable-length score rows
// (DSA page, section 1.1 eq.(2); section 2 on radix top-k over rows given by
// sequence lengths).  One workgroup per row runs the radix select of
// topk_common.h.
#include "tlsl_device.h"
#include "tlsl_internal.h"
#include "topk_common.h"

namespace tlsl {

constexpr int TS_NT = 512;

__global__ __launch_bounds__(TS_NT) void topk_select_kernel(const float* scores, const int64_t* row_start,
                                                            const int32_t* row_len, int k, int32_t* S,
                                                            float* Ss) {
    __shared__ TopkSmem sm;
    const int r = blockIdx.x;
    const int L = max(row_len[r], 0);
    block_topk_row<TS_NT>(scores + row_start[r], L, k, S + (size_t)r * k, Ss ? Ss + (size_t)r * k : nullptr, sm);
}

size_t topk_ws_bytes(int, int, int) { return 0; }

hipError_t launch_topk_select(const float* scores, const int64_t* row_start, const int32_t* row_len, int R,
                              int k, int, int32_t* S, float* S_score, void*, hipStream_t st) {
    hipLaunchKernelGGL(topk_select_kernel, dim3(R), dim3(TS_NT), 0, st, scores, row_start, row_len, k, S, S_score);
    return hipGetLastError();
}

}  // namespace tlsl
