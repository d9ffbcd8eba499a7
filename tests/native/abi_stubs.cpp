// abi_stubs.cpp -- stand-ins for the kernel launchers and device queries, so
// that the host layer (abi.cpp, plan.cpp) can be built with g++ under the
// address and undefined-behaviour sanitizers and driven without a GPU.  Each
// launcher records that it was reached and returns hipSuccess; nothing is
// dereferenced.  TEST INFRASTRUCTURE ONLY.
#include <stdint.h>
#include <stdio.h>

#include "../../token_level_sparse_lightning_amd/csrc/tlsl_internal.h"

int g_launches = 0;

extern "C" const char* hipGetErrorString(hipError_t) { return "stubbed HIP error"; }

namespace tlsl {
int device_cu_count() { return 256; }
void timer_mark(const char*, hipStream_t, bool) {}
hipError_t launch_index_prefill(const IndexerShape&, const void*, const float*, const void*, const float*,
                                const float*, int, int, int, int32_t*, float*, void*, const PrefillPlan&,
                                hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_index_prefill_rerank(const IndexerShape&, const void*, const float*, const void*, const float*,
                                       const void*, const void*, const float*, int, int, int, int, int32_t*, float*,
                                       int32_t*, void*, const PrefillPlan&, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_index_decode(const IndexerShape&, const void*, const float*, const void*, const float*,
                               const float*, const int64_t*, int, int, float*, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t topk_noalloc_scratch(void** out) {
    *out = reinterpret_cast<void*>(uintptr_t(0x20000));
    return hipSuccess;
}
hipError_t launch_topk_select(const float*, const int64_t*, const int32_t*, int, int, int, int32_t*, float*, void*,
                              hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_indexer_kl(const void*, const void*, const float*, const int32_t*, const float*, int, int, int,
                             int, float*, float*, float*, float*, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_selection_quality(const float*, const int64_t*, const int32_t*, int, const int32_t*, int, int, int,
                                    float*, float*, void*, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_cutoff_margin(const float*, const int64_t*, const int32_t*, int, int, int, float*, void*,
                                hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_sparse_attn_prefill(const AttnShape&, const void*, const void*, const int32_t*, int, int, int,
                                      float, void*, float*, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_fill_all_history(int32_t*, int, int, int, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_sparse_attn_decode(const AttnShape&, const void*, const void*, const int64_t*, const int32_t*,
                                     int, int, float, void*, float*, void*, hipStream_t) {
    ++g_launches;
    return hipErrorInvalidValue;  // the launch-error path: mapped to TLSL_ERR_HIP
}
int g_debug_checks = 0;
int debug_check_seqlens(const int64_t*, int, bool, hipStream_t, const char*) {
    ++g_debug_checks;
    return 0;
}
int debug_check_rows(const int64_t*, const int32_t*, int, hipStream_t, const char*) {
    ++g_debug_checks;
    return 0;
}
}  // namespace tlsl
