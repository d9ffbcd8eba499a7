// tlsl_internal.h -- host-side launcher interface between the C ABI layer and
// the kernels.  Launchers assume validated arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tlsl {

// Compute units of the current device (queried once per device).
int device_cu_count();

// Sets the thread-local message that tlsl_last_error returns (cleared for
// TLSL_OK) and returns `code`.
int report(int code, const char* fmt, ...);

// Kernel timer hook: records the armed event pair around a launch of the
// kernel called `kernel` on stream `st` (no-op unless that kernel is armed).
void timer_mark(const char* kernel, hipStream_t st, bool after);

#define TLSL_TIMED_LAUNCH(name, st, ...)        \
    do {                                        \
        ::tlsl::timer_mark(name, st, false);    \
        __VA_ARGS__;                            \
        ::tlsl::timer_mark(name, st, true);     \
    } while (0)

// ---- indexer ---------------------------------------------------------------
struct IndexerShape {
    int dt;      // 0 f32, 1 bf16, 2 fp8
    int HI, DI;
};
bool indexer_supported(const IndexerShape& s);

struct PrefillPlan {
    int cap;            // candidate buffer entries per query row
    int stride;         // key stride of the threshold sample
    size_t ws_bytes;    // workspace needed
    size_t off_buf, off_cnt, off_fbcount, off_fblist, off_fbscratch;
    int fb_blocks;      // workgroups of the fallback pass
};
PrefillPlan plan_prefill(const IndexerShape& s, int B, int n, int k);

hipError_t launch_index_prefill(const IndexerShape& s, const void* q, const float* q_scale,
                                const void* k, const float* k_scale, const float* w, int B,
                                int n, int topk, int32_t* S, float* S_score, void* ws,
                                const PrefillPlan& plan, hipStream_t st);

hipError_t launch_index_decode(const IndexerShape& s, const void* q, const float* q_scale,
                               const void* kc, const float* k_scale, const float* w,
                               const int64_t* cu, int B, int max_len, float* scores,
                               hipStream_t st);

// ---- row top-k ---------------------------------------------------------------
size_t topk_ws_bytes(int R, int k, int max_len);
hipError_t launch_topk_select(const float* scores, const int64_t* row_start,
                              const int32_t* row_len, int R, int k, int max_len, int32_t* S,
                              float* S_score, void* ws, hipStream_t st);

// ---- sparse attention ---------------------------------------------------------
struct AttnShape {
    int dt;  // 0 f32, 1 bf16
    int H, Dqk, Dv;
};
bool attn_supported(const AttnShape& s);
size_t attn_decode_ws_bytes(const AttnShape& s, int B, int k);
hipError_t launch_sparse_attn_prefill(const AttnShape& s, const void* q, const void* kv,
                                      const int32_t* S, int B, int n, int k, float scale,
                                      void* out, float* lse, hipStream_t st);
hipError_t launch_sparse_attn_decode(const AttnShape& s, const void* q, const void* kv,
                                     const int64_t* cu, const int32_t* S, int B, int k,
                                     float scale, void* out, float* lse, void* ws,
                                     hipStream_t st);

}  // namespace tlsl
