// abi.cpp -- the extern "C" entry points declared in include/tlsl.h: argument
// validation (all of it on the host, before anything is launched), workspace
// sizing and dispatch to the gfx950 kernels.  No exception crosses the ABI.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/tlsl.h"
#include "tlsl_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return TLSL_OK;
}

bool aligned16(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

const char* dt_name(int dt) {
    switch (dt) {
        case TLSL_F32: return "f32";
        case TLSL_BF16: return "bf16";
        case TLSL_FP8_E4M3: return "fp8_e4m3";
        default: return "?";
    }
}

// Shared checks of the workspace protocol.  Returns 1 if the caller only
// asked for the size (already written), 0 to proceed, <0 on error.
int workspace_protocol(void* workspace, size_t* ws_bytes, size_t need) {
    if (!ws_bytes) return fail(TLSL_ERR_NULL, "ws_bytes is NULL");
    if (!workspace) {
        *ws_bytes = need;
        return 1;
    }
    if (*ws_bytes < need) return fail(TLSL_ERR_WORKSPACE, "workspace of %zu bytes, %zu required", *ws_bytes, need);
    if (!aligned16(workspace)) return fail(TLSL_ERR_ALIGN, "workspace is not 16-byte aligned");
    return 0;
}

int launch_result(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(TLSL_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

int check_indexer(int dt, const void* q, const float* q_scale, const void* k, const float* k_scale, const float* w,
                  int HI, int dI, const char* fn) {
    if (dt != TLSL_F32 && dt != TLSL_BF16 && dt != TLSL_FP8_E4M3) return fail(TLSL_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, dt);
    if (!q || !k || !w) return fail(TLSL_ERR_NULL, "%s: qI, kI and wI must be non-NULL", fn);
    if (dt == TLSL_FP8_E4M3 && (!q_scale || !k_scale)) return fail(TLSL_ERR_NULL, "%s: fp8 needs q_scale and k_scale", fn);
    if (dt != TLSL_FP8_E4M3 && (q_scale || k_scale))
        return fail(TLSL_ERR_SHAPE, "%s: scales are only meaningful for fp8 inputs", fn);
    if (HI <= 0 || dI <= 0) return fail(TLSL_ERR_SHAPE, "%s: HI=%d and dI=%d must be positive", fn, HI, dI);
    tlsl::IndexerShape s{dt, HI, dI};
    if (!tlsl::indexer_supported(s))
        return fail(TLSL_ERR_UNSUPPORTED, "%s: (dtype %s, HI=%d, dI=%d) is not built (f32: dI 32|64; bf16: dI 32|64|128; "
                    "fp8: dI 128; HI 1..64)", fn, dt_name(dt), HI, dI);
    if (!aligned16(q) || !aligned16(k) || !aligned16(w) || !aligned16(q_scale) || !aligned16(k_scale))
        return fail(TLSL_ERR_ALIGN, "%s: tensor pointers must be 16-byte aligned", fn);
    return 0;
}

}  // namespace

int tlsl::report(int code, const char* fmt, ...) {
    if (code == TLSL_OK || !fmt) {
        g_err[0] = '\0';
        return code;
    }
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

extern "C" {

const char* tlsl_last_error(void) { return g_err; }

const char* tlsl_version(void) { return "tlsl 0.1 (gfx950)"; }

int index_prefill(const void* qI, const float* q_scale, const void* kI, const float* k_scale, const float* wI, int B,
                  int n, int HI, int dI, int k, tlsl_dtype dt, int32_t* S, float* S_score, void* workspace,
                  size_t* ws_bytes, hipStream_t stream) {
    int rc = check_indexer(dt, qI, q_scale, kI, k_scale, wI, HI, dI, "index_prefill");
    if (rc) return rc;
    if (!S) return fail(TLSL_ERR_NULL, "index_prefill: S must be non-NULL");
    if (B <= 0 || n <= 0) return fail(TLSL_ERR_SHAPE, "index_prefill: B=%d and n=%d must be positive", B, n);
    if (k <= 0) return fail(TLSL_ERR_SHAPE, "index_prefill: k=%d must be positive", k);
    if (k > 4096) return fail(TLSL_ERR_UNSUPPORTED, "index_prefill: k=%d above the supported 4096", k);
    if ((int64_t)B * n > (int64_t)1 << 30) return fail(TLSL_ERR_SHAPE, "index_prefill: B*n too large");
    if (!aligned16(S) || !aligned16(S_score)) return fail(TLSL_ERR_ALIGN, "index_prefill: S/S_score not 16-byte aligned");
    tlsl::IndexerShape s{dt, HI, dI};
    const tlsl::PrefillPlan plan = tlsl::plan_prefill(s, B, n, k);
    rc = workspace_protocol(workspace, ws_bytes, plan.ws_bytes);
    if (rc) return rc > 0 ? ok() : rc;
    return launch_result(tlsl::launch_index_prefill(s, qI, q_scale, kI, k_scale, wI, B, n, k, S, S_score, workspace,
                                                    plan, stream),
                         "index_prefill");
}

int index_decode(const void* qI, const float* q_scale, const void* kI_cache, const float* k_scale, const float* wI,
                 const int64_t* cu_seqlens, int B, int HI, int dI, int max_len, tlsl_dtype dt, float* scores,
                 void* workspace, size_t* ws_bytes, hipStream_t stream) {
    int rc = check_indexer(dt, qI, q_scale, kI_cache, k_scale, wI, HI, dI, "index_decode");
    if (rc) return rc;
    if (!cu_seqlens || !scores) return fail(TLSL_ERR_NULL, "index_decode: cu_seqlens and scores must be non-NULL");
    if (B <= 0) return fail(TLSL_ERR_SHAPE, "index_decode: B=%d must be positive", B);
    if (max_len <= 0) return fail(TLSL_ERR_SHAPE, "index_decode: max_len=%d must be positive", max_len);
    if (!aligned16(scores) || !aligned16(cu_seqlens)) return fail(TLSL_ERR_ALIGN, "index_decode: pointers not 16-byte aligned");
    (void)workspace;
    if (ws_bytes) *ws_bytes = 0;  // needs no workspace
    tlsl::IndexerShape s{dt, HI, dI};
    return launch_result(tlsl::launch_index_decode(s, qI, q_scale, kI_cache, k_scale, wI, cu_seqlens, B, max_len,
                                                   scores, stream),
                         "index_decode");
}

int topk_select(const float* scores, const int64_t* row_start, const int32_t* row_len, int R, int k, int max_len,
                int32_t* S, float* S_score, void* workspace, size_t* ws_bytes, hipStream_t stream) {
    if (!scores || !row_start || !row_len || !S) return fail(TLSL_ERR_NULL, "topk_select: NULL pointer argument");
    if (R <= 0) return fail(TLSL_ERR_SHAPE, "topk_select: R=%d must be positive", R);
    if (k <= 0) return fail(TLSL_ERR_SHAPE, "topk_select: k=%d must be positive", k);
    if (k > 4096) return fail(TLSL_ERR_UNSUPPORTED, "topk_select: k=%d above the supported 4096", k);
    if (max_len < 0) return fail(TLSL_ERR_SHAPE, "topk_select: max_len=%d must be >= 0", max_len);
    if (!aligned16(S) || !aligned16(S_score) || !aligned16(row_start) || !aligned16(row_len))
        return fail(TLSL_ERR_ALIGN, "topk_select: pointers not 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(scores) & 3u) != 0) return fail(TLSL_ERR_ALIGN, "topk_select: scores not 4-byte aligned");
    const int rc = workspace_protocol(workspace, ws_bytes, tlsl::topk_ws_bytes(R, k, max_len));
    if (rc) return rc > 0 ? ok() : rc;
    return launch_result(tlsl::launch_topk_select(scores, row_start, row_len, R, k, max_len, S, S_score, workspace,
                                                  stream),
                         "topk_select");
}

int sparse_attn_prefill(const void* q, const void* kv, const int32_t* S, int B, int n, int H, int Dqk, int Dv, int k,
                        float softmax_scale, tlsl_dtype dt, void* out, float* lse, void* workspace, size_t* ws_bytes,
                        hipStream_t stream) {
    if (!q || !kv || !S || !out) return fail(TLSL_ERR_NULL, "sparse_attn_prefill: NULL pointer argument");
    if (B <= 0 || n <= 0 || k <= 0 || H <= 0) return fail(TLSL_ERR_SHAPE, "sparse_attn_prefill: B, n, H and k must be positive");
    if ((int64_t)B * n > (int64_t)1 << 30) return fail(TLSL_ERR_SHAPE, "sparse_attn_prefill: B*n too large");
    if (k > 4096) return fail(TLSL_ERR_UNSUPPORTED, "sparse_attn_prefill: k=%d above the supported 4096", k);
    if (dt != TLSL_F32 && dt != TLSL_BF16) return fail(TLSL_ERR_UNSUPPORTED, "sparse_attn_prefill: dtype %d not supported", dt);
    tlsl::AttnShape s{dt, H, Dqk, Dv};
    if (!tlsl::attn_supported(s))
        return fail(TLSL_ERR_UNSUPPORTED, "sparse_attn_prefill: (dtype %s, H=%d, Dqk=%d, Dv=%d) not built "
                    "(bf16: Dqk 576, Dv 512, H<=128; f32: Dqk 80, Dv 64, H<=16)", dt_name(dt), H, Dqk, Dv);
    if (!(softmax_scale > 0.f) || !isfinite(softmax_scale))
        return fail(TLSL_ERR_SHAPE, "sparse_attn_prefill: softmax_scale must be positive and finite");
    if (!aligned16(q) || !aligned16(kv) || !aligned16(S) || !aligned16(out) || !aligned16(lse))
        return fail(TLSL_ERR_ALIGN, "sparse_attn_prefill: pointers not 16-byte aligned");
    (void)workspace;
    if (ws_bytes) *ws_bytes = 0;  // needs no workspace
    return launch_result(tlsl::launch_sparse_attn_prefill(s, q, kv, S, B, n, k, softmax_scale, out, lse, stream),
                         "sparse_attn_prefill");
}

int dense_attn_prefill(const void* q, const void* kv, int B, int n, int H, int Dqk, int Dv, float softmax_scale,
                       tlsl_dtype dt, void* out, float* lse, void* workspace, size_t* ws_bytes, hipStream_t stream) {
    if (!q || !kv || !out) return fail(TLSL_ERR_NULL, "dense_attn_prefill: NULL pointer argument");
    if (B <= 0 || n <= 0 || H <= 0) return fail(TLSL_ERR_SHAPE, "dense_attn_prefill: B, n and H must be positive");
    if ((int64_t)B * n > (int64_t)1 << 30) return fail(TLSL_ERR_SHAPE, "dense_attn_prefill: B*n too large");
    if (n > 4096) return fail(TLSL_ERR_UNSUPPORTED, "dense_attn_prefill: n=%d above the supported 4096", n);
    if (dt != TLSL_F32 && dt != TLSL_BF16) return fail(TLSL_ERR_UNSUPPORTED, "dense_attn_prefill: dtype %d not supported", dt);
    tlsl::AttnShape s{dt, H, Dqk, Dv};
    if (!tlsl::attn_supported(s))
        return fail(TLSL_ERR_UNSUPPORTED, "dense_attn_prefill: (dtype %s, H=%d, Dqk=%d, Dv=%d) not built "
                    "(bf16: Dqk 576, Dv 512, H<=128; f32: Dqk 80, Dv 64, H<=16)", dt_name(dt), H, Dqk, Dv);
    if (!(softmax_scale > 0.f) || !isfinite(softmax_scale))
        return fail(TLSL_ERR_SHAPE, "dense_attn_prefill: softmax_scale must be positive and finite");
    if (!aligned16(q) || !aligned16(kv) || !aligned16(out) || !aligned16(lse))
        return fail(TLSL_ERR_ALIGN, "dense_attn_prefill: pointers not 16-byte aligned");
    (void)workspace;
    if (ws_bytes) *ws_bytes = 0;  // needs no workspace
    // the sparse kernel with n slots per row and no index array: slot i is position i
    return launch_result(tlsl::launch_sparse_attn_prefill(s, q, kv, nullptr, B, n, n, softmax_scale, out, lse, stream),
                         "dense_attn_prefill");
}

int sparse_attn_decode(const void* q, const void* kv_cache, const int64_t* cu_seqlens, const int32_t* S, int B, int H,
                       int Dqk, int Dv, int k, float softmax_scale, tlsl_dtype dt, void* out, float* lse,
                       void* workspace, size_t* ws_bytes, hipStream_t stream) {
    if (!q || !kv_cache || !cu_seqlens || !S || !out) return fail(TLSL_ERR_NULL, "sparse_attn_decode: NULL pointer argument");
    if (B <= 0 || k <= 0 || H <= 0) return fail(TLSL_ERR_SHAPE, "sparse_attn_decode: B, H and k must be positive");
    if (k > 4096) return fail(TLSL_ERR_UNSUPPORTED, "sparse_attn_decode: k=%d above the supported 4096", k);
    if (dt != TLSL_F32 && dt != TLSL_BF16) return fail(TLSL_ERR_UNSUPPORTED, "sparse_attn_decode: dtype %d not supported", dt);
    tlsl::AttnShape s{dt, H, Dqk, Dv};
    if (!tlsl::attn_supported(s))
        return fail(TLSL_ERR_UNSUPPORTED, "sparse_attn_decode: (dtype %s, H=%d, Dqk=%d, Dv=%d) not built", dt_name(dt), H, Dqk, Dv);
    if (!(softmax_scale > 0.f) || !isfinite(softmax_scale))
        return fail(TLSL_ERR_SHAPE, "sparse_attn_decode: softmax_scale must be positive and finite");
    if (!aligned16(q) || !aligned16(kv_cache) || !aligned16(S) || !aligned16(out) || !aligned16(lse) || !aligned16(cu_seqlens))
        return fail(TLSL_ERR_ALIGN, "sparse_attn_decode: pointers not 16-byte aligned");
    const size_t need = tlsl::attn_decode_ws_bytes(s, B, k);
    const int rc = workspace_protocol(workspace, ws_bytes, need);
    if (rc) return rc > 0 ? ok() : rc;
    return launch_result(tlsl::launch_sparse_attn_decode(s, q, kv_cache, cu_seqlens, S, B, k, softmax_scale, out, lse,
                                                         workspace, stream),
                         "sparse_attn_decode");
}

}  // extern "C"
