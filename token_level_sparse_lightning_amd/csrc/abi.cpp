// abi.cpp -- the extern "C" entry points declared in include/tlsl.h: argument
// validation (all of it on the host, before anything is launched), workspace
// sizing and dispatch to the gfx950 kernels.  No exception crosses the ABI.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

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

int check_topk(const float* scores, const int64_t* row_start, const int32_t* row_len, int R, int k, int max_len,
               const int32_t* S, const float* S_score, const char* fn) {
    if (!scores || !row_start || !row_len || !S) return fail(TLSL_ERR_NULL, "%s: NULL pointer argument", fn);
    if (R <= 0) return fail(TLSL_ERR_SHAPE, "%s: R=%d must be positive", fn, R);
    if (k <= 0) return fail(TLSL_ERR_SHAPE, "%s: k=%d must be positive", fn, k);
    if (k > 4096) return fail(TLSL_ERR_UNSUPPORTED, "%s: k=%d above the supported 4096", fn, k);
    if (max_len < 0) return fail(TLSL_ERR_SHAPE, "%s: max_len=%d must be >= 0", fn, max_len);
    if (!aligned16(S) || !aligned16(S_score) || !aligned16(row_start) || !aligned16(row_len))
        return fail(TLSL_ERR_ALIGN, "%s: pointers not 16-byte aligned", fn);
    if ((reinterpret_cast<uintptr_t>(scores) & 3u) != 0) return fail(TLSL_ERR_ALIGN, "%s: scores not 4-byte aligned", fn);
    return 0;
}

// debug switch: -1 until the environment has been read
std::atomic<int> g_debug{-1};

int debug_state() {
    int v = g_debug.load(std::memory_order_relaxed);
    if (v < 0) {
        const char* e = getenv("TLSL_DEBUG");
        const int from_env = (e && *e && strcmp(e, "0") != 0) ? 1 : 0;
        int expected = -1;
        g_debug.compare_exchange_strong(expected, from_env);
        v = g_debug.load(std::memory_order_relaxed);
    }
    return v;
}

}  // namespace

bool tlsl::debug_enabled() { return debug_state() == 1; }

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

int tlsl_set_debug(int on) {
    const int prev = debug_state();
    g_debug.store(on ? 1 : 0, std::memory_order_relaxed);
    return prev;
}

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

int index_prefill_rerank(const void* qI8, const float* q_scale, const void* kI8, const float* k_scale, const void* qI,
                         const void* kI, const float* wI, int B, int n, int HI, int dI, int k, int k_coarse, int32_t* S,
                         float* S_score, int32_t* C, void* workspace, size_t* ws_bytes, hipStream_t stream) {
    int rc = check_indexer(TLSL_FP8_E4M3, qI8, q_scale, kI8, k_scale, wI, HI, dI, "index_prefill_rerank");
    if (rc) return rc;
    if (!qI || !kI || !S) return fail(TLSL_ERR_NULL, "index_prefill_rerank: qI, kI and S must be non-NULL");
    if (dI != 128) return fail(TLSL_ERR_UNSUPPORTED, "index_prefill_rerank: dI=%d not built (128)", dI);
    if (B <= 0 || n <= 0) return fail(TLSL_ERR_SHAPE, "index_prefill_rerank: B=%d and n=%d must be positive", B, n);
    if (k <= 0 || k_coarse < k) return fail(TLSL_ERR_SHAPE, "index_prefill_rerank: need 1 <= k <= k_coarse");
    if (k_coarse > 4096) return fail(TLSL_ERR_UNSUPPORTED, "index_prefill_rerank: k_coarse=%d above the supported 4096",
                                     k_coarse);
    if ((int64_t)B * n > (int64_t)1 << 30) return fail(TLSL_ERR_SHAPE, "index_prefill_rerank: B*n too large");
    if (!aligned16(qI) || !aligned16(kI) || !aligned16(S) || !aligned16(S_score) || !aligned16(C))
        return fail(TLSL_ERR_ALIGN, "index_prefill_rerank: pointers not 16-byte aligned");
    const tlsl::IndexerShape coarse{TLSL_FP8_E4M3, HI, dI};
    const tlsl::PrefillPlan plan = tlsl::plan_prefill(coarse, B, n, k_coarse);
    const size_t c_bytes = C ? 0 : (((size_t)B * n * k_coarse * sizeof(int32_t) + 255) & ~(size_t)255);
    rc = workspace_protocol(workspace, ws_bytes, plan.ws_bytes + c_bytes);
    if (rc) return rc > 0 ? ok() : rc;
    int32_t* Cx = C ? C : reinterpret_cast<int32_t*>(static_cast<unsigned char*>(workspace) + plan.ws_bytes);
    return launch_result(tlsl::launch_index_prefill_rerank(coarse, qI8, q_scale, kI8, k_scale, qI, kI, wI, B, n, k,
                                                           k_coarse, S, S_score, Cx, workspace, plan, stream),
                         "index_prefill_rerank");
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
    if (tlsl::debug_enabled() && (rc = tlsl::debug_check_seqlens(cu_seqlens, B, true, stream, "index_decode"))) return rc;
    return launch_result(tlsl::launch_index_decode(s, qI, q_scale, kI_cache, k_scale, wI, cu_seqlens, B, max_len,
                                                   scores, stream),
                         "index_decode");
}

int topk_select(const float* scores, const int64_t* row_start, const int32_t* row_len, int R, int k, int max_len,
                int32_t* S, float* S_score, void* workspace, size_t* ws_bytes, hipStream_t stream) {
    int rc = check_topk(scores, row_start, row_len, R, k, max_len, S, S_score, "topk_select");
    if (rc) return rc;
    rc = workspace_protocol(workspace, ws_bytes, tlsl::topk_ws_bytes(R, k, max_len));
    if (rc) return rc > 0 ? ok() : rc;
    if (tlsl::debug_enabled() && (rc = tlsl::debug_check_rows(row_start, row_len, R, stream, "topk_select"))) return rc;
    return launch_result(tlsl::launch_topk_select(scores, row_start, row_len, R, k, max_len, S, S_score, workspace,
                                                  stream),
                         "topk_select");
}

int topk_select_noalloc(const float* scores, const int64_t* row_start, const int32_t* row_len, int R, int k,
                        int max_len, int32_t* S, float* S_score, hipStream_t stream) {
    int rc = check_topk(scores, row_start, row_len, R, k, max_len, S, S_score, "topk_select_noalloc");
    if (rc) return rc;
    const size_t need = tlsl::topk_ws_bytes(R, k, max_len);
    if (need > (size_t)TLSL_NOALLOC_SCRATCH_BYTES)
        return fail(TLSL_ERR_WORKSPACE,
                    "topk_select_noalloc: R=%d rows at k=%d need %zu bytes of scratch, above its fixed %zu "
                    "(call topk_select with a workspace instead)",
                    R, k, need, (size_t)TLSL_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    const hipError_t e = tlsl::topk_noalloc_scratch(&ws);
    if (e != hipSuccess)
        return fail(TLSL_ERR_HIP, "topk_select_noalloc: device address of the scratch array: %s", hipGetErrorString(e));
    if (tlsl::debug_enabled() &&
        (rc = tlsl::debug_check_rows(row_start, row_len, R, stream, "topk_select_noalloc")))
        return rc;
    return launch_result(tlsl::launch_topk_select(scores, row_start, row_len, R, k, max_len, S, S_score, ws, stream),
                         "topk_select_noalloc");
}

int indexer_loss_grad(const void* qI, const void* kI, const float* wI, const int32_t* S, const float* p, int B, int n,
                      int HI, int dI, int k, tlsl_dtype dt, float* loss, float* dq, float* dk, float* dw,
                      hipStream_t stream) {
    if (!qI || !kI || !wI || !S || !p || !loss || !dq || !dk || !dw)
        return fail(TLSL_ERR_NULL, "indexer_loss_grad: NULL pointer argument");
    if (B <= 0 || n <= 0 || HI <= 0 || dI <= 0 || k <= 0)
        return fail(TLSL_ERR_SHAPE, "indexer_loss_grad: B, n, HI, dI and k must be positive");
    if ((int64_t)B * n > (int64_t)1 << 30) return fail(TLSL_ERR_SHAPE, "indexer_loss_grad: B*n too large");
    if (dt != TLSL_BF16 || dI != 128 || HI > 64 || k > 4096)
        return fail(TLSL_ERR_UNSUPPORTED, "indexer_loss_grad: (dtype %s, HI=%d, dI=%d, k=%d) not built "
                    "(bf16, dI 128, HI 1..64, k 1..4096)", dt_name(dt), HI, dI, k);
    if (n >= (1 << 22))  // one sequence's dK rows are addressed with 32-bit byte offsets below 2^31
        return fail(TLSL_ERR_UNSUPPORTED, "indexer_loss_grad: n=%d above the supported 4194303", n);
    if (!aligned16(qI) || !aligned16(kI) || !aligned16(wI) || !aligned16(S) || !aligned16(p) || !aligned16(loss) ||
        !aligned16(dq) || !aligned16(dk) || !aligned16(dw))
        return fail(TLSL_ERR_ALIGN, "indexer_loss_grad: pointers not 16-byte aligned");
    return launch_result(tlsl::launch_indexer_kl(qI, kI, wI, S, p, B, n, HI, k, loss, dq, dk, dw, stream),
                         "indexer_loss_grad");
}

int selection_quality(const float* teacher, const int64_t* row_start, const int32_t* row_len, int R, const int32_t* S,
                      int k, int m, int max_len, float* recall, float* mass, void* workspace, size_t* ws_bytes,
                      hipStream_t stream) {
    if (!S || !recall || !mass) return fail(TLSL_ERR_NULL, "selection_quality: NULL pointer argument");
    if (k <= 0) return fail(TLSL_ERR_SHAPE, "selection_quality: k=%d must be positive", k);
    int rc = check_topk(teacher, row_start, row_len, R, m, max_len, S, nullptr, "selection_quality");
    if (rc) return rc;
    if (!aligned16(recall) || !aligned16(mass)) return fail(TLSL_ERR_ALIGN, "selection_quality: pointers not 16-byte aligned");
    rc = workspace_protocol(workspace, ws_bytes, tlsl::selection_quality_ws_bytes(R, m, max_len));
    if (rc) return rc > 0 ? ok() : rc;
    if (tlsl::debug_enabled() && (rc = tlsl::debug_check_rows(row_start, row_len, R, stream, "selection_quality")))
        return rc;
    return launch_result(tlsl::launch_selection_quality(teacher, row_start, row_len, R, S, k, m, max_len, recall, mass,
                                                        workspace, stream),
                         "selection_quality");
}

int cutoff_margin(const float* scores, const int64_t* row_start, const int32_t* row_len, int R, int k, int max_len,
                  float* margin, void* workspace, size_t* ws_bytes, hipStream_t stream) {
    if (!margin) return fail(TLSL_ERR_NULL, "cutoff_margin: margin is NULL");
    if (k >= 4096) return fail(TLSL_ERR_UNSUPPORTED, "cutoff_margin: k=%d above the supported 4095", k);
    int32_t dummy_s alignas(16) = 0;
    int rc = check_topk(scores, row_start, row_len, R, k, max_len, &dummy_s, nullptr, "cutoff_margin");
    if (rc) return rc;
    if (!aligned16(margin)) return fail(TLSL_ERR_ALIGN, "cutoff_margin: margin not 16-byte aligned");
    rc = workspace_protocol(workspace, ws_bytes, tlsl::cutoff_margin_ws_bytes(R, k, max_len));
    if (rc) return rc > 0 ? ok() : rc;
    if (tlsl::debug_enabled() && (rc = tlsl::debug_check_rows(row_start, row_len, R, stream, "cutoff_margin")))
        return rc;
    return launch_result(tlsl::launch_cutoff_margin(scores, row_start, row_len, R, k, max_len, margin, workspace, stream),
                         "cutoff_margin");
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

int dsa_prefill(const void* qI, const float* q_scale, const void* kI, const float* k_scale, const float* wI, int HI,
                int dI, tlsl_dtype idx_dt, const void* q, const void* kv, int H, int Dqk, int Dv, float softmax_scale,
                tlsl_dtype attn_dt, int B, int n, int k, int32_t* S, void* out, float* lse, void* workspace,
                size_t* ws_bytes, hipStream_t stream) {
    int rc = check_indexer(idx_dt, qI, q_scale, kI, k_scale, wI, HI, dI, "dsa_prefill");
    if (rc) return rc;
    if (!q || !kv || !out) return fail(TLSL_ERR_NULL, "dsa_prefill: q, kv and out must be non-NULL");
    if (B <= 0 || n <= 0 || k <= 0 || H <= 0) return fail(TLSL_ERR_SHAPE, "dsa_prefill: B, n, k and H must be positive");
    if ((int64_t)B * n > (int64_t)1 << 30) return fail(TLSL_ERR_SHAPE, "dsa_prefill: B*n too large");
    if (k > 4096) return fail(TLSL_ERR_UNSUPPORTED, "dsa_prefill: k=%d above the supported 4096", k);
    if (attn_dt != TLSL_F32 && attn_dt != TLSL_BF16)
        return fail(TLSL_ERR_UNSUPPORTED, "dsa_prefill: attention dtype %d not supported", attn_dt);
    tlsl::AttnShape as{attn_dt, H, Dqk, Dv};
    if (!tlsl::attn_supported(as))
        return fail(TLSL_ERR_UNSUPPORTED, "dsa_prefill: attention (dtype %s, H=%d, Dqk=%d, Dv=%d) not built",
                    dt_name(attn_dt), H, Dqk, Dv);
    if (!(softmax_scale > 0.f) || !isfinite(softmax_scale))
        return fail(TLSL_ERR_SHAPE, "dsa_prefill: softmax_scale must be positive and finite");
    if (!aligned16(q) || !aligned16(kv) || !aligned16(out) || !aligned16(lse) || !aligned16(S))
        return fail(TLSL_ERR_ALIGN, "dsa_prefill: pointers not 16-byte aligned");
    // every row keeps all of its history when n <= k: the dense path gives the
    // same result without the indexer; otherwise indexer, top-k and gather
    const bool dense = n <= k;
    const tlsl::IndexerShape is{idx_dt, HI, dI};
    const tlsl::PrefillPlan plan = tlsl::plan_prefill(is, B, n, k);
    const size_t s_bytes = S ? 0 : (((size_t)B * n * k * sizeof(int32_t) + 255) & ~(size_t)255);
    const size_t need = dense ? 256 : plan.ws_bytes + s_bytes;  // never 0: NULL always means "size query"
    rc = workspace_protocol(workspace, ws_bytes, need);
    if (rc) return rc > 0 ? ok() : rc;
    if (dense) {
        if (S) {
            const hipError_t e = tlsl::launch_fill_all_history(S, B, n, k, stream);
            if (e != hipSuccess) return launch_result(e, "dsa_prefill");
        }
        return launch_result(tlsl::launch_sparse_attn_prefill(as, q, kv, nullptr, B, n, n, softmax_scale, out, lse,
                                                              stream),
                             "dsa_prefill");
    }
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    int32_t* Sx = S ? S : reinterpret_cast<int32_t*>(ws + plan.ws_bytes);
    const hipError_t e = tlsl::launch_index_prefill(is, qI, q_scale, kI, k_scale, wI, B, n, k, Sx, nullptr, ws, plan,
                                                    stream);
    if (e != hipSuccess) return launch_result(e, "dsa_prefill");
    return launch_result(tlsl::launch_sparse_attn_prefill(as, q, kv, Sx, B, n, k, softmax_scale, out, lse, stream),
                         "dsa_prefill");
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
    int rc = workspace_protocol(workspace, ws_bytes, need);
    if (rc) return rc > 0 ? ok() : rc;
    if (tlsl::debug_enabled() && (rc = tlsl::debug_check_seqlens(cu_seqlens, B, false, stream, "sparse_attn_decode")))
        return rc;
    return launch_result(tlsl::launch_sparse_attn_decode(s, q, kv_cache, cu_seqlens, S, B, k, softmax_scale, out, lse,
                                                         workspace, stream),
                         "sparse_attn_decode");
}

}  // extern "C"
