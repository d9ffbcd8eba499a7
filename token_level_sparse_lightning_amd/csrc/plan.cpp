// plan.cpp -- host-side planning shared by the C ABI and the launchers: which
// shapes are built, workspace sizes and layouts, split counts.  Plain C++ with
// no device code, so the argument-checking layer can also be built and tested
// on a machine without a GPU (and under the address / undefined-behaviour
// sanitizers).
#include <algorithm>

#include "tlsl_internal.h"

namespace tlsl {

namespace {
constexpr int kF32 = 0, kBF16 = 1, kFP8 = 2;
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
}  // namespace

// ---- indexer ---------------------------------------------------------------
bool indexer_supported(const IndexerShape& s) {
    if (s.HI < 1 || s.HI > 64) return false;
    if (s.dt == kFP8) return s.DI == 128;
    if (s.dt == kBF16) return s.DI == 32 || s.DI == 64 || s.DI == 128;
    if (s.dt == kF32) return s.DI == 32 || s.DI == 64;
    return false;
}

// Candidate buffers of 2k + 256 entries (rounded to 256) per query row, the
// threshold sample stride, and the fallback lists and scratch rows.
PrefillPlan plan_prefill(const IndexerShape& s, int B, int n, int k) {
    PrefillPlan p{};
    p.cap = (int)((2 * (size_t)k + 256 + 255) / 256 * 256);
    p.stride = std::max(1, k / 64);  // ~64 sample keys expected inside the top-k
    p.fb_blocks = 128;
    const size_t rows = (size_t)B * n;
    size_t off = 0;
    p.off_buf = off;
    off = align256(off + rows * p.cap * 8);  // (score bits, position) pairs
    p.off_cnt = off;
    off = align256(off + rows * sizeof(int));
    p.off_fbcount = off;
    off = align256(off + sizeof(int));
    p.off_fblist = off;
    off = align256(off + rows * sizeof(int));
    p.off_fbscratch = off;
    off = align256(off + (size_t)p.fb_blocks * n * sizeof(float));
    p.ws_bytes = off;
    (void)s;
    return p;
}

// ---- row top-k ---------------------------------------------------------------
TopkLayout topk_layout(int R, int k) {
    TopkLayout t{};
    t.cap = (int)((2 * (size_t)k + 256 + 255) / 256 * 256);
    t.off_theta = 0;
    t.off_cnt = align256((size_t)R * sizeof(float));
    t.off_buf = t.off_cnt + align256((size_t)R * kTopkCntStride * sizeof(int));
    t.bytes = t.off_buf + align256((size_t)R * t.cap * 8);
    return t;
}

size_t topk_ws_bytes(int R, int k, int) { return topk_layout(R, k).bytes; }

// ---- selection-quality diagnostics ----------------------------------------------
// the teacher's top-m (int32 per slot), then topk_select's own workspace
size_t selection_quality_ws_bytes(int R, int m, int max_len) {
    return align256((size_t)R * m * sizeof(int32_t)) + topk_ws_bytes(R, m, max_len);
}
// the top-(k+1) positions and scores, then topk_select's own workspace
size_t cutoff_margin_ws_bytes(int R, int k, int max_len) {
    return 2 * align256((size_t)R * (k + 1) * sizeof(int32_t)) + topk_ws_bytes(R, k + 1, max_len);
}

// ---- sparse attention ---------------------------------------------------------
bool attn_supported(const AttnShape& s) {
    if (s.dt == kBF16) return s.Dqk == 576 && s.Dv == 512 && s.H >= 1 && s.H <= 128;
    if (s.dt == kF32) return s.Dqk == 80 && s.Dv == 64 && s.H >= 1 && s.H <= 16;
    return false;
}

// About one workgroup per compute unit over the batch's rows and head groups,
// at least 128 slots per split.
int attn_decode_splits(const AttnShape& s, int B, int k) {
    const int hpw = s.dt == kBF16 ? 64 : 16;
    const int hg = (s.H + hpw - 1) / hpw;
    const int cus = device_cu_count();
    int ns = (cus + B * hg - 1) / (B * hg);
    const int maxs = (k + 127) / 128;
    if (ns > maxs) ns = maxs;
    return ns < 1 ? 1 : ns;
}

size_t attn_decode_ws_bytes(const AttnShape& s, int B, int k) {
    const int ns = attn_decode_splits(s, B, k);
    if (ns == 1) return 256;  // never empty, so that a NULL workspace always means "size query"
    const size_t parts = (size_t)B * ns * s.H;
    return parts * s.Dv * sizeof(float) + align256(parts * 2 * sizeof(float)) + 256;
}

}  // namespace tlsl
