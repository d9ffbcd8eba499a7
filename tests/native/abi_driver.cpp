// abi_driver.cpp -- drives every entry point of include/tlsl.h through its
// validation and workspace-query paths and one accepted call each, against the
// launcher stand-ins of abi_stubs.cpp.  Built and run under ASan + UBSan by
// tests/test_sanitizers.py; prints "abi driver ok" and exits 0 when every
// return code is the documented one.  TEST INFRASTRUCTURE ONLY.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/tlsl.h"

extern int g_launches;
namespace tlsl {
extern int g_debug_checks;
}
static int g_fail = 0;
static float sc0() { return 0.05f; }

#define EXPECT(call, code)                                                                       \
    do {                                                                                         \
        const int rc_ = (call);                                                                  \
        if (rc_ != (code)) {                                                                     \
            fprintf(stderr, "line %d: %s returned %d, expected %d (%s)\n", __LINE__, #call, rc_, \
                    (int)(code), tlsl_last_error());                                             \
            ++g_fail;                                                                            \
        }                                                                                        \
    } while (0)

int main() {
    // dummy device pointers: 16-byte aligned, never dereferenced by the host layer
    void* P = reinterpret_cast<void*>(uintptr_t(0x10000));
    float* F = static_cast<float*>(P);
    int32_t* I32 = static_cast<int32_t*>(P);
    int64_t* I64 = static_cast<int64_t*>(P);
    void* odd = reinterpret_cast<void*>(uintptr_t(0x10004));
    size_t ws = 0, need = 0;

    // ---- index_prefill
    EXPECT(index_prefill(P, F, P, F, F, 1, 100, 64, 128, 16, TLSL_FP8_E4M3, I32, F, nullptr, &need, nullptr), TLSL_OK);
    if (need == 0) { fprintf(stderr, "index_prefill: zero workspace\n"); ++g_fail; }
    ws = need - 1;
    EXPECT(index_prefill(P, F, P, F, F, 1, 100, 64, 128, 16, TLSL_FP8_E4M3, I32, F, P, &ws, nullptr), TLSL_ERR_WORKSPACE);
    ws = need;
    EXPECT(index_prefill(P, F, P, F, F, 1, 100, 64, 128, 16, TLSL_FP8_E4M3, I32, F, P, &ws, nullptr), TLSL_OK);
    EXPECT(index_prefill(P, F, P, F, F, 1, 100, 64, 128, 16, TLSL_FP8_E4M3, I32, F, P, nullptr, nullptr), TLSL_ERR_NULL);
    EXPECT(index_prefill(nullptr, F, P, F, F, 1, 100, 64, 128, 16, TLSL_FP8_E4M3, I32, F, P, &ws, nullptr), TLSL_ERR_NULL);
    EXPECT(index_prefill(P, nullptr, P, F, F, 1, 100, 64, 128, 16, TLSL_FP8_E4M3, I32, F, P, &ws, nullptr), TLSL_ERR_NULL);
    EXPECT(index_prefill(P, F, P, F, F, 1, 100, 64, 128, 16, TLSL_BF16, I32, F, P, &ws, nullptr), TLSL_ERR_SHAPE);
    EXPECT(index_prefill(P, nullptr, P, nullptr, F, 0, 100, 64, 128, 16, TLSL_BF16, I32, F, P, &ws, nullptr), TLSL_ERR_SHAPE);
    EXPECT(index_prefill(P, nullptr, P, nullptr, F, 1, 100, 64, 128, 0, TLSL_BF16, I32, F, P, &ws, nullptr), TLSL_ERR_SHAPE);
    EXPECT(index_prefill(P, nullptr, P, nullptr, F, 1, 100, 64, 128, 4097, TLSL_BF16, I32, F, P, &ws, nullptr), TLSL_ERR_UNSUPPORTED);
    EXPECT(index_prefill(P, nullptr, P, nullptr, F, 1, 100, 65, 128, 16, TLSL_BF16, I32, F, P, &ws, nullptr), TLSL_ERR_UNSUPPORTED);
    EXPECT(index_prefill(P, nullptr, P, nullptr, F, 1, 100, 64, 96, 16, TLSL_BF16, I32, F, P, &ws, nullptr), TLSL_ERR_UNSUPPORTED);
    EXPECT(index_prefill(P, nullptr, P, nullptr, F, 1, 100, 64, 128, 16, (tlsl_dtype)7, I32, F, P, &ws, nullptr), TLSL_ERR_UNSUPPORTED);
    EXPECT(index_prefill(odd, nullptr, P, nullptr, F, 1, 100, 64, 128, 16, TLSL_BF16, I32, F, P, &ws, nullptr), TLSL_ERR_ALIGN);
    EXPECT(index_prefill(P, nullptr, P, nullptr, F, 1 << 16, 1 << 15, 64, 128, 16, TLSL_BF16, I32, F, P, &ws, nullptr), TLSL_ERR_SHAPE);

    // ---- index_prefill_rerank
    EXPECT(index_prefill_rerank(P, F, P, F, P, P, F, 1, 100, 64, 128, 16, 64, I32, F, nullptr, nullptr, &need, nullptr),
           TLSL_OK);
    ws = need;
    EXPECT(index_prefill_rerank(P, F, P, F, P, P, F, 1, 100, 64, 128, 16, 64, I32, F, nullptr, P, &ws, nullptr), TLSL_OK);
    EXPECT(index_prefill_rerank(P, F, P, F, P, P, F, 1, 100, 64, 128, 65, 64, I32, F, nullptr, P, &ws, nullptr),
           TLSL_ERR_SHAPE);
    EXPECT(index_prefill_rerank(P, F, P, F, P, P, F, 1, 100, 64, 64, 16, 64, I32, F, nullptr, P, &ws, nullptr),
           TLSL_ERR_UNSUPPORTED);
    EXPECT(index_prefill_rerank(P, nullptr, P, F, P, P, F, 1, 100, 64, 128, 16, 64, I32, F, nullptr, P, &ws, nullptr),
           TLSL_ERR_NULL);

    // ---- index_decode
    EXPECT(index_decode(P, F, P, F, F, I64, 4, 64, 128, 1000, TLSL_FP8_E4M3, F, nullptr, &ws, nullptr), TLSL_OK);
    if (ws != 0) { fprintf(stderr, "index_decode: nonzero workspace\n"); ++g_fail; }
    EXPECT(index_decode(P, F, P, F, F, nullptr, 4, 64, 128, 1000, TLSL_FP8_E4M3, F, nullptr, &ws, nullptr), TLSL_ERR_NULL);
    EXPECT(index_decode(P, F, P, F, F, I64, 0, 64, 128, 1000, TLSL_FP8_E4M3, F, nullptr, &ws, nullptr), TLSL_ERR_SHAPE);
    EXPECT(index_decode(P, F, P, F, F, I64, 4, 64, 128, 0, TLSL_FP8_E4M3, F, nullptr, &ws, nullptr), TLSL_ERR_SHAPE);
    EXPECT(index_decode(P, F, P, F, F, I64, 4, 64, 128, 1000, TLSL_FP8_E4M3, static_cast<float*>(odd), nullptr, &ws, nullptr), TLSL_ERR_ALIGN);

    // ---- topk_select
    EXPECT(topk_select(F, I64, I32, 64, 2048, 131072, I32, F, nullptr, &need, nullptr), TLSL_OK);
    ws = need;
    EXPECT(topk_select(F, I64, I32, 64, 2048, 131072, I32, F, P, &ws, nullptr), TLSL_OK);
    ws = need / 2;
    EXPECT(topk_select(F, I64, I32, 64, 2048, 131072, I32, F, P, &ws, nullptr), TLSL_ERR_WORKSPACE);
    EXPECT(topk_select(F, I64, I32, 0, 2048, 131072, I32, F, nullptr, &need, nullptr), TLSL_ERR_SHAPE);
    EXPECT(topk_select(F, I64, I32, 64, 5000, 131072, I32, F, nullptr, &need, nullptr), TLSL_ERR_UNSUPPORTED);
    EXPECT(topk_select(F, I64, I32, 64, 2048, -1, I32, F, nullptr, &need, nullptr), TLSL_ERR_SHAPE);
    EXPECT(topk_select(static_cast<float*>(reinterpret_cast<void*>(uintptr_t(0x10002))), I64, I32, 64, 2048, 10, I32,
                       F, nullptr, &need, nullptr), TLSL_ERR_ALIGN);

    // ---- topk_select_noalloc: the same checks, a fixed scratch instead of a workspace
    EXPECT(topk_select_noalloc(F, I64, I32, 64, 2048, 131072, I32, F, nullptr), TLSL_OK);
    EXPECT(topk_select_noalloc(F, I64, I32, 481, 2048, 131072, I32, F, nullptr), TLSL_ERR_WORKSPACE);
    EXPECT(topk_select_noalloc(F, I64, I32, 480, 2048, 131072, I32, F, nullptr), TLSL_OK);
    EXPECT(topk_select_noalloc(nullptr, I64, I32, 64, 2048, 131072, I32, F, nullptr), TLSL_ERR_NULL);
    EXPECT(topk_select_noalloc(F, I64, I32, 64, 4097, 131072, I32, F, nullptr), TLSL_ERR_UNSUPPORTED);

    // ---- indexer_loss_grad
    EXPECT(indexer_loss_grad(P, P, F, I32, F, 1, 100, 64, 128, 2048, TLSL_BF16, F, F, F, F, nullptr), TLSL_OK);
    EXPECT(indexer_loss_grad(P, P, F, I32, nullptr, 1, 100, 64, 128, 2048, TLSL_BF16, F, F, F, F, nullptr), TLSL_ERR_NULL);
    EXPECT(indexer_loss_grad(P, P, F, I32, F, 1, 100, 64, 128, 2048, TLSL_FP8_E4M3, F, F, F, F, nullptr), TLSL_ERR_UNSUPPORTED);
    EXPECT(indexer_loss_grad(P, P, F, I32, F, 1, 100, 64, 64, 2048, TLSL_BF16, F, F, F, F, nullptr), TLSL_ERR_UNSUPPORTED);
    EXPECT(indexer_loss_grad(P, P, F, I32, F, 1, 0, 64, 128, 2048, TLSL_BF16, F, F, F, F, nullptr), TLSL_ERR_SHAPE);
    EXPECT(indexer_loss_grad(P, odd, F, I32, F, 1, 100, 64, 128, 2048, TLSL_BF16, F, F, F, F, nullptr), TLSL_ERR_ALIGN);

    // ---- dsa_prefill: dense path (n <= k: fill S + attention), sparse path (prefill + attention)
    EXPECT(dsa_prefill(P, F, P, F, F, 64, 128, TLSL_FP8_E4M3, P, P, 128, 576, 512, sc0(), TLSL_BF16, 1, 2048, 2048, I32,
                       P, F, nullptr, &need, nullptr), TLSL_OK);
    ws = need;
    EXPECT(dsa_prefill(P, F, P, F, F, 64, 128, TLSL_FP8_E4M3, P, P, 128, 576, 512, sc0(), TLSL_BF16, 1, 2048, 2048, I32,
                       P, F, P, &ws, nullptr), TLSL_OK);
    EXPECT(dsa_prefill(P, F, P, F, F, 64, 128, TLSL_FP8_E4M3, P, P, 128, 576, 512, sc0(), TLSL_BF16, 1, 4096, 2048,
                       nullptr, P, F, nullptr, &need, nullptr), TLSL_OK);
    ws = need;
    EXPECT(dsa_prefill(P, F, P, F, F, 64, 128, TLSL_FP8_E4M3, P, P, 128, 576, 512, sc0(), TLSL_BF16, 1, 4096, 2048,
                       nullptr, P, F, P, &ws, nullptr), TLSL_OK);
    EXPECT(dsa_prefill(P, F, P, F, F, 64, 128, TLSL_FP8_E4M3, P, P, 127, 576, 500, sc0(), TLSL_BF16, 1, 4096, 2048,
                       nullptr, P, F, P, &ws, nullptr), TLSL_ERR_UNSUPPORTED);
    EXPECT(dsa_prefill(P, F, P, F, F, 64, 128, TLSL_FP8_E4M3, nullptr, P, 128, 576, 512, sc0(), TLSL_BF16, 1, 4096,
                       2048, nullptr, P, F, P, &ws, nullptr), TLSL_ERR_NULL);

    // ---- selection_quality / cutoff_margin
    EXPECT(selection_quality(F, I64, I32, 64, I32, 2048, 64, 131072, F, F, nullptr, &need, nullptr), TLSL_OK);
    ws = need;
    EXPECT(selection_quality(F, I64, I32, 64, I32, 2048, 64, 131072, F, F, P, &ws, nullptr), TLSL_OK);
    EXPECT(selection_quality(F, I64, I32, 64, nullptr, 2048, 64, 131072, F, F, P, &ws, nullptr), TLSL_ERR_NULL);
    EXPECT(selection_quality(F, I64, I32, 64, I32, 2048, 5000, 131072, F, F, P, &ws, nullptr), TLSL_ERR_UNSUPPORTED);
    EXPECT(cutoff_margin(F, I64, I32, 64, 2048, 131072, F, nullptr, &need, nullptr), TLSL_OK);
    ws = need;
    EXPECT(cutoff_margin(F, I64, I32, 64, 2048, 131072, F, P, &ws, nullptr), TLSL_OK);
    EXPECT(cutoff_margin(F, I64, I32, 64, 4096, 131072, F, P, &ws, nullptr), TLSL_ERR_UNSUPPORTED);

    // ---- attention
    const float sc = 0.05f;
    EXPECT(sparse_attn_prefill(P, P, I32, 1, 100, 128, 576, 512, 2048, sc, TLSL_BF16, P, F, nullptr, &ws, nullptr), TLSL_OK);
    EXPECT(sparse_attn_prefill(P, P, I32, 1, 100, 129, 576, 512, 2048, sc, TLSL_BF16, P, F, nullptr, &ws, nullptr), TLSL_ERR_UNSUPPORTED);
    EXPECT(sparse_attn_prefill(P, P, I32, 1, 100, 128, 576, 512, 2048, -1.f, TLSL_BF16, P, F, nullptr, &ws, nullptr), TLSL_ERR_SHAPE);
    EXPECT(sparse_attn_prefill(P, P, I32, 1, 100, 128, 576, 512, 2048, INFINITY, TLSL_BF16, P, F, nullptr, &ws, nullptr), TLSL_ERR_SHAPE);
    EXPECT(sparse_attn_prefill(P, P, I32, 1, 100, 128, 576, 512, 2048, NAN, TLSL_BF16, P, F, nullptr, &ws, nullptr), TLSL_ERR_SHAPE);
    EXPECT(sparse_attn_prefill(P, P, I32, 1, 100, 4, 80, 64, 64, sc, TLSL_FP8_E4M3, P, F, nullptr, &ws, nullptr), TLSL_ERR_UNSUPPORTED);
    EXPECT(dense_attn_prefill(P, P, 1, 4096, 128, 576, 512, sc, TLSL_BF16, P, F, nullptr, &ws, nullptr), TLSL_OK);
    EXPECT(dense_attn_prefill(P, P, 1, 4097, 128, 576, 512, sc, TLSL_BF16, P, F, nullptr, &ws, nullptr), TLSL_ERR_UNSUPPORTED);
    EXPECT(sparse_attn_decode(P, P, I64, I32, 64, 128, 576, 512, 2048, sc, TLSL_BF16, P, F, nullptr, &need, nullptr), TLSL_OK);
    ws = need;
    EXPECT(sparse_attn_decode(P, P, I64, I32, 64, 128, 576, 512, 2048, sc, TLSL_BF16, P, F, P, &ws, nullptr), TLSL_ERR_HIP);
    if (strstr(tlsl_last_error(), "stubbed HIP error") == nullptr) {
        fprintf(stderr, "launch error message not reported: %s\n", tlsl_last_error());
        ++g_fail;
    }
    EXPECT(sparse_attn_decode(P, P, I64, I32, 64, 128, 576, 512, 2048, sc, TLSL_BF16, P, F, nullptr, nullptr, nullptr), TLSL_ERR_NULL);
    if (strlen(tlsl_version()) == 0) ++g_fail;

    // accepted calls: index_prefill, index_prefill_rerank, index_decode, topk_select, topk_select_noalloc (2),
    // indexer_loss_grad, dsa_prefill dense (fill + attention) and sparse (index +
    // attention), selection_quality, cutoff_margin, sparse_attn_prefill, dense_attn_prefill, sparse_attn_decode (the
    // last one's stand-in fails on purpose)
    if (g_launches != 16) {
        fprintf(stderr, "expected 16 launches, saw %d\n", g_launches);
        ++g_fail;
    }
    // the debug switch: off by default; on, the calls with device-side
    // metadata run their device check before the launch
    if (tlsl::g_debug_checks != 0) { fprintf(stderr, "device checks ran with the debug switch off\n"); ++g_fail; }
    if (tlsl_set_debug(1) != 0) { fprintf(stderr, "debug switch on by default\n"); ++g_fail; }
    size_t ws2 = 0;
    EXPECT(index_decode(P, F, P, F, F, I64, 4, 64, 128, 1000, TLSL_FP8_E4M3, F, nullptr, &ws2, nullptr), TLSL_OK);
    EXPECT(topk_select(F, I64, I32, 64, 2048, 131072, I32, F, nullptr, &need, nullptr), TLSL_OK);  // size query only
    ws2 = need;
    EXPECT(topk_select(F, I64, I32, 64, 2048, 131072, I32, F, P, &ws2, nullptr), TLSL_OK);
    if (tlsl::g_debug_checks != 2) {
        fprintf(stderr, "expected 2 device checks with the debug switch on, saw %d\n", tlsl::g_debug_checks);
        ++g_fail;
    }
    if (tlsl_set_debug(0) != 1) { fprintf(stderr, "debug switch did not report its previous state\n"); ++g_fail; }
    if (g_fail) return 1;
    printf("abi driver ok\n");
    return 0;
}
