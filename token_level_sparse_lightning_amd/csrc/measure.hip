// measure.hip -- measurement aids declared in include/tlsl_measure.h: the
// per-kernel event timer used by the launchers, a streaming-copy kernel and a
// matrix-core loop kernel for roofline calibration.  Nothing here takes part
// in the token-selection method.
#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/tlsl.h"
#include "../../include/tlsl_measure.h"
#include "tlsl_device.h"
#include "tlsl_internal.h"

namespace tlsl {
namespace {

struct KernelTimer {
    std::atomic<bool> armed{false};
    std::mutex mu;
    char name[96] = "";
    std::vector<hipEvent_t> ev;  // [2*i] before, [2*i+1] after launch i
    int cap = 0, used = 0;
    bool open = false;

    void release() {
        for (hipEvent_t e : ev) (void)hipEventDestroy(e);
        ev.clear();
        cap = used = 0;
        open = false;
    }
};

KernelTimer g_timer;

}  // namespace

void timer_mark(const char* kernel, hipStream_t st, bool after) {
    if (!g_timer.armed.load(std::memory_order_acquire)) return;
    std::lock_guard<std::mutex> lk(g_timer.mu);
    if (strcmp(kernel, g_timer.name) != 0) return;
    if (!after) {
        if (g_timer.used >= g_timer.cap) return;
        if (hipEventRecord(g_timer.ev[2 * g_timer.used], st) == hipSuccess) g_timer.open = true;
    } else if (g_timer.open) {
        if (hipEventRecord(g_timer.ev[2 * g_timer.used + 1], st) == hipSuccess) ++g_timer.used;
        g_timer.open = false;
    }
}

// ---- calibration kernels ----------------------------------------------------
constexpr int CC_NT = 256, CC_UNROLL = 4;

__global__ __launch_bounds__(CC_NT) void calib_copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                            size_t n) {
    const size_t step = (size_t)gridDim.x * CC_NT * CC_UNROLL;
    for (size_t base = (size_t)blockIdx.x * CC_NT * CC_UNROLL + threadIdx.x; base < n; base += step) {
        uint4 v[CC_UNROLL];
#pragma unroll
        for (int u = 0; u < CC_UNROLL; ++u) {
            const size_t i = base + (size_t)u * CC_NT;
            v[u] = i < n ? src[i] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < CC_UNROLL; ++u) {
            const size_t i = base + (size_t)u * CC_NT;
            if (i < n) dst[i] = v[u];
        }
    }
}

constexpr int CM_NT = 256, CM_CHAINS = 8;

template <int DT>
__global__ __launch_bounds__(CM_NT) void calib_mfma_kernel(int iters, float* __restrict__ sink) {
    const uint32_t t = threadIdx.x;
    // small finite operands that depend on the lane, so nothing folds
    const uint32_t ab = DT == kBF16 ? (0x3C003C00u ^ (t & 7u)) : (0x30303030u ^ (t & 3u));
    const uint4 x = make_uint4(ab, ab ^ 1u, ab ^ 2u, ab ^ 3u);
    v4f acc[CM_CHAINS];
#pragma unroll
    for (int j = 0; j < CM_CHAINS; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
    // two rounds per trip: keeps each accumulator in the same registers
    for (int it = 0; it < iters; it += 2) {
#pragma unroll
        for (int j = 0; j < 2 * CM_CHAINS; ++j) {
            if constexpr (DT == kBF16) {
                acc[j % CM_CHAINS] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(v8bf, x), __builtin_bit_cast(v8bf, x), acc[j % CM_CHAINS], 0, 0, 0);
            } else {
                const v8i y = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)x.x, (int)x.y, (int)x.z, (int)x.w};
                acc[j % CM_CHAINS] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(y, y, acc[j % CM_CHAINS], 0, 0, 0, 0,
                                                                                      0, 0);
            }
        }
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < CM_CHAINS; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    sink[(size_t)blockIdx.x * CM_NT + t] = s;
}

}  // namespace tlsl

// ---- C ABI ------------------------------------------------------------------
extern "C" {

int tlsl_timer_arm(const char* kernel, int max_launches) {
    using tlsl::g_timer;
    if (!kernel) return tlsl::report(TLSL_ERR_NULL, "tlsl_timer_arm: kernel is NULL");
    if (max_launches < 1 || max_launches > 65536)
        return tlsl::report(TLSL_ERR_SHAPE, "tlsl_timer_arm: max_launches=%d outside 1..65536", max_launches);
    if (strlen(kernel) >= sizeof g_timer.name)
        return tlsl::report(TLSL_ERR_SHAPE, "tlsl_timer_arm: kernel name too long");
    g_timer.armed.store(false, std::memory_order_release);
    std::lock_guard<std::mutex> lk(g_timer.mu);
    g_timer.release();
    g_timer.ev.resize(2 * (size_t)max_launches);
    for (size_t i = 0; i < g_timer.ev.size(); ++i) {
        if (hipEventCreate(&g_timer.ev[i]) != hipSuccess) {
            g_timer.ev.resize(i);
            g_timer.release();
            return tlsl::report(TLSL_ERR_HIP, "tlsl_timer_arm: hipEventCreate failed");
        }
    }
    strcpy(g_timer.name, kernel);
    g_timer.cap = max_launches;
    g_timer.armed.store(true, std::memory_order_release);
    return tlsl::report(TLSL_OK, nullptr);
}

int tlsl_timer_collect(int* launches, double* total_ms, double* min_ms, double* max_ms) {
    using tlsl::g_timer;
    if (!g_timer.armed.exchange(false, std::memory_order_acq_rel))
        return tlsl::report(TLSL_ERR_SHAPE, "tlsl_timer_collect: the timer is not armed");
    std::lock_guard<std::mutex> lk(g_timer.mu);
    double tot = 0.0, mn = 0.0, mx = 0.0;
    const int n = g_timer.used;
    if (n > 0 && hipEventSynchronize(g_timer.ev[2 * n - 1]) != hipSuccess) {
        g_timer.release();
        return tlsl::report(TLSL_ERR_HIP, "tlsl_timer_collect: hipEventSynchronize failed");
    }
    for (int i = 0; i < n; ++i) {
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, g_timer.ev[2 * i], g_timer.ev[2 * i + 1]) != hipSuccess) {
            g_timer.release();
            return tlsl::report(TLSL_ERR_HIP, "tlsl_timer_collect: hipEventElapsedTime failed");
        }
        tot += ms;
        mn = i == 0 ? ms : fmin(mn, (double)ms);
        mx = i == 0 ? ms : fmax(mx, (double)ms);
    }
    g_timer.release();
    if (launches) *launches = n;
    if (total_ms) *total_ms = tot;
    if (min_ms) *min_ms = mn;
    if (max_ms) *max_ms = mx;
    return tlsl::report(TLSL_OK, nullptr);
}

int tlsl_calib_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
    if (!src || !dst) return tlsl::report(TLSL_ERR_NULL, "tlsl_calib_copy: src and dst must be non-NULL");
    if (bytes == 0 || (bytes & 15u)) return tlsl::report(TLSL_ERR_SHAPE, "tlsl_calib_copy: bytes=%zu", bytes);
    if (((uintptr_t)src & 15u) || ((uintptr_t)dst & 15u))
        return tlsl::report(TLSL_ERR_ALIGN, "tlsl_calib_copy: pointers must be 16-byte aligned");
    const size_t n = bytes / 16;
    const size_t per_block = (size_t)tlsl::CC_NT * tlsl::CC_UNROLL;
    const size_t want = (n + per_block - 1) / per_block;
    const int grid = (int)(want < (size_t)tlsl::device_cu_count() * 16 ? want : (size_t)tlsl::device_cu_count() * 16);
    tlsl::timer_mark("calib_copy_kernel", stream, false);
    hipLaunchKernelGGL(tlsl::calib_copy_kernel, dim3(grid), dim3(tlsl::CC_NT), 0, stream,
                       static_cast<const uint4*>(src), static_cast<uint4*>(dst), n);
    tlsl::timer_mark("calib_copy_kernel", stream, true);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return tlsl::report(TLSL_ERR_HIP, "tlsl_calib_copy: %s", hipGetErrorString(e));
    return tlsl::report(TLSL_OK, nullptr);
}

int tlsl_calib_mfma(int dt, int blocks, int iters, float* sink, double* flops, hipStream_t stream) {
    if (!sink || !flops) return tlsl::report(TLSL_ERR_NULL, "tlsl_calib_mfma: sink and flops must be non-NULL");
    if (blocks <= 0 || iters <= 0 || (iters & 1))
        return tlsl::report(TLSL_ERR_SHAPE, "tlsl_calib_mfma: blocks=%d iters=%d (iters even and positive)", blocks,
                            iters);
    double per = 0.0;
    tlsl::timer_mark("calib_mfma_kernel", stream, false);
    if (dt == TLSL_BF16) {
        hipLaunchKernelGGL(tlsl::calib_mfma_kernel<tlsl::kBF16>, dim3(blocks), dim3(tlsl::CM_NT), 0, stream, iters, sink);
        per = 2.0 * 16 * 16 * 32;
    } else if (dt == TLSL_FP8_E4M3) {
        hipLaunchKernelGGL(tlsl::calib_mfma_kernel<tlsl::kFP8>, dim3(blocks), dim3(tlsl::CM_NT), 0, stream, iters, sink);
        per = 2.0 * 16 * 16 * 128;
    } else {
        return tlsl::report(TLSL_ERR_UNSUPPORTED, "tlsl_calib_mfma: dtype %d (bf16 and fp8 only)", dt);
    }
    tlsl::timer_mark("calib_mfma_kernel", stream, true);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return tlsl::report(TLSL_ERR_HIP, "tlsl_calib_mfma: %s", hipGetErrorString(e));
    *flops = per * (double)blocks * (tlsl::CM_NT / 64) * (double)iters * tlsl::CM_CHAINS;
    return tlsl::report(TLSL_OK, nullptr);
}

}  // extern "C"
