// debug.hip -- optional device-side checks of the index metadata that callers
// hand over in device memory: the sequence boundaries of a decode batch
// (cu_seqlens) and the score rows of the top-k calls (row_start, row_len).
// The host layer cannot read them, and the kernels take them as well formed
// (a decreasing boundary or a negative start would send their loads out of
// bounds).  The checks run only while the debug switch is on (tlsl_set_debug,
// or TLSL_DEBUG in the environment): one single-workgroup kernel per call,
// whose verdict the host copies back after synchronising the caller's
// stream, so that a malformed batch returns an error before anything else
// is launched.
#include <limits.h>

#include <mutex>

#include "../../include/tlsl.h"
#include "tlsl_device.h"
#include "tlsl_internal.h"

namespace tlsl {

constexpr int DB_NT = 1024;
constexpr int64_t kDbgMaxLen = (int64_t(1) << 31) - (int64_t(1) << 12);  // longest supported sequence or row

// Verdict of the last check on a device: {code, index, value, value}; code 0
// means well formed.  Every check writes all four words, so nothing needs
// clearing between calls.
static __device__ __align__(16) long long dbg_verdict[4];

enum : int {
    kDbgOk = 0,
    kDbgFirstNotZero = 1,  // cu_seqlens[0] != 0
    kDbgDecreasing = 2,    // cu_seqlens[b] < cu_seqlens[b-1]
    kDbgSeqTooLong = 3,    // cu_seqlens[b] - cu_seqlens[b-1] >= kDbgMaxLen
    kDbgNegStart = 4,      // row_start[r] < 0
    kDbgNegLen = 5,        // row_len[r] < 0
    kDbgRowTooLong = 6,    // row_len[r] >= kDbgMaxLen
};

// The lowest offending index wins; the thread that found it writes the
// verdict (each index is examined by one thread, which reports its first
// failed condition).
__device__ __forceinline__ void publish(long long idx, int code, long long v0, long long v1, long long* out) {
    __shared__ unsigned long long lowest;
    if (threadIdx.x == 0) lowest = ULLONG_MAX;
    __syncthreads();
    if (code != kDbgOk) atomicMin(&lowest, (unsigned long long)idx);
    __syncthreads();
    if (code != kDbgOk && (unsigned long long)idx == lowest) {
        out[0] = code;
        out[1] = idx;
        out[2] = v0;
        out[3] = v1;
    }
    if (threadIdx.x == 0 && lowest == ULLONG_MAX) {
        out[0] = kDbgOk;
        out[1] = -1;
        out[2] = 0;
        out[3] = 0;
    }
}

__global__ __launch_bounds__(DB_NT) void check_seqlens_kernel(const int64_t* cu, int B, int first_zero,
                                                              long long* out) {
    long long idx = -1, v0 = 0, v1 = 0;
    int code = kDbgOk;
    for (int b = threadIdx.x; b <= B && code == kDbgOk; b += DB_NT) {
        const int64_t x = cu[b];
        if (b == 0) {
            if (first_zero && x != 0) code = kDbgFirstNotZero;
            v0 = x;
        } else {
            const int64_t p = cu[b - 1];
            if (x < p) code = kDbgDecreasing;
            else if (x - p >= kDbgMaxLen) code = kDbgSeqTooLong;
            v0 = x;
            v1 = p;
        }
        idx = b;
    }
    publish(idx, code, v0, v1, out);
}

__global__ __launch_bounds__(DB_NT) void check_rows_kernel(const int64_t* row_start, const int32_t* row_len, int R,
                                                           long long* out) {
    long long idx = -1, v0 = 0, v1 = 0;
    int code = kDbgOk;
    for (int r = threadIdx.x; r < R && code == kDbgOk; r += DB_NT) {
        const int64_t s = row_start[r];
        const int32_t n = row_len[r];
        if (s < 0) code = kDbgNegStart;
        else if (n < 0) code = kDbgNegLen;
        else if (n >= kDbgMaxLen) code = kDbgRowTooLong;
        idx = r;
        v0 = s;
        v1 = n;
    }
    publish(idx, code, v0, v1, out);
}

// Device address of the verdict on the current device (taken once per device
// with hipGetSymbolAddress; the array's name is not a device address on the
// host).
static hipError_t verdict_addr(long long** out) {
    static std::mutex mu;
    static void* addr[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(dbg_verdict));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *out = static_cast<long long*>(addr[dev]);
    return hipSuccess;
}

// Runs the launched check's verdict back to the host (the stream is
// synchronised: the debug mode is for finding malformed inputs, not for
// timing).
static int read_verdict(long long* d, hipStream_t st, long long (&h)[4], const char* fn) {
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = hipMemcpyAsync(h, d, sizeof h, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return report(TLSL_ERR_HIP, "%s: device check failed: %s", fn, hipGetErrorString(e));
    return TLSL_OK;
}

// One verdict array per device: checks are serialised on the host (launch,
// copy back, synchronise) so that two threads checking at once cannot read
// each other's verdict.
static std::mutex g_check_mu;

int debug_check_seqlens(const int64_t* cu, int B, bool first_zero, hipStream_t st, const char* fn) {
    std::lock_guard<std::mutex> lock(g_check_mu);
    long long* d = nullptr;
    hipError_t e = verdict_addr(&d);
    if (e != hipSuccess) return report(TLSL_ERR_HIP, "%s: device check failed: %s", fn, hipGetErrorString(e));
    hipLaunchKernelGGL(check_seqlens_kernel, dim3(1), dim3(DB_NT), 0, st, cu, B, first_zero ? 1 : 0, d);
    long long h[4];
    const int rc = read_verdict(d, st, h, fn);
    if (rc) return rc;
    switch ((int)h[0]) {
        case kDbgOk: return TLSL_OK;
        case kDbgFirstNotZero:
            return report(TLSL_ERR_SHAPE, "%s: cu_seqlens[0] = %lld, must be 0 (device check)", fn, h[2]);
        case kDbgDecreasing:
            return report(TLSL_ERR_SHAPE, "%s: cu_seqlens[%lld] = %lld is below cu_seqlens[%lld] = %lld (device check)",
                          fn, h[1], h[2], h[1] - 1, h[3]);
        case kDbgSeqTooLong:
            return report(TLSL_ERR_SHAPE, "%s: sequence %lld holds %lld entries, above the supported %lld (device check)",
                          fn, h[1] - 1, h[2] - h[3], (long long)kDbgMaxLen - 1);
        default: return report(TLSL_ERR_HIP, "%s: device check returned code %lld", fn, h[0]);
    }
}

int debug_check_rows(const int64_t* row_start, const int32_t* row_len, int R, hipStream_t st, const char* fn) {
    std::lock_guard<std::mutex> lock(g_check_mu);
    long long* d = nullptr;
    hipError_t e = verdict_addr(&d);
    if (e != hipSuccess) return report(TLSL_ERR_HIP, "%s: device check failed: %s", fn, hipGetErrorString(e));
    hipLaunchKernelGGL(check_rows_kernel, dim3(1), dim3(DB_NT), 0, st, row_start, row_len, R, d);
    long long h[4];
    const int rc = read_verdict(d, st, h, fn);
    if (rc) return rc;
    switch ((int)h[0]) {
        case kDbgOk: return TLSL_OK;
        case kDbgNegStart:
            return report(TLSL_ERR_SHAPE, "%s: row_start[%lld] = %lld is negative (device check)", fn, h[1], h[2]);
        case kDbgNegLen:
            return report(TLSL_ERR_SHAPE, "%s: row_len[%lld] = %lld is negative (device check)", fn, h[1], h[3]);
        case kDbgRowTooLong:
            return report(TLSL_ERR_SHAPE, "%s: row_len[%lld] = %lld, above the supported %lld (device check)", fn, h[1],
                          h[3], (long long)kDbgMaxLen - 1);
        default: return report(TLSL_ERR_HIP, "%s: device check returned code %lld", fn, h[0]);
    }
}

}  // namespace tlsl
