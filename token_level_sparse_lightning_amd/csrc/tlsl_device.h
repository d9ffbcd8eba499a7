// tlsl_device.h -- device helpers shared by the gfx950 kernels of the DSA
// token-selection library: matrix-core fragments, order-preserving score keys
// and wave / workgroup scans.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tlsl {

constexpr int kF32 = 0, kBF16 = 1, kFP8 = 2;

typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// ---------------------------------------------------------------------------
// 16x16 matrix-core products.
//
// All three forms produce a 16x16 fp32 tile; lane l holds column (l & 15) and
// rows 4*(l >> 4) + r, r = 0..3.  The operands are "row fragments": lane l
// holds row (l & 15) of A (or column (l & 15) of B) and, for the reduction
// dimension of length DI, the contiguous range [g*DI/4, (g+1)*DI/4) with
// g = l >> 4.  The hardware assigns reduction indices to lanes and registers
// in its own order; because A and B fragments are filled by the same rule,
// the sum over the reduction dimension is complete whatever that order is.
//
// A fragment is kept as 16-byte chunks; NCH = DI * elem_bytes / 64.
// ---------------------------------------------------------------------------
template <int DT>
struct ElemBytes;
template <>
struct ElemBytes<kF32> { static constexpr int v = 4; };
template <>
struct ElemBytes<kBF16> { static constexpr int v = 2; };
template <>
struct ElemBytes<kFP8> { static constexpr int v = 1; };

template <int DT, int DI>
struct Mma {
    static constexpr int ROWB = DI * ElemBytes<DT>::v;  // bytes of one row
    static constexpr int NCH = ROWB / 64;               // 16-B chunks per lane
    static_assert(ROWB % 64 == 0, "row must split into 4 lane groups of 16-B chunks");

    // matrix-core instructions per product, and the s-th of them on its own
    // (run() is the sequence of all steps)
    static constexpr int STEPS = DT == kF32 ? 4 * NCH : (DT == kBF16 ? NCH : NCH / 2);

    __device__ __forceinline__ static v4f step(const uint4* a, const uint4* b, int s, v4f acc) {
        if constexpr (DT == kF32) {
            const uint4 x = a[s >> 2], y = b[s >> 2];
            const uint32_t xa = (s & 3) == 0 ? x.x : (s & 3) == 1 ? x.y : (s & 3) == 2 ? x.z : x.w;
            const uint32_t ya = (s & 3) == 0 ? y.x : (s & 3) == 1 ? y.y : (s & 3) == 2 ? y.z : y.w;
            return __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(xa), __uint_as_float(ya), acc, 0, 0, 0);
        } else if constexpr (DT == kBF16) {
            return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a[s]), __builtin_bit_cast(v8bf, b[s]),
                                                           acc, 0, 0, 0);
        } else {
            const uint4 a0 = a[2 * s], a1 = a[2 * s + 1], b0 = b[2 * s], b1 = b[2 * s + 1];
            const v8i av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
            const v8i bv = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
            return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 0, 0, 0, 0, 0, 0);
        }
    }

    __device__ __forceinline__ static v4f run(const uint4* a, const uint4* b, v4f acc) {
        if constexpr (DT == kF32) {
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[c].x), __uint_as_float(b[c].x), acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[c].y), __uint_as_float(b[c].y), acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[c].z), __uint_as_float(b[c].z), acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[c].w), __uint_as_float(b[c].w), acc, 0, 0, 0);
            }
        } else if constexpr (DT == kBF16) {
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                v8bf av = __builtin_bit_cast(v8bf, a[c]);
                v8bf bv = __builtin_bit_cast(v8bf, b[c]);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
            }
        } else {
            static_assert(NCH % 2 == 0, "fp8 products take 32 bytes per lane");
#pragma unroll
            for (int c = 0; c < NCH; c += 2) {
                v8i av = {(int)a[c].x, (int)a[c].y, (int)a[c].z, (int)a[c].w,
                          (int)a[c + 1].x, (int)a[c + 1].y, (int)a[c + 1].z, (int)a[c + 1].w};
                v8i bv = {(int)b[c].x, (int)b[c].y, (int)b[c].z, (int)b[c].w,
                          (int)b[c + 1].x, (int)b[c + 1].y, (int)b[c + 1].z, (int)b[c + 1].w};
                // format code 0 = fp8 e4m3 for both operands, no block scaling
                acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 0, 0, 0, 0, 0, 0);
            }
        }
        return acc;
    }
};

// ReLU in one integer instruction: a float with the sign bit set is a negative
// int, so max(bits, 0) maps every negative value (and -0.0) to +0.0 and keeps
// the rest.  fmaxf() would add a NaN-quieting instruction per element; NaN
// inputs are outside the contract.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// ---------------------------------------------------------------------------
// Lightning Indexer epilogue (eq.(1) of the DSA page): for one query, given the
// per-head dot products of 4 key blocks of 16 keys and the lane's head
// weights, return in lane l the head-summed score of key l of the 64-key
// subtile.  The reduction order is fixed, so every kernel that calls this
// produces bit-identical scores for the same inputs.
//
// part[kb]: lane's sum over its own 4*HB heads for key (16*kb + (l & 15)).
// Lane groups g = l >> 4 hold disjoint head sets; a two-step transpose-reduce
// (swap halves, then swap 16-lane rows) leaves lane l with key l's full sum.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float reduce_heads_64(const float part[4]) {
    // step 1: exchange blocks {0,1} <-> {2,3} between the two 32-lane halves
    auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[2]), false, false);
    auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[1]), __float_as_uint(part[3]), false, false);
    float r0 = __uint_as_float(s02[0]) + __uint_as_float(s02[1]);  // lower half: block 0, upper: block 2
    float r1 = __uint_as_float(s13[0]) + __uint_as_float(s13[1]);  // lower half: block 1, upper: block 3
    // step 2: exchange between 16-lane rows 0<->1 and 2<->3
    auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(r0), __float_as_uint(r1), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// ---------------------------------------------------------------------------
// Butterfly steps across 16-lane rows (lane l with l^16) and across wave
// halves (l with l^32) through the permlane swaps: no LDS traffic, so they do
// not wait behind outstanding LDS reads.  Both lanes of a pair get the same
// bits (max and + are commutative).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float xor16_max(float x) {
    auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
    auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float xor16_sum(float x) {
    auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
    auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// ---------------------------------------------------------------------------
// Order-preserving 32-bit key of an fp32 score: larger score <=> larger key,
// -0.0 and +0.0 map to the same key.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t score_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(u);
}

// ---------------------------------------------------------------------------
// Wave-level helpers (wave64).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// number of set bits of m in lanes below the calling lane
__device__ __forceinline__ int rank_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}
// number of set bits of m in lanes above the calling lane
__device__ __forceinline__ int rank_above(uint64_t m) {
    return __popcll(m) - rank_below(m) - (int)((m >> lane_id()) & 1ull);
}

__device__ __forceinline__ int wave_incl_scan(int v) {
    const int l = lane_id();
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int o = __shfl_up(v, d, 64);
        if (l >= d) v += o;
    }
    return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    return v;
}
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v = fminf(v, __shfl_xor(v, d, 64));
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
    return v;
}

// Order the wave's own LDS traffic (a wave's LDS operations complete in order;
// this keeps the compiler from reordering across the point).
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// ---------------------------------------------------------------------------
// Radix digit search over a histogram: find the bin d (scanning from the top
// bin down) where the running count first reaches `need`.  Wave version: a
// single wave owns `hist` (NB bins, NB a multiple of 64).
// Returns d; *above = count in bins > d.
// ---------------------------------------------------------------------------
template <int NB>
__device__ __forceinline__ int wave_find_bin(const uint32_t* hist, int need, int* above) {
    constexpr int PER = NB / 64;
    const int l = lane_id();
    // lane l owns bins top - PER*l - j, j = 0..PER-1 (descending)
    int cnts[PER];
    int local = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        cnts[j] = (int)hist[NB - 1 - (PER * l + j)];
        local += cnts[j];
    }
    int incl = wave_incl_scan(local);
    int excl = incl - local;
    bool here = (excl < need) && (incl >= need);
    uint64_t m = ballot(here);
    int src = (int)__builtin_ctzll(m);
    int d = 0, ab = 0;
    if (here) {
        int run = excl;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            if (run + cnts[j] >= need) { d = NB - 1 - (PER * l + j); ab = run; break; }
            run += cnts[j];
        }
    }
    d = __shfl(d, src, 64);
    ab = __shfl(ab, src, 64);
    *above = ab;
    return d;
}

// Workgroup version: all NT threads call; `hist` has NB bins in LDS;
// `scratch` holds at least NT/64 + 2 ints of LDS.  Ends with a barrier so the
// result can be read by every thread and `hist` reused.
template <int NT, int NB>
__device__ __forceinline__ int block_find_bin(const uint32_t* hist, int need, int* above, int* scratch) {
    static_assert(NB % NT == 0, "bins per thread");
    constexpr int PER = NB / NT;
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, l = lane_id(), w = tid >> 6;
    int cnts[PER];
    int local = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        cnts[j] = (int)hist[NB - 1 - (PER * tid + j)];
        local += cnts[j];
    }
    int incl = wave_incl_scan(local);
    if (l == 63) scratch[w] = incl;
    __syncthreads();
    int wbase = 0;
    for (int i = 0; i < w; ++i) wbase += scratch[i];
    incl += wbase;
    int excl = incl - local;
    if (excl < need && incl >= need) {
        int run = excl;
        for (int j = 0; j < PER; ++j) {
            if (run + cnts[j] >= need) { scratch[NW] = NB - 1 - (PER * tid + j); scratch[NW + 1] = run; break; }
            run += cnts[j];
        }
    }
    __syncthreads();
    int d = scratch[NW];
    *above = scratch[NW + 1];
    __syncthreads();
    return d;
}

// Exclusive scan of two 0/1 flags over a workgroup of NT threads, in thread
// order.  Returns (rank of a among set a-flags, rank of b among set b-flags)
// and the totals.  `scratch` holds 2*NT/64 ints of LDS; ends with a barrier.
template <int NT>
__device__ __forceinline__ void block_scan2(bool a, bool b, int* ra, int* rb, int* ta, int* tb, int* scratch) {
    constexpr int NW = NT / 64;
    const int w = threadIdx.x >> 6, l = lane_id();
    uint64_t ma = ballot(a), mb = ballot(b);
    if (l == 0) { scratch[w] = __popcll(ma); scratch[NW + w] = __popcll(mb); }
    __syncthreads();
    int ba = 0, bb = 0, sa = 0, sb = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        int ca = scratch[i], cb = scratch[NW + i];
        if (i < w) { ba += ca; bb += cb; }
        sa += ca; sb += cb;
    }
    *ra = ba + rank_below(ma);
    *rb = bb + rank_below(mb);
    *ta = sa;
    *tb = sb;
    __syncthreads();
}

// Minimum and maximum of a uint32 over a workgroup of NT threads (every thread
// gets both).  `scratch` holds 2*NT/64 ints of LDS; ends with a barrier.
template <int NT>
__device__ __forceinline__ void block_minmax_u32(uint32_t* lo, uint32_t* hi, int* scratch) {
    constexpr int NW = NT / 64;
    const int w = threadIdx.x >> 6, l = lane_id();
    uint32_t a = *lo, b = *hi;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        a = min(a, (uint32_t)__shfl_xor((int)a, d, 64));
        b = max(b, (uint32_t)__shfl_xor((int)b, d, 64));
    }
    if (l == 0) { scratch[w] = (int)a; scratch[NW + w] = (int)b; }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        a = min(a, (uint32_t)scratch[i]);
        b = max(b, (uint32_t)scratch[NW + i]);
    }
    __syncthreads();
    *lo = a;
    *hi = b;
}

// Exclusive scan of two ints over a workgroup of NT threads, in thread order,
// with their totals.  `scratch` holds 2*NT/64 ints of LDS; ends with a barrier.
template <int NT>
__device__ __forceinline__ void block_scan_int2(int a, int b, int* ea, int* eb, int* ta, int* tb, int* scratch) {
    constexpr int NW = NT / 64;
    const int w = threadIdx.x >> 6, l = lane_id();
    const int ia = wave_incl_scan(a), ib = wave_incl_scan(b);
    if (l == 63) { scratch[w] = ia; scratch[NW + w] = ib; }
    __syncthreads();
    int ba = 0, bb = 0, sa = 0, sb = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int ca = scratch[i], cb = scratch[NW + i];
        if (i < w) { ba += ca; bb += cb; }
        sa += ca; sb += cb;
    }
    *ea = ba + ia - a;
    *eb = bb + ib - b;
    *ta = sa;
    *tb = sb;
    __syncthreads();
}

// Copies n (>= 1) items with index i in [0, n) from global memory through
// `store(i, load(i))`, B loads in flight per thread: every load of a batch is
// issued (indices clamped to n-1, so always in bounds) before any is used.
template <int NT, int B, class Load, class Store>
__device__ __forceinline__ void batched_copy(int n, Load load, Store store) {
    for (int i0 = threadIdx.x; i0 < n; i0 += NT * B) {
        decltype(load(0)) v[B];
#pragma unroll
        for (int u = 0; u < B; ++u) v[u] = load(min(i0 + u * NT, n - 1));
#pragma unroll
        for (int u = 0; u < B; ++u)
            if (i0 + u * NT < n) store(i0 + u * NT, v[u]);
    }
}

}  // namespace tlsl
