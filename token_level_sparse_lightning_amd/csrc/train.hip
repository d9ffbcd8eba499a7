// train.hip -- the indexer's sparse-stage training step on gfx950: the loss of
// the DSA page, section 1.2 eq.(8), KL(p_{t,S_t} || Softmax(I_{t,S_t})) with
// both distributions normalised over the selected set (a teacher cut from a
// dense distribution is divided by its kept mass, the rule after eq.(8)), and
// its gradient into the indexer's inputs q^I, k^I and w^I (the inputs are
// detached from the main model, so the gradient stops there).
//
// One workgroup (four waves) per query row t; the row's slot positions are
// staged in LDS first, so no global load waits behind the dK additions:
//  1. the selected keys' scores I_i = sum_j w_j ReLU(q_j . k_{S_i}) are
//     recomputed with the indexer's scoring tile (bit-identical to the
//     prefill's S_score), 64 gathered keys per wave step (the next step's
//     keys in flight), into LDS;
//  2. softmax over the valid slots, the teacher normalised by its mass on
//     them, the row's loss and g_i = Softmax(I)_i - P_i;
//  3. per 64-slot tile (keys gathered into LDS), wave w owns head block w:
//       X^T = K Q^T (keys x its 16 heads) on the matrix cores,
//       A^T[s, j] = g_s w_j [X^T[s, j] > 0], dw_j += g_s ReLU(X^T[s, j]),
//       dQ^T += K^T A^T (dims x heads; K^T read with the LDS transpose load),
//     then, after the four waves have put A^T in LDS, wave w owns dims
//     32w..32w+31 of D = A^T Q (keys x dims), read back transposed, and adds D
//     to the gathered keys' rows of dK; the next tile's keys are loaded into
//     registers meanwhile.
// A^T enters the products split into two bf16 terms (high part and
// remainder), so the coefficients carry ~16 significant bits and the
// gradients keep fp32-level accuracy.  dK rows collect contributions from
// every query that selected the key; they are added with float atomics, so
// dK's summation order (not its value beyond rounding) varies between runs;
// the loss, dQ and dW are computed in a fixed order.
#include <math.h>

#include <algorithm>

#include "idx_tile.h"
#include "tlsl_device.h"
#include "tlsl_internal.h"

namespace tlsl {

constexpr int TR_NT = 256;                 // four waves
constexpr int TR_DI = 128;                 // indexer dims (bf16)
constexpr int TR_KROW = TR_DI * 2 + 32;    // LDS row of a gathered key (bytes, padded)
constexpr int TR_QROW = TR_DI * 2 + 32;    // LDS row of one query head
constexpr int TR_AROW = 64 * 2 + 16;       // LDS row of A^T transposed: 64 keys of one head

typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_t lds_v4s_t;

struct TrainArgs {
    const unsigned char* q;  // [rows][HI][DI] bf16
    const unsigned char* k;  // [B*n][DI] bf16
    const float* w;          // [rows][HI]
    const int32_t* S;        // [rows][topk]
    const float* p;          // [rows][topk]
    int n, HI, topk;
    float* loss;             // [rows]
    float* dq;               // [rows][HI][DI]
    float* dk;               // [B*n][DI], accumulated (zeroed first)
    float* dw;               // [rows][HI]
};

// LDS transpose load of a 16-lane group: lane r supplies the address of row
// s0 + r/4, columns c0 + 4(r%4) .. +3 (bf16) of a row-major tile; lane i
// receives rows s0 .. s0+3 of column c0 + i (in that order).
__device__ __forceinline__ uint2 lds_tr4(const unsigned char* p) {
    const v4s_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)p);
    return __builtin_bit_cast(uint2, v);
}

__device__ __forceinline__ uint32_t bf16x2(float lo, float hi) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    const b2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_lo_value(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi_value(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }

__device__ __forceinline__ v4f mma_bf16(const uint4& a, const uint4& b, v4f acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), acc, 0, 0,
                                                  0);
}

template <int NW>
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if (lane_id() == 0) red[w] = v;
    __syncthreads();
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) s += red[i];
    return s;
}
template <int NW>
__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if (lane_id() == 0) red[w] = v;
    __syncthreads();
    float s = red[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) s = fmaxf(s, red[i]);
    return s;
}

__global__ __launch_bounds__(TR_NT) void zero_f32_kernel(float* x, size_t n) {
    for (size_t i = (size_t)blockIdx.x * TR_NT + threadIdx.x; i < n; i += (size_t)gridDim.x * TR_NT) x[i] = 0.f;
}

__global__ __launch_bounds__(TR_NT, 2) void indexer_kl_kernel(TrainArgs a) {
    constexpr int DI = TR_DI, NCH = DI * 2 / 64;  // 4 chunks of 16 bytes per lane and row
    using I = Idx<kBF16, 4, DI>;
    __shared__ __align__(16) unsigned char qt[64 * TR_QROW];     // the row's query, heads padded to 64
    __shared__ __align__(16) unsigned char kt[64 * TR_KROW];     // the tile's gathered keys
    __shared__ __align__(16) unsigned char at[2][64 * TR_AROW];  // A^T split, stored [head][key]
    // dynamic: the slots' scores, then g (float[64 nsub]); the slots' positions
    // (int[64 nsub], -1 where the slot is invalid or outside [0, t])
    extern __shared__ __align__(16) unsigned char trdyn[];
    __shared__ float red[8];

    const int tid = threadIdx.x, l = lane_id(), g = l >> 4, c = l & 15;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int row = blockIdx.x;
    const int t = row % a.n;
    const size_t tok0 = (size_t)row - t;
    const int K = a.topk;
    const int nsub = (K + 63) / 64;
    const int32_t* Srow = a.S + (size_t)row * K;
    const float* prow = a.p + (size_t)row * K;
    const unsigned char* kbase = a.k + tok0 * (DI * 2);
    float* gb = reinterpret_cast<float*>(trdyn);
    int* spl = reinterpret_cast<int*>(trdyn + (size_t)nsub * 64 * 4);

    // ---- the query and the row's positions into LDS ---------------------------
    for (int i = tid; i < 64 * (DI * 2 / 16); i += TR_NT) {
        const int h = i / (DI * 2 / 16), ch = i % (DI * 2 / 16);
        uint4 v = make_uint4(0, 0, 0, 0);
        if (h < a.HI) v = *reinterpret_cast<const uint4*>(a.q + ((size_t)row * a.HI + h) * (DI * 2) + ch * 16);
        *reinterpret_cast<uint4*>(qt + h * TR_QROW + ch * 16) = v;
    }
    for (int i = tid; i < nsub * 64; i += TR_NT) {
        const int sp = i < K ? Srow[i] : -1;
        spl[i] = (sp >= 0 && sp <= t) ? sp : -1;
    }
    __syncthreads();

    // ---- 1. scores of the selected keys -------------------------------------
    // Each wave scores subtiles wv, wv + 4, ...; the next subtile's keys are
    // loaded while the current one is scored.
    {
        uint4 qf[4][NCH];
        float wvv[4][4];
        I::load_query(a.q + (size_t)row * a.HI * (DI * 2), a.w + (size_t)row * a.HI, 1.f, a.HI, true, qf, wvv);
        // lane (g, c) of key block kb holds key 16kb + c of the subtile
        auto load_sub = [&](int j, uint4(&kf)[4][NCH]) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int sp = spl[64 * j + 16 * kb + c];
                const uint4* src =
                    reinterpret_cast<const uint4*>(kbase + (size_t)(sp >= 0 ? sp : 0) * (DI * 2) + g * (DI * 2 / 4));
#pragma unroll
                for (int ch = 0; ch < NCH; ++ch) kf[kb][ch] = src[ch];
            }
        };
        if (wv < nsub) {
            uint4 kf[4][NCH];
            load_sub(wv, kf);
            for (int j = wv; j < nsub; j += 4) {
                uint4 kn[4][NCH];
                load_sub(min(j + 4, nsub - 1), kn);  // past the end: a repeat, unused
                const float sc = I::score(qf, wvv, kf);
                const int slot = 64 * j + l;
                if (slot < K) gb[slot] = spl[slot] >= 0 ? sc : -INFINITY;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int ch = 0; ch < NCH; ++ch) kf[kb][ch] = kn[kb][ch];
            }
        }
    }
    __syncthreads();

    // ---- 2. softmax over S_t, the normalised teacher, loss and g ------------
    float mx = -INFINITY;
    for (int i = tid; i < K; i += TR_NT) mx = fmaxf(mx, gb[i]);
    mx = block_max<4>(mx, red);
    float z = 0.f, pm = 0.f;
    for (int i = tid; i < K; i += TR_NT) {
        if (gb[i] != -INFINITY) {
            z += expf(gb[i] - mx);
            pm += prow[i];
        }
    }
    z = block_sum<4>(z, red);
    pm = block_sum<4>(pm, red);
    const bool live = mx != -INFINITY && pm > 0.f;
    const float logz = live ? mx + logf(z) : 0.f;
    float lsum = 0.f;
    for (int i = tid; i < K; i += TR_NT) {
        float gi = 0.f;
        if (live && gb[i] != -INFINITY) {
            const float P = prow[i] / pm;
            const float lr = gb[i] - logz;  // log Softmax(I)_i
            if (P > 0.f) lsum += P * (logf(P) - lr);
            gi = expf(lr) - P;
        }
        gb[i] = gi;
    }
    for (int i = K + tid; i < nsub * 64; i += TR_NT) gb[i] = 0.f;  // the last tile's slots past k
    lsum = block_sum<4>(lsum, red);  // (its barriers also publish g)
    if (tid == 0) a.loss[row] = live ? lsum : 0.f;

    // ---- 3. backward, tile by tile -------------------------------------------
    const int hb = wv;                  // head block of this wave (X^T, A^T, dQ^T, dW)
    const int h = 16 * hb + c;          // the lane's head in those products
    const float wh = h < a.HI ? a.w[(size_t)row * a.HI + h] : 0.f;
    // q^T fragments for D = A^T Q: dims 32*wv + 16*db2 + c, heads 32m + 8g + e
    uint4 qT[2][2];
#pragma unroll
    for (int db2 = 0; db2 < 2; ++db2)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int r = l & 15;
            const int d0 = 32 * wv + 16 * db2;
            const unsigned char* base = qt + (32 * m + 8 * g + (r >> 2)) * TR_QROW + (d0 + 4 * (r & 3)) * 2;
            const uint2 lo = lds_tr4(base), hi = lds_tr4(base + 4 * TR_QROW);
            qT[db2][m] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
    v4f dqa[8];
#pragma unroll
    for (int db = 0; db < 8; ++db) dqa[db] = v4f{0.f, 0.f, 0.f, 0.f};
    float dwa = 0.f;
    // Gather item of a thread: key row tid/4 of the tile, 64 bytes at
    // (tid%4)*64.  Tile j+1 is loaded into registers while tile j is
    // computed and stored into the tile buffer once every wave is done with
    // tile j; its loads are issued before tile j's dK additions, so waiting
    // for them does not wait for those.
    const int grow = tid >> 2, gq = tid & 3;
    uint4 pf[4];
    auto gather_load = [&](int j) {
        const int sp = spl[64 * j + grow];
        const uint4* src = reinterpret_cast<const uint4*>(kbase + (size_t)(sp >= 0 ? sp : 0) * (DI * 2) + gq * 64);
#pragma unroll
        for (int u = 0; u < 4; ++u) pf[u] = src[u];
    };
    auto gather_store = [&](int j) {
        const bool ok = spl[64 * j + grow] >= 0;
        uint4* dst = reinterpret_cast<uint4*>(kt + grow * TR_KROW + gq * 64);
#pragma unroll
        for (int u = 0; u < 4; ++u) dst[u] = ok ? pf[u] : make_uint4(0, 0, 0, 0);
    };
    // dK rows of this sequence as a buffer resource: an invalid slot's
    // additions get an offset past the end, and the hardware drops them, so
    // the additions are issued unconditionally (a fixed count of memory
    // operations per tile).  n * DI * 4 < 2^31 (checked by the caller).
    const __amdgpu_buffer_rsrc_t dkr = __builtin_amdgcn_make_buffer_rsrc(a.dk + tok0 * DI, 0, a.n * DI * 4, 0x00020000);
    if (live && nsub > 0) {
        gather_load(0);
        gather_store(0);
        __syncthreads();
    }
    // nothing loaded before the loop (w of the lane's head) is left pending
    // into it, where a wait for it would also wait for the tile in flight
    __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
    for (int j = 0; j < nsub && live; ++j) {
        const bool more = j + 1 < nsub;
        if (more) gather_load(j + 1);
        // X^T = K Q^T for this wave's head block: lane (g, c) gets keys 16kb + 4g + r, head h
        v4f x[4];
        {
            uint4 qf[NCH];
            const uint4* qs = reinterpret_cast<const uint4*>(qt + h * TR_QROW + g * (DI * 2 / 4));
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) qf[ch] = qs[ch];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                uint4 kf[NCH];
                const uint4* ks = reinterpret_cast<const uint4*>(kt + (16 * kb + c) * TR_KROW + g * (DI * 2 / 4));
#pragma unroll
                for (int ch = 0; ch < NCH; ++ch) kf[ch] = ks[ch];
                x[kb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ch = 0; ch < NCH; ++ch) x[kb] = mma_bf16(kf[ch], qf[ch], x[kb]);
            }
        }
        // A^T = g w [X^T > 0] split into bf16 high part and remainder; dW
        uint32_t ahi[4][2], alo[4][2];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const float4 gs = *reinterpret_cast<const float4*>(gb + 64 * j + 16 * kb + 4 * g);
            const float gv[4] = {gs.x, gs.y, gs.z, gs.w};
            float av[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float xv = x[kb][r];
                dwa = __builtin_fmaf(gv[r], relu(xv), dwa);
                av[r] = xv > 0.f ? gv[r] * wh : 0.f;
            }
#pragma unroll
            for (int r2 = 0; r2 < 2; ++r2) {
                const uint32_t hp = bf16x2(av[2 * r2], av[2 * r2 + 1]);
                ahi[kb][r2] = hp;
                alo[kb][r2] = bf16x2(av[2 * r2] - bf16_lo_value(hp), av[2 * r2 + 1] - bf16_hi_value(hp));
            }
            // [head][key] rows for the transposed read of D = A^T Q
            *reinterpret_cast<uint2*>(at[0] + h * TR_AROW + (16 * kb + 4 * g) * 2) = make_uint2(ahi[kb][0], ahi[kb][1]);
            *reinterpret_cast<uint2*>(at[1] + h * TR_AROW + (16 * kb + 4 * g) * 2) = make_uint2(alo[kb][0], alo[kb][1]);
        }
        // dQ^T (dims x heads) += K^T (dims x keys) A^T (keys x heads); keys of
        // step m: 32m + 4g + e (e < 4) and 32m + 16 + 4g + (e - 4)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const uint4 bh = make_uint4(ahi[2 * m][0], ahi[2 * m][1], ahi[2 * m + 1][0], ahi[2 * m + 1][1]);
            const uint4 bl = make_uint4(alo[2 * m][0], alo[2 * m][1], alo[2 * m + 1][0], alo[2 * m + 1][1]);
#pragma unroll
            for (int db = 0; db < 8; ++db) {
                const int r = l & 15;
                const unsigned char* base = kt + (32 * m + 4 * g + (r >> 2)) * TR_KROW + (16 * db + 4 * (r & 3)) * 2;
                const uint2 k0 = lds_tr4(base), k1 = lds_tr4(base + 16 * TR_KROW);
                const uint4 kA = make_uint4(k0.x, k0.y, k1.x, k1.y);
                dqa[db] = mma_bf16(kA, bh, dqa[db]);
                dqa[db] = mma_bf16(kA, bl, dqa[db]);
            }
        }
        __syncthreads();  // A^T of all heads in LDS
        // D = A^T Q (keys x this wave's 32 dims), heads of step m: 32m + 8g + e
        v4f da[4][2];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
            for (int db2 = 0; db2 < 2; ++db2) da[kb][db2] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int r = l & 15;
                const int off = (32 * m + 8 * g + (r >> 2)) * TR_AROW + (16 * kb + 4 * (r & 3)) * 2;
                const uint2 h0 = lds_tr4(at[0] + off), h1 = lds_tr4(at[0] + off + 4 * TR_AROW);
                const uint2 l0 = lds_tr4(at[1] + off), l1 = lds_tr4(at[1] + off + 4 * TR_AROW);
                const uint4 Ah = make_uint4(h0.x, h0.y, h1.x, h1.y), Al = make_uint4(l0.x, l0.y, l1.x, l1.y);
#pragma unroll
                for (int db2 = 0; db2 < 2; ++db2) {
                    da[kb][db2] = mma_bf16(Ah, qT[db2][m], da[kb][db2]);
                    da[kb][db2] = mma_bf16(Al, qT[db2][m], da[kb][db2]);
                }
            }
        }
        // lane (g, c): keys 16kb + 4g + r, dim 32wv + 16db2 + c
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const int4 sp4 = *reinterpret_cast<const int4*>(spl + 64 * j + 16 * kb + 4 * g);
            const int spv[4] = {sp4.x, sp4.y, sp4.z, sp4.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int off = spv[r] >= 0 ? (spv[r] * DI + 32 * wv + c) * 4 : (int)0x80000000;
#pragma unroll
                for (int db2 = 0; db2 < 2; ++db2)
                    __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(da[kb][db2][r], dkr, off + 64 * db2, 0, 0);
            }
        }
        __syncthreads();  // every wave is done with the tile and A^T
        if (more) {
            gather_store(j + 1);
            __syncthreads();
        }
    }

    // ---- 4. dQ and dW of the row ----------------------------------------------
    if (h < a.HI) {
        float* dst = a.dq + ((size_t)row * a.HI + h) * DI;
#pragma unroll
        for (int db = 0; db < 8; ++db)
            *reinterpret_cast<float4*>(dst + 16 * db + 4 * g) = make_float4(dqa[db][0], dqa[db][1], dqa[db][2], dqa[db][3]);
    }
    dwa = xor32_sum(xor16_sum(dwa));
    if (g == 0 && h < a.HI) a.dw[(size_t)row * a.HI + h] = dwa;
}

hipError_t launch_indexer_kl(const void* q, const void* k, const float* w, const int32_t* S, const float* p, int B,
                             int n, int HI, int topk, float* loss, float* dq, float* dk, float* dw, hipStream_t st) {
    TrainArgs a;
    a.q = static_cast<const unsigned char*>(q);
    a.k = static_cast<const unsigned char*>(k);
    a.w = w;
    a.S = S;
    a.p = p;
    a.n = n;
    a.HI = HI;
    a.topk = topk;
    a.loss = loss;
    a.dq = dq;
    a.dk = dk;
    a.dw = dw;
    const size_t nk = (size_t)B * n * TR_DI;
    const int zb = (int)std::min<size_t>((nk + TR_NT - 1) / TR_NT, (size_t)device_cu_count() * 8);
    TLSL_TIMED_LAUNCH("zero_f32_kernel", st, hipLaunchKernelGGL(zero_f32_kernel, dim3(zb), dim3(TR_NT), 0, st, dk, nk));
    const size_t dyn = (size_t)((topk + 63) / 64) * 64 * 8;  // scores/g and positions of the row's slots
    TLSL_TIMED_LAUNCH("indexer_kl_kernel", st,
                      hipLaunchKernelGGL(indexer_kl_kernel, dim3(B * n), dim3(TR_NT), dyn, st, a));
    return hipGetLastError();
}

}  // namespace tlsl
