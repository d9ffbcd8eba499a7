// attn.hip -- attention over the selected shared latent entries on gfx950.
//
// DSA page, section 1.1 eq.(3): the main attention of query t reads only the
// entries c_s, s in S_t.  In the weight-absorbed MQA form (section 2) every
// head reads the same entry, whose full width is the key and whose first Dv
// components are the value.  One workgroup owns one query row (and, in decode,
// one slice of its slots); wave w owns heads 16w..16w+15 and keeps their query
// fragment and their fp32 output accumulator in registers.  Per tile of 32
// slots the workgroup gathers the selected rows once into LDS, twice laid out:
//   - row-major [slot][Dqk]  -> A operand of  Z^T = C Q^T  (slots x heads)
//   - transposed [Dv][slot]  -> A operand of  O^T = V^T P^T (dims x heads)
// so both products read 16-byte contiguous fragments.  The slot order inside
// the first product is permuted so that each lane's logits are exactly the
// P^T fragment the second product needs: the probabilities never leave
// registers.  Softmax is online (running max and sum per head, base-2
// exponentials with log2(e) folded into the scale).
#include <math.h>

#include "tlsl_device.h"
#include "tlsl_internal.h"

namespace tlsl {

constexpr int AT_TS = 32;  // slots per tile

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

struct AttnArgs {
    const unsigned char* q;   // [rows][H][Dqk]
    const unsigned char* kv;  // entries [.][Dqk]
    const int32_t* S;         // [rows][k]
    const int64_t* cu;        // decode: [B+1]; prefill: null
    int n;                    // prefill sequence length (rows = B*n)
    int H, k, nsplit;
    float scale_log2;         // softmax_scale * log2(e)
    unsigned char* out;       // [rows][H][Dv] (no split) -- dtype of the inputs
    float* lse;               // [rows][H] or null
    float* part_o;            // split: [rows][nsplit][H][Dv] fp32 (unnormalised)
    float* part_ml;           // split: [rows][nsplit][H][2] (running max in log2 units, sum)
};

template <int DT, int NW, int DQK, int DV, bool DECODE>
__global__ __launch_bounds__(NW * 64) void sparse_attn_kernel(AttnArgs a) {
    constexpr int EB = ElemBytes<DT>::v;
    constexpr int NT = NW * 64;
    using MQ = Mma<DT, DQK>;
    using MP = Mma<DT, AT_TS>;
    constexpr int NCQ = MQ::NCH;
    constexpr int NCP = MP::NCH;
    constexpr int CROW = DQK * EB;            // bytes of one entry
    constexpr int CSTR = CROW + 16;           // padded LDS row
    constexpr int VROW = AT_TS * EB;          // bytes of one transposed value row
    constexpr int VSTR = VROW + 16;  // 16-byte aligned rows for the 16-byte fragment reads
    constexpr int VPC = 16 / EB;              // values per 16-B chunk
    constexpr int NDB = DV / 16;              // output dim blocks
    static_assert(DV % 16 == 0 && DV <= DQK, "value width");
    __shared__ __align__(16) unsigned char ctile[AT_TS * CSTR];
    __shared__ __align__(16) unsigned char vt[DV * VSTR];
    __shared__ int svalid[AT_TS];

    const int tid = threadIdx.x, w = tid >> 6, l = lane_id(), g = l >> 4, c = l & 15;
    // which row / slot range
    int row, split;
    int64_t kv_base;
    int limit;
    if constexpr (DECODE) {
        row = blockIdx.x / a.nsplit;
        split = blockIdx.x % a.nsplit;
        kv_base = a.cu[row];
        limit = (int)(a.cu[row + 1] - kv_base) - 1;
    } else {
        row = blockIdx.x;
        split = 0;
        const int b = row / a.n;
        kv_base = (int64_t)b * a.n;
        limit = row - b * a.n;
    }
    const int per = (a.k + a.nsplit - 1) / a.nsplit;
    const int sbeg = split * per;
    const int send = min(a.k, sbeg + per);
    const int32_t* Srow = a.S + (size_t)row * a.k;

    // query fragment (B operand of Z^T = C Q^T): column = head 16w + c
    const int h = 16 * w + c;
    const bool hvalid = h < a.H;
    uint4 qf[NCQ];
    {
        const uint4* src = reinterpret_cast<const uint4*>(a.q + ((size_t)row * a.H + (hvalid ? h : 0)) * CROW + g * (CROW / 4));
#pragma unroll
        for (int ch = 0; ch < NCQ; ++ch) qf[ch] = hvalid ? src[ch] : make_uint4(0, 0, 0, 0);
    }
    v4f o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = v4f{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    for (int s0 = sbeg; s0 < send; s0 += AT_TS) {
        // ---- gather the tile ------------------------------------------------
        __syncthreads();
        int my_valid = 0;
        if (tid < AT_TS) {
            const int si = s0 + tid;
            const int pos = si < send ? Srow[si] : -1;
            my_valid = (pos >= 0 && pos <= limit) ? 1 : 0;
            svalid[tid] = my_valid ? pos : -1;
        }
        if (!__syncthreads_or(my_valid)) continue;
        // value part: item = (slot quad, chunk of VPC dims); row-major and transposed
        // slot quad varies fastest across lanes: the transposed writes of one
        // instruction then cover 8 rows x 8 quads, spread over all banks
        for (int it = tid; it < (AT_TS / 4) * (DV / VPC); it += NT) {
            const int qd = it % (AT_TS / 4), oc = it / (AT_TS / 4);
            uint4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int pos = svalid[4 * qd + u];
                v[u] = pos >= 0 ? *reinterpret_cast<const uint4*>(a.kv + (size_t)(kv_base + pos) * CROW + oc * 16)
                                : make_uint4(0, 0, 0, 0);
                *reinterpret_cast<uint4*>(ctile + (4 * qd + u) * CSTR + oc * 16) = v[u];
            }
            if constexpr (EB == 2) {
                const uint16_t* e0 = reinterpret_cast<const uint16_t*>(&v[0]);
                const uint16_t* e1 = reinterpret_cast<const uint16_t*>(&v[1]);
                const uint16_t* e2 = reinterpret_cast<const uint16_t*>(&v[2]);
                const uint16_t* e3 = reinterpret_cast<const uint16_t*>(&v[3]);
#pragma unroll
                for (int i = 0; i < VPC; ++i) {
                    uint2 pk = make_uint2((uint32_t)e0[i] | ((uint32_t)e1[i] << 16), (uint32_t)e2[i] | ((uint32_t)e3[i] << 16));
                    *reinterpret_cast<uint2*>(vt + (oc * VPC + i) * VSTR + 4 * qd * EB) = pk;
                }
            } else {
                const uint32_t* e0 = reinterpret_cast<const uint32_t*>(&v[0]);
                const uint32_t* e1 = reinterpret_cast<const uint32_t*>(&v[1]);
                const uint32_t* e2 = reinterpret_cast<const uint32_t*>(&v[2]);
                const uint32_t* e3 = reinterpret_cast<const uint32_t*>(&v[3]);
#pragma unroll
                for (int i = 0; i < VPC; ++i)
                    *reinterpret_cast<uint4*>(vt + (oc * VPC + i) * VSTR + 4 * qd * EB) = make_uint4(e0[i], e1[i], e2[i], e3[i]);
            }
        }
        // position part (dims DV..DQK-1): row-major only
        constexpr int RC = (DQK - DV) / VPC;  // chunks per row
        for (int it = tid; it < AT_TS * RC; it += NT) {
            const int r = it / RC, oc = DV / VPC + it % RC;
            const int pos = svalid[r];
            *reinterpret_cast<uint4*>(ctile + r * CSTR + oc * 16) =
                pos >= 0 ? *reinterpret_cast<const uint4*>(a.kv + (size_t)(kv_base + pos) * CROW + oc * 16)
                         : make_uint4(0, 0, 0, 0);
        }
        __syncthreads();

        // ---- logits: Z^T[slot][head]; lane (g,c) gets slots 8g..8g+7 of head c
        float z[8];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const int slot_row = 8 * (c >> 2) + 4 * sb + (c & 3);
            const uint4* cp = reinterpret_cast<const uint4*>(ctile + slot_row * CSTR + g * (CROW / 4));
            uint4 cf[NCQ];
#pragma unroll
            for (int ch = 0; ch < NCQ; ++ch) cf[ch] = cp[ch];
            const v4f acc = MQ::run(cf, qf, v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int slot = 8 * g + 4 * sb + r;
                z[4 * sb + r] = svalid[slot] >= 0 ? acc[r] * a.scale_log2 : -INFINITY;
            }
        }
        // ---- online softmax per head -----------------------------------------
        float mx = z[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) mx = fmaxf(mx, z[j]);
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx);
        float p[8];
        float alpha = 1.f;
        if (m_new == -INFINITY) {
#pragma unroll
            for (int j = 0; j < 8; ++j) p[j] = 0.f;
        } else {
            alpha = exp2f(m_run - m_new);
            float ps = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                p[j] = exp2f(z[j] - m_new);
                ps += p[j];
            }
            l_run = l_run * alpha + ps;
            m_run = m_new;
        }
        if (__ballot(alpha != 1.f)) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) o[db] *= alpha;
        }
        // P^T fragment: column = head c, slots 8g..8g+7
        uint4 pf[NCP];
        if constexpr (EB == 2) {
            pf[0] = make_uint4((uint32_t)f32_to_bf16_rne(p[0]) | ((uint32_t)f32_to_bf16_rne(p[1]) << 16),
                               (uint32_t)f32_to_bf16_rne(p[2]) | ((uint32_t)f32_to_bf16_rne(p[3]) << 16),
                               (uint32_t)f32_to_bf16_rne(p[4]) | ((uint32_t)f32_to_bf16_rne(p[5]) << 16),
                               (uint32_t)f32_to_bf16_rne(p[6]) | ((uint32_t)f32_to_bf16_rne(p[7]) << 16));
        } else {
            pf[0] = make_uint4(__float_as_uint(p[0]), __float_as_uint(p[1]), __float_as_uint(p[2]), __float_as_uint(p[3]));
            pf[1] = make_uint4(__float_as_uint(p[4]), __float_as_uint(p[5]), __float_as_uint(p[6]), __float_as_uint(p[7]));
        }
        // ---- O^T[d][head] += V^T[d][slots] P^T[slots][head] -------------------
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const uint4* vp = reinterpret_cast<const uint4*>(vt + (16 * db + c) * VSTR + g * (VROW / 4));
            uint4 vf[NCP];
#pragma unroll
            for (int ch = 0; ch < NCP; ++ch) vf[ch] = vp[ch];
            o[db] = MP::run(vf, pf, o[db]);
        }
    }

    // ---- finish --------------------------------------------------------------
    float l_tot = l_run + __shfl_xor(l_run, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    if (a.part_o) {
        // split: unnormalised partials
        const size_t pidx = ((size_t)row * a.nsplit + split) * a.H + h;
        if (hvalid) {
            float* po = a.part_o + pidx * DV;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                *reinterpret_cast<float4*>(po + 16 * db + 4 * g) = make_float4(o[db][0], o[db][1], o[db][2], o[db][3]);
            if (g == 0) {
                a.part_ml[pidx * 2] = m_run;
                a.part_ml[pidx * 2 + 1] = l_tot;
            }
        }
        return;
    }
    if (!hvalid) return;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    unsigned char* op = a.out + ((size_t)row * a.H + h) * DV * EB;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        const int d0 = 16 * db + 4 * g;
        if constexpr (EB == 2) {
            uint2 pk = make_uint2((uint32_t)f32_to_bf16_rne(o[db][0] * inv) | ((uint32_t)f32_to_bf16_rne(o[db][1] * inv) << 16),
                                  (uint32_t)f32_to_bf16_rne(o[db][2] * inv) | ((uint32_t)f32_to_bf16_rne(o[db][3] * inv) << 16));
            *reinterpret_cast<uint2*>(op + d0 * 2) = pk;
        } else {
            *reinterpret_cast<float4*>(op + d0 * 4) = make_float4(o[db][0] * inv, o[db][1] * inv, o[db][2] * inv, o[db][3] * inv);
        }
    }
    if (a.lse && g == 0)
        a.lse[(size_t)row * a.H + h] = l_tot > 0.f ? (m_run + log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
}

// Merge the split partials of a decode row: o = sum_s 2^(m_s-M) o_s / sum_s 2^(m_s-M) l_s.
// One workgroup per (row, head); each thread owns DV/CB_NT consecutive dims.
constexpr int CB_NT = 128;

template <int DT, int DV>
__global__ __launch_bounds__(CB_NT) void attn_combine_kernel(const float* part_o, const float* part_ml, int H, int nsplit,
                                                             unsigned char* out, float* lse) {
    constexpr int EB = ElemBytes<DT>::v;
    constexpr int PER = (DV + CB_NT - 1) / CB_NT;
    const int row = blockIdx.x / H, h = blockIdx.x % H;
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, part_ml[(((size_t)row * nsplit + s) * H + h) * 2]);
    float L = 0.f, acc[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) acc[j] = 0.f;
    if (M != -INFINITY) {
        for (int s = 0; s < nsplit; ++s) {
            const size_t pidx = ((size_t)row * nsplit + s) * H + h;
            const float ms = part_ml[pidx * 2];
            const float f = ms == -INFINITY ? 0.f : exp2f(ms - M);
            L += f * part_ml[pidx * 2 + 1];
            const float* po = part_o + pidx * DV;
#pragma unroll
            for (int j = 0; j < PER; ++j) {
                const int d = threadIdx.x * PER + j;
                if (d < DV) acc[j] += f * po[d];
            }
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const size_t ob = ((size_t)row * H + h) * DV;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int d = threadIdx.x * PER + j;
        if (d >= DV) continue;
        if constexpr (EB == 2)
            reinterpret_cast<uint16_t*>(out)[ob + d] = f32_to_bf16_rne(acc[j] * inv);
        else
            reinterpret_cast<float*>(out)[ob + d] = acc[j] * inv;
    }
    if (lse && threadIdx.x == 0) lse[(size_t)row * H + h] = L > 0.f ? (M + log2f(L)) * 0.6931471805599453f : -INFINITY;
}

// ---------------------------------------------------------------------------
bool attn_supported(const AttnShape& s) {
    if (s.dt == kBF16) return s.Dqk == 576 && s.Dv == 512 && s.H >= 1 && s.H <= 128;
    if (s.dt == kF32) return s.Dqk == 80 && s.Dv == 64 && s.H >= 1 && s.H <= 16;
    return false;
}

static int decode_splits(int B, int k) {
    int ns = (256 + B - 1) / B;
    const int maxs = (k + 127) / 128;
    if (ns > maxs) ns = maxs;
    return ns < 1 ? 1 : ns;
}

size_t attn_decode_ws_bytes(const AttnShape& s, int B, int k) {
    const int ns = decode_splits(B, k);
    if (ns == 1) return 256;  // never empty, so that a NULL workspace always means "size query"
    const size_t parts = (size_t)B * ns * s.H;
    return parts * s.Dv * sizeof(float) + ((parts * 2 * sizeof(float) + 255) & ~(size_t)255) + 256;
}

template <int DT, int NW, int DQK, int DV, bool DEC>
static void launch_attn_t(const AttnArgs& a, int grid, hipStream_t st) {
    hipLaunchKernelGGL((sparse_attn_kernel<DT, NW, DQK, DV, DEC>), dim3(grid), dim3(NW * 64), 0, st, a);
}

template <bool DEC>
static void dispatch_attn(const AttnShape& s, const AttnArgs& a, int grid, hipStream_t st) {
    if (s.dt == kBF16) {
        if (s.H <= 16) launch_attn_t<kBF16, 1, 576, 512, DEC>(a, grid, st);
        else launch_attn_t<kBF16, 8, 576, 512, DEC>(a, grid, st);
    } else {
        launch_attn_t<kF32, 1, 80, 64, DEC>(a, grid, st);
    }
}

hipError_t launch_sparse_attn_prefill(const AttnShape& s, const void* q, const void* kv, const int32_t* S, int B,
                                      int n, int k, float scale, void* out, float* lse, hipStream_t st) {
    AttnArgs a{};
    a.q = static_cast<const unsigned char*>(q);
    a.kv = static_cast<const unsigned char*>(kv);
    a.S = S;
    a.cu = nullptr;
    a.n = n;
    a.H = s.H;
    a.k = k;
    a.nsplit = 1;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.out = static_cast<unsigned char*>(out);
    a.lse = lse;
    dispatch_attn<false>(s, a, B * n, st);
    return hipGetLastError();
}

hipError_t launch_sparse_attn_decode(const AttnShape& s, const void* q, const void* kv, const int64_t* cu,
                                     const int32_t* S, int B, int k, float scale, void* out, float* lse, void* ws,
                                     hipStream_t st) {
    const int ns = decode_splits(B, k);
    AttnArgs a{};
    a.q = static_cast<const unsigned char*>(q);
    a.kv = static_cast<const unsigned char*>(kv);
    a.S = S;
    a.cu = cu;
    a.n = 0;
    a.H = s.H;
    a.k = k;
    a.nsplit = ns;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.out = static_cast<unsigned char*>(out);
    a.lse = lse;
    if (ns > 1) {
        const size_t parts = (size_t)B * ns * s.H;
        a.part_o = static_cast<float*>(ws);
        a.part_ml = reinterpret_cast<float*>(static_cast<unsigned char*>(ws) + parts * s.Dv * sizeof(float));
    }
    dispatch_attn<true>(s, a, B * ns, st);
    if (ns > 1) {
        if (s.dt == kBF16)
            hipLaunchKernelGGL((attn_combine_kernel<kBF16, 512>), dim3(B * s.H), dim3(CB_NT), 0, st, a.part_o, a.part_ml,
                               s.H, ns, a.out, lse);
        else
            hipLaunchKernelGGL((attn_combine_kernel<kF32, 64>), dim3(B * s.H), dim3(CB_NT), 0, st, a.part_o, a.part_ml,
                               s.H, ns, a.out, lse);
    }
    return hipGetLastError();
}

}  // namespace tlsl
