// attn.hip -- attention over the selected shared latent entries on gfx950.
//
// DSA page, section 1.1 eq.(3): the main attention of query t reads only the
// entries c_s, s in S_t.  In the weight-absorbed MQA form (section 2) every
// head reads the same entry, whose full width is the key and whose first Dv
// components are the value.
//
// A workgroup owns one query row (decode: one slice of a row's slots) and 16*HBW
// heads.  Each block of 16 heads belongs to DSPLIT waves that split the work:
// the logits Z^T = C Q^T over the reduction dims (partial logits are exchanged
// through LDS) and the output O^T = V^T P^T over the value dims -- so each wave
// holds part of a query fragment and part of an output accumulator in
// registers.  Per tile of 32 slots the selected rows are gathered once into
// LDS, row-major [slot][Dqk] (bf16: straight from global memory by the direct
// global->LDS load, two tiles ahead, three rotating buffers, one barrier per
// tile; fp32: through registers): the A operand of Z^T is read from it
// directly and, for bf16,
// the A operand of O^T (V^T) with the LDS transpose load; fp32 keeps a second,
// transposed [Dv][slot] copy.  The slot order inside the first product is
// permuted so that each lane's probabilities are exactly the P^T fragment the
// second product needs.  Softmax is online (running max and
// sum per head, base-2 exponentials with log2(e) folded into the scale).  When
// a row needs two head groups, their workgroups are numbered 8 apart so that
// they run on the same XCD and the second gather of each row is served by that
// XCD's L2.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "tlsl_device.h"
#include "tlsl_internal.h"

namespace tlsl {

constexpr int AT_TS = 32;      // slots per tile
constexpr int AT_KMAX = 4096;  // slots per workgroup (k <= 4096)

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(3))) unsigned char lds_uc;

// two floats to packed bf16 (round to nearest even; one gfx950 instruction)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) { return (uint16_t)pack_bf16x2(f, 0.f); }

struct AttnArgs {
    const unsigned char* q;   // [rows][H][Dqk]
    const unsigned char* kv;  // entries [.][Dqk]
    const int32_t* S;         // [rows][k]; NULL: slot i of every row is position i (dense prefill)
    const int64_t* cu;        // decode: [B+1]; prefill: null
    int n;                    // prefill sequence length (rows = B*n)
    int H, k, nsplit;
    int rows;                 // prefill: B*n; decode: B*nsplit
    float scale_log2;         // softmax_scale * log2(e)
    unsigned char* out;       // [rows][H][Dv] (no split) -- dtype of the inputs
    float* lse;               // [rows][H] or null
    float* part_o;            // split: [rows][nsplit][H][Dv] fp32 (unnormalised)
    float* part_ml;           // split: [rows][nsplit][H][2] (running max in log2 units, sum)
};

template <int DT, int HBW, int DSPLIT, int DQK, int DV, bool DECODE>
__global__ __launch_bounds__(HBW * DSPLIT * 64) void sparse_attn_kernel(AttnArgs a) {
    constexpr int EB = ElemBytes<DT>::v;
    constexpr int NW = HBW * DSPLIT;
    constexpr int NT = NW * 64;
    constexpr int HPW = 16 * HBW;             // heads per workgroup
    constexpr int QKD = DQK / DSPLIT;         // reduction dims per wave
    constexpr int NCQ = QKD * EB / 64;        // 16-B chunks per lane of the wave's query fragment
    constexpr int DVW = DV / DSPLIT;          // value dims per wave
    constexpr int NDB = DVW / 16;             // output dim blocks per wave
    constexpr int NCP = AT_TS * EB / 64;      // chunks per lane of a P^T / V^T fragment
    constexpr int CROW = DQK * EB;            // bytes of one entry
    constexpr int VROW = AT_TS * EB;          // bytes of one transposed value row
    constexpr int VSTR = VROW + 16;           // 16-byte aligned rows for the 16-byte fragment reads
    constexpr int VPC = 16 / EB;              // values per 16-B chunk
    static_assert((QKD * EB) % 64 == 0 && DVW % 16 == 0 && DV <= DQK, "shape");
    // LDS tile rows.  bf16: unpadded rows of 72 16-byte chunks; chunk k of
    // row r sits at chunk k ^ f(r) of its group of 16 (the last 8 chunks:
    // k ^ f(r)/2 inside those 8), f(r) = 4*(r/8) + r%4.  The 16 rows one lane
    // group reads for the logits have f = 0..15 and so do the rows of one
    // transpose load, so both reads, and the 16 (slot, chunk) items of one
    // store, fall in distinct banks.  fp32: padded rows, those 16 apart
    // shifted by 64 bytes.
    static_assert(EB == 4 || CROW == 72 * 16, "bf16 tile layout assumes 576-wide entries");
    constexpr int CSTR = EB == 2 ? CROW : CROW + 16;
    auto cpos = [](int r, int k) -> int {  // byte offset of chunk k of row r
        if constexpr (EB == 2) {
            const int f = ((r >> 3) << 2) | (r & 3);
            const int kk = k < 64 ? ((k & ~15) | ((k ^ f) & 15)) : (64 | ((k ^ (f >> 1)) & 7));
            return r * CSTR + 16 * kk;
        } else {
            return r * CSTR + (r >> 4) * 64 + 16 * k;
        }
    };
    // bf16: three tile buffers, gathered straight into LDS two tiles ahead of
    // the tile being computed; fp32: one buffer, stored from registers
    constexpr int NBUF = EB == 2 ? 3 : 1;
    constexpr int CTB = AT_TS * CSTR + (EB == 2 ? 0 : (AT_TS / 16) * 64);  // bytes of one tile buffer
    __shared__ __align__(16) unsigned char ctile[NBUF][CTB];
    // fp32 values are also kept transposed ([d][slot]) for the P.V product;
    // bf16 values are read transposed from ctile by the LDS transpose load
    __shared__ __align__(16) unsigned char vt[EB == 2 ? 16 : DV * VSTR];
    __shared__ __align__(16) int slots[AT_KMAX];  // the row's slot range: entry gathered (0 if invalid)
    __shared__ uint32_t tile_mask[AT_KMAX / AT_TS];  // by tile
    __shared__ int tlist[AT_KMAX / AT_TS];           // listed tiles (at least one valid slot)
    __shared__ uint32_t lmask[AT_KMAX / AT_TS];      // their masks
    __shared__ int ntl_sh;
    // partial logits of each wave, lane-contiguous (conflict-free exchange);
    // bf16: one set per tile parity (one barrier per tile separates a set's
    // reads from its next writes only two tiles later)
    constexpr int NZX = EB == 2 ? 2 : 1;
    __shared__ __align__(16) float4 zx0[NZX][DSPLIT > 1 ? NT : 1];
    __shared__ __align__(16) float4 zx1[NZX][DSPLIT > 1 ? NT : 1];

    const int tid = threadIdx.x, l = lane_id(), g = l >> 4, c = l & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hb = w / DSPLIT, half = w % DSPLIT;
    // workgroup -> (row, head group); two head groups of a row sit 8 apart
    const int HG = (a.H + HPW - 1) / HPW;
    int rs, hgi;
    if (HG == 1) {
        rs = blockIdx.x;
        hgi = 0;
    } else {
        const int grp = blockIdx.x / (8 * HG), rem = blockIdx.x % (8 * HG);
        hgi = rem / 8;
        rs = grp * 8 + rem % 8;
    }
    if (rs >= a.rows) return;
    int qrow, split;
    int64_t kv_base;
    int limit;
    if constexpr (DECODE) {
        qrow = rs / a.nsplit;
        split = rs % a.nsplit;
        kv_base = a.cu[qrow];
        limit = (int)(a.cu[qrow + 1] - kv_base) - 1;
    } else {
        // latest rows first: the rows with the longest histories start early
        // and the short ones fill the tail
        qrow = a.rows - 1 - rs;
        split = 0;
        const int b = qrow / a.n;
        kv_base = (int64_t)b * a.n;
        limit = qrow - b * a.n;
    }
    const int per = (a.k + a.nsplit - 1) / a.nsplit;
    const int sbeg = split * per;
    const int send = min(a.k, sbeg + per);
    const int nsl = max(send - sbeg, 0);
    const int ntiles = (nsl + AT_TS - 1) / AT_TS;
    // no S (dense prefill): slot i is position i
    const int32_t* Srow = a.S ? a.S + (size_t)qrow * a.k : nullptr;

    // the row's slot range, staged once: the entry each slot gathers, padded
    // to whole tiles, with a validity mask per tile (bit j: slot j); each wave covers
    // 64 consecutive slots, i.e. two tiles, per ballot
    for (int base = 64 * w; base < ntiles * AT_TS; base += NT) {
        const int i = base + l;
        const int pos = i < nsl ? (Srow ? Srow[sbeg + i] : sbeg + i) : -1;
        const bool v = pos >= 0 && pos <= limit;
        // an invalid slot gathers the sequence's entry 0 (in bounds); its
        // logit is masked to -inf
        if (i < ntiles * AT_TS) slots[i] = v ? pos : 0;
        const uint64_t vb = ballot(v);
        if (l == 0) {
            tile_mask[base / AT_TS] = (uint32_t)vb;
            if (base / AT_TS + 1 < ntiles) tile_mask[base / AT_TS + 1] = (uint32_t)(vb >> 32);
        }
    }
    __syncthreads();
    // tiles without a valid slot are skipped: list the others in order, with
    // their masks
    if (w == 0) {
        int m = 0;
        for (int b = 0; b < ntiles; b += 64) {
            const uint32_t mk = b + l < ntiles ? tile_mask[b + l] : 0u;
            const uint64_t any = ballot(mk != 0u);
            if (mk != 0u) {
                tlist[m + rank_below(any)] = b + l;
                lmask[m + rank_below(any)] = mk;
            }
            m += __popcll(any);
        }
        if (l == 0) ntl_sh = m;
    }

    // query fragment (B operand of Z^T = C Q^T): column = head h, this wave's
    // share of the reduction dims
    const int h = hgi * HPW + 16 * hb + c;
    const bool hvalid = h < a.H;
    const int kd0 = half * QKD;  // first reduction dim of this wave
    uint4 qf[NCQ];
    {
        const uint4* src = reinterpret_cast<const uint4*>(a.q + ((size_t)qrow * a.H + (hvalid ? h : 0)) * CROW +
                                                          (kd0 + g * (QKD / 4)) * EB);
#pragma unroll
        for (int ch = 0; ch < NCQ; ++ch) qf[ch] = hvalid ? src[ch] : make_uint4(0, 0, 0, 0);
        // wait here, once: otherwise the compiler places this wait (vmcnt(0))
        // inside the tile loop, where it would also wait for the bf16 gather
        __builtin_amdgcn_s_waitcnt(0xF70);
    }
    v4f o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = v4f{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    __syncthreads();
    const int ntl = ntl_sh;

    // ---- fp32 gather of one tile: value part (quad of slots x 16-byte chunk)
    // and position part (row x chunk); registers first, LDS after the compute
    // (bf16 gathers straight into LDS, below) ----
    constexpr int VITEMS = (AT_TS / 4) * (DV / VPC);
    constexpr int VPER = (VITEMS + NT - 1) / NT;
    constexpr int RC = (DQK - DV) / VPC;  // position-part chunks per row
    constexpr int RITEMS = AT_TS * RC;
    constexpr int RPER = (RITEMS + NT - 1) / NT;
    // plain 4 x u32 vectors: copied with vector loads and stores (a struct
    // copy would go through a stack slot)
    struct Pre {
        v4u v[VPER][4];
        v4u r[RPER > 0 ? RPER : 1];
    };
    // each thread gathers the same (slot quad, chunk) items of every tile:
    // their base addresses are fixed, a load adds the slot's entry offset
    const unsigned char* kvrow = a.kv + (size_t)kv_base * CROW;
    int vqd[VPER], rrow[RPER > 0 ? RPER : 1];
    const unsigned char* vsrc[VPER];
    const unsigned char* rsrc[RPER > 0 ? RPER : 1];
    // value item -> (slot quad, chunk), the quad varying fastest
    auto vitem = [](int it, int& qd, int& oc) {
        qd = it % (AT_TS / 4);
        oc = it / (AT_TS / 4);
    };
#pragma unroll
    for (int j = 0; j < VPER; ++j) {
        // items past the end repeat the last one, so every thread issues the
        // same loads and the compiler's wait counts stay exact
        int qd, oc;
        vitem(min(tid + j * NT, VITEMS - 1), qd, oc);
        vqd[j] = qd;
        vsrc[j] = kvrow + oc * 16;
    }
#pragma unroll
    for (int j = 0; j < RPER; ++j) {
        const int it = min(tid + j * NT, RITEMS - 1);
        rrow[j] = it / RC;
        rsrc[j] = kvrow + (DV / VPC + it % RC) * 16;
    }
    auto load_tile = [&](int t, Pre& P) {
        const int* sl = slots + t * AT_TS;
#pragma unroll
        for (int j = 0; j < VPER; ++j) {
            const int4 q4 = *reinterpret_cast<const int4*>(sl + 4 * vqd[j]);
            const int qs[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                // an invalid slot reads the row's entry 0 (always in bounds):
                // its logit is masked to -inf, so its probability is exactly 0
                const uint32_t pos = (uint32_t)qs[u];
                P.v[j][u] = *reinterpret_cast<const v4u*>(vsrc[j] + (size_t)pos * CROW);
            }
        }
#pragma unroll
        for (int j = 0; j < RPER; ++j) {
            const uint32_t pos = (uint32_t)sl[rrow[j]];
            P.r[j] = *reinterpret_cast<const v4u*>(rsrc[j] + (size_t)pos * CROW);
        }
    };
    auto store_tile = [&](const Pre& P, unsigned char* ct) {
#pragma unroll
        for (int j = 0; j < VPER; ++j) {
            const int it = tid + j * NT;
            if (it < VITEMS) {
                int qd, oc;
                vitem(it, qd, oc);
#pragma unroll
                for (int u = 0; u < 4; ++u) *reinterpret_cast<v4u*>(ct + cpos(4 * qd + u, oc)) = P.v[j][u];
                if constexpr (EB == 4) {
#pragma unroll
                    for (int i = 0; i < VPC; ++i)
                        *reinterpret_cast<v4u*>(vt + (oc * VPC + i) * VSTR + 4 * qd * EB) =
                            v4u{P.v[j][0][i], P.v[j][1][i], P.v[j][2][i], P.v[j][3][i]};
                }
            }
        }
#pragma unroll
        for (int j = 0; j < RPER; ++j) {
            const int it = tid + j * NT;
            if (it < RITEMS) {
                const int r = it / RC, oc = DV / VPC + it % RC;
                *reinterpret_cast<v4u*>(ct + cpos(r, oc)) = P.r[j];
            }
        }
    };
    // per-lane LDS offsets of the fragment reads (the same in every tile)
    // logits: chunk (kd0 + g*QKD/4)*EB/16 + ch of row sigma = 8*(c/4) + c%4
    int qoff[NCQ];
    const int sig = 8 * (c >> 2) + (c & 3);
#pragma unroll
    for (int ch = 0; ch < NCQ; ++ch) qoff[ch] = cpos(sig, (kd0 + g * (QKD / 4)) * EB / 16 + ch);
    // bf16 transpose loads: lane r of a 16-lane group addresses row 8g + r/4
    // at dims d0 + 4*(r%4) .. +3, d0 = half*DVW + 16*db
    int poff[8];
    if constexpr (EB == 2) {
        static_assert(NDB == 16, "bf16 value blocks");
        const int rr = l & 15;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            const int d = half * DVW + 16 * db + 4 * (rr & 3);
            poff[db] = cpos(8 * g + (rr >> 2), d / 8) + 2 * (d & 7);
        }
    }
    // one 16-byte chunk of the reduction dimension through the matrix cores
    auto mma_chunk = [](const uint4& x, const uint4& y, v4f acc) -> v4f {
        if constexpr (DT == kBF16) {
            return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, x), __builtin_bit_cast(v8bf, y), acc, 0, 0, 0);
        } else {
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(x.x), __uint_as_float(y.x), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(x.y), __uint_as_float(y.y), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(x.z), __uint_as_float(y.z), acc, 0, 0, 0);
            return __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(x.w), __uint_as_float(y.w), acc, 0, 0, 0);
        }
    };

    // one tile: logits, exchange, softmax, P.V.  `mid` runs after the P.V
    // fragments are read and before the P.V products; `pre` and `post` run
    // just before and just after the barrier of the logit exchange (bf16: the
    // gather's wait and its next issue)
    auto compute = [&](uint32_t tm, const unsigned char* ct, int par, auto&& pre, auto&& post, auto&& mid) {
        const uint32_t tmg = tm >> (8 * g);  // validity of this lane's slots 8g..8g+7

        // ---- logits: Z^T[slot][head]; lane (g,c) gets slots 8g..8g+7 of head c
        float z[8];
        {
            // rows sigma = 8*(c/4) + c%4 and sigma + 4: the same f (bf16) and the
            // same 16-row shift (fp32), so 4 rows apart
            uint4 ca[NCQ], cb[NCQ];
#pragma unroll
            for (int ch = 0; ch < NCQ; ++ch) {
                ca[ch] = *reinterpret_cast<const uint4*>(ct + qoff[ch]);
                cb[ch] = *reinterpret_cast<const uint4*>(ct + qoff[ch] + 4 * CSTR);
            }
            // every fragment read is in flight before the first product
            __builtin_amdgcn_sched_barrier(0);
            v4f acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ch = 0; ch < NCQ; ++ch) {
                acc0 = mma_chunk(ca[ch], qf[ch], acc0);
                acc1 = mma_chunk(cb[ch], qf[ch], acc1);
            }
            if constexpr (DSPLIT > 1) {
                // add the partner wave's partial logits (the same sum in both waves)
                zx0[par][tid] = make_float4(acc0[0], acc0[1], acc0[2], acc0[3]);
                zx1[par][tid] = make_float4(acc1[0], acc1[1], acc1[2], acc1[3]);
                pre();
                __syncthreads();
                post();
                const float4 o0 = zx0[par][tid ^ 64], o1 = zx1[par][tid ^ 64];
                acc0[0] += o0.x; acc0[1] += o0.y; acc0[2] += o0.z; acc0[3] += o0.w;
                acc1[0] += o1.x; acc1[1] += o1.y; acc1[2] += o1.z; acc1[3] += o1.w;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                z[r] = (tmg >> r) & 1u ? acc0[r] * a.scale_log2 : -INFINITY;
                z[4 + r] = (tmg >> (4 + r)) & 1u ? acc1[r] * a.scale_log2 : -INFINITY;
            }
        }
        // V^T fragments of the tile, read before the softmax so that their
        // latency overlaps it
        uint4 vb[NDB][NCP];
        if constexpr (EB == 2) {
            // transpose loads from the row-major tile: within each 16-lane
            // group, lane r addresses row (slot) s0 + r/4 at dims d0 + 4*(r%4)
            // .. +3, and lane i receives slots s0..s0+3 of dim d0 + i; two
            // loads (s0 = 8g, 8g+4) give the lane's 8-slot fragment
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                // blocks 8 apart are 16 chunks apart: same XOR, +256 bytes
                const unsigned char* tp = ct + poff[db & 7] + 256 * (db >> 3);
                const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)tp);
                const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(tp + 4 * CSTR));
                const uint2 a = __builtin_bit_cast(uint2, lo), b2 = __builtin_bit_cast(uint2, hi);
                vb[db][0] = make_uint4(a.x, a.y, b2.x, b2.y);
            }
        } else {
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const uint4* vp = reinterpret_cast<const uint4*>(vt + (half * DVW + 16 * db + c) * VSTR + g * (VROW / 4));
#pragma unroll
                for (int ch = 0; ch < NCP; ++ch) vb[db][ch] = vp[ch];
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // ---- online softmax per head -----------------------------------------
        float mx = z[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) mx = fmaxf(mx, z[j]);
        mx = xor32_max(xor16_max(mx));
        // lazy reference: it moves only when a logit exceeds it by more than 8
        // (a factor 256), so the weights stay <= 256 and rescaling the
        // accumulators is rare; the normalised result does not depend on it
        const bool grow = mx > m_run + 8.f;  // any finite mx while m_run = -inf
        if (__ballot(grow)) {
            const float m_new = grow ? mx : m_run;
            const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;  // 0 from -inf
#pragma unroll
            for (int db = 0; db < NDB; ++db) o[db] *= alpha;
            l_run *= alpha;
            m_run = m_new;
        }
        const float m_ref = m_run == -INFINITY ? 0.f : m_run;
        float p[8];
        float ps = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            p[j] = __builtin_amdgcn_exp2f(z[j] - m_ref);  // z - m_ref <= 8; -inf gives 0
            ps += p[j];
        }
        l_run += ps;
        // P^T fragment: column = head c, slots 8g..8g+7
        uint4 pf[NCP];
        if constexpr (EB == 2) {
            pf[0] = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                               pack_bf16x2(p[6], p[7]));
        } else {
            pf[0] = make_uint4(__float_as_uint(p[0]), __float_as_uint(p[1]), __float_as_uint(p[2]), __float_as_uint(p[3]));
            pf[1] = make_uint4(__float_as_uint(p[4]), __float_as_uint(p[5]), __float_as_uint(p[6]), __float_as_uint(p[7]));
        }
        mid();
        // ---- O^T[d][head] += V^T[d][slots] P^T[slots][head] -------------------
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int ch = 0; ch < NCP; ++ch) o[db] = mma_chunk(vb[db][ch], pf[ch], o[db]);
        }
    };
    // bf16 pipeline pieces: a wave's partial logits of one tile (its
    // reduction dims), and the rest of a tile once the full logits are known
    auto logits_partial = [&](const unsigned char* ct, v4f& acc0, v4f& acc1) {
        uint4 ca[NCQ], cb[NCQ];
#pragma unroll
        for (int ch = 0; ch < NCQ; ++ch) {
            ca[ch] = *reinterpret_cast<const uint4*>(ct + qoff[ch]);
            cb[ch] = *reinterpret_cast<const uint4*>(ct + qoff[ch] + 4 * CSTR);
        }
        acc0 = v4f{0.f, 0.f, 0.f, 0.f};
        acc1 = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ch = 0; ch < NCQ; ++ch) {
            acc0 = mma_chunk(ca[ch], qf[ch], acc0);
            acc1 = mma_chunk(cb[ch], qf[ch], acc1);
        }
    };
    auto finish_tile = [&](uint32_t tm, const unsigned char* ct, const v4f& acc0, const v4f& acc1) {
        // unscaled logits: the scale (positive) is applied inside the
        // exponent, and the maximum commutes with it; invalid slots -inf
        // (wave-uniform test: only partial tiles have any)
        float z[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            z[r] = acc0[r];
            z[4 + r] = acc1[r];
        }
        if (tm != 0xffffffffu) {
            const uint32_t tmg = tm >> (8 * g);
#pragma unroll
            for (int j = 0; j < 8; ++j) z[j] = (tmg >> j) & 1u ? z[j] : -INFINITY;
        }
        uint4 vb[NDB];
        if constexpr (EB == 2) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const unsigned char* tp = ct + poff[db & 7] + 256 * (db >> 3);
                const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)tp);
                const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(tp + 4 * CSTR));
                const uint2 x = __builtin_bit_cast(uint2, lo), y = __builtin_bit_cast(uint2, hi);
                vb[db] = make_uint4(x.x, x.y, y.x, y.y);
            }
        }
        float mx = z[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) mx = fmaxf(mx, z[j]);
        mx = xor32_max(xor16_max(mx)) * a.scale_log2;
        const bool grow = mx > m_run + 8.f;
        if (__ballot(grow)) {
            const float m_new = grow ? mx : m_run;
            const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
#pragma unroll
            for (int db = 0; db < NDB; ++db) o[db] *= alpha;
            l_run *= alpha;
            m_run = m_new;
        }
        const float nref = m_run == -INFINITY ? 0.f : -m_run;
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) p[j] = __builtin_amdgcn_exp2f(fmaf(z[j], a.scale_log2, nref));  // <= 2^8; -inf gives 0
        float ps = p[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) ps += p[j];
        l_run += ps;
        const uint4 pf = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                                    pack_bf16x2(p[6], p[7]));
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db] = mma_chunk(vb[db], pf, o[db]);
    };
    auto none = [] {};
    if constexpr (NBUF == 1) {
        // one buffer: compute, then store the next tile
        Pre P;
        if (ntl > 0) {
            load_tile(tlist[0], P);
            store_tile(P, ctile[0]);
        }
        __syncthreads();
        for (int ti = 0; ti < ntl; ++ti) {
            load_tile(tlist[min(ti + 1, ntl - 1)], P);
            asm volatile("" ::: "memory");
            compute(lmask[ti], ctile[0], 0, none, none, none);
            __syncthreads();
            if (ti + 1 >= ntl) break;
            store_tile(P, ctile[0]);
            __syncthreads();
        }
    } else {
        // bf16: the tile's 36 KB go from global memory into LDS by the direct
        // global->LDS load, 1 KB (64 lanes x 16 bytes) per instruction, M0 the
        // block's LDS address; wave w loads blocks w, w+NW, ... < 36.  Lane l
        // of block b fills tile byte 1024b + 16l, i.e. row r = (64b + l)/72,
        // stored chunk (64b + l) % 72, whose source is the entry's chunk
        // under the inverse swizzle (the XOR is its own inverse).  The loads
        // are inline asm: the compiler neither waits for them before
        // unrelated LDS reads nor counts them; the waits below (vmcnt, then
        // the exchange barrier) make a tile visible before any wave reads it.
        // Tile k sits in buffer k % 3; tile k+2 is issued right after the
        // barrier of tile k, into the buffer tile k-1 left (whose last reads,
        // the transpose loads of tile k-1, preceded that barrier), and has
        // landed by the barrier of tile k+1.  An invalid slot reads entry 0 of
        // the row's sequence (in bounds); its logit is masked to -inf.
        constexpr int NBLK = AT_TS * CROW / 1024;  // 36
        constexpr int DPW = (NBLK + NW - 1) / NW;  // blocks per wave: 5 (8 waves), 9 (4 waves)
        const int nblk = (NBLK - w + NW - 1) / NW;  // DPW or DPW - 1
        int drow[DPW], doff[DPW];
#pragma unroll
        for (int i = 0; i < DPW; ++i) {
            const int p = min(64 * (w + NW * i) + l, AT_TS * (CROW / 16) - 1);
            const int r = p / (CROW / 16), kk = p % (CROW / 16);
            const int f = ((r >> 3) << 2) | (r & 3);
            drow[i] = r;
            doff[i] = 16 * (kk < 64 ? ((kk & ~15) | ((kk ^ f) & 15)) : (64 | ((kk ^ (f >> 1)) & 7)));
        }
        const uint32_t ct_lds = (uint32_t)(uintptr_t)(lds_uc*)&ctile[0][0];
        // the entries of this thread's gather rows, read one interval before
        // the gather is issued
        int dpos[DPW];
        auto fetch_pos = [&](int t) {
            const int* sl = slots + t * AT_TS;
#pragma unroll
            for (int i = 0; i < DPW; ++i) dpos[i] = sl[drow[i]];
        };
        // Addresses: the sequence's first entry in a scalar base register and
        // a 32-bit byte offset (one 24-bit multiply-add) when its entries
        // span less than 4 GiB (wave-uniform; up to 3.7M entries of 1152
        // bytes), else full 64-bit addresses.
        const bool off32 = (int64_t)(limit + 1) * CROW <= (int64_t)0xFFFFFFFF;
        auto issue_dma = [&](int buf) {
            const uint32_t B = ct_lds + buf * CTB;
            if (off32) {
#pragma unroll
                for (int i = 0; i < DPW; ++i) {
                    if (i == DPW - 1 && nblk < DPW) break;
                    const uint32_t vo = __umul24((uint32_t)dpos[i], (uint32_t)CROW) + (uint32_t)doff[i];
                    const uint32_t m0v = B + 1024 * (w + NW * i);
                    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                                 :
                                 : "s"(m0v), "v"(vo), "s"(kvrow)
                                 : "memory");
                }
            } else {
#pragma unroll
                for (int i = 0; i < DPW; ++i) {
                    if (i == DPW - 1 && nblk < DPW) break;
                    const uint64_t a64 = (uint64_t)(uintptr_t)(kvrow + (size_t)dpos[i] * CROW + doff[i]);
                    const uint32_t m0v = B + 1024 * (w + NW * i);
                    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                                 :
                                 : "s"(m0v), "v"(a64)
                                 : "memory");
                }
            }
        };
        if (ntl > 0) {
            fetch_pos(tlist[0]);
            issue_dma(0);
            if (ntl > 1) {
                fetch_pos(tlist[1]);
                issue_dma(1);
                // tile 0 landed; tile 1 (this wave's last DPW or DPW - 1
                // loads) may be in flight
                if (nblk == DPW)
                    __builtin_amdgcn_s_waitcnt(0xF70 | DPW);  // vmcnt(DPW)
                else
                    __builtin_amdgcn_s_waitcnt(0xF70 | (DPW - 1));
            } else {
                __builtin_amdgcn_s_waitcnt(0xF70);      // vmcnt(0)
            }
            __syncthreads();
            // Software-pipelined tiles: interval ti (between two barriers) takes
            // the partner's partial logits of tile ti, issues tile ti+1's logit
            // fragment reads and products, and then runs tile ti's softmax and
            // P.V while those products are on the matrix cores; it ends by
            // publishing tile ti+1's partial logits.  Tile ti+2 is gathered
            // during interval ti into the buffer tile ti-1 left (its last
            // reads, the V^T of tile ti-1, came before this interval's first
            // barrier) and has landed by the barrier that closes it.  The
            // positions of a gather are read one interval earlier, and the
            // list entry of the tile after it one more interval ahead, so that
            // no LDS round trip precedes the gather's issue.
            if (ntl > 2) fetch_pos(tlist[2]);
            int tl3 = tlist[min(3, ntl - 1)];
            v4f a0, a1;  // this wave's partial logits of the current tile
            logits_partial(ctile[0], a0, a1);
            zx0[0][tid] = make_float4(a0[0], a0[1], a0[2], a0[3]);
            zx1[0][tid] = make_float4(a1[0], a1[1], a1[2], a1[3]);
            __builtin_amdgcn_s_waitcnt(0xF70);  // tile 1 landed
            __syncthreads();
            int cur = 0;
            // one interval; the exchange parity is a compile-time constant (the
            // loop runs two intervals per iteration), so the exchange addresses
            // are immediate offsets and the partial logits need no copies
            auto interval = [&](int ti, auto parc, v4f& c0, v4f& c1, v4f& n0, v4f& n1) {
                constexpr int par = decltype(parc)::value;
                const bool more2 = ti + 2 < ntl;
                const int nx1 = cur == 2 ? 0 : cur + 1, nx2 = nx1 == 2 ? 0 : nx1 + 1;
                if (more2) issue_dma(nx2);
                const uint32_t tm = lmask[ti];
                const float4 q0 = zx0[par][tid ^ 64], q1 = zx1[par][tid ^ 64];
                // positions of tile ti+3 (past the end: the last tile's, unused),
                // read ahead of the fragments so that their waits cover them
                fetch_pos(tl3);
                tl3 = tlist[min(ti + 4, ntl - 1)];
                // tile ti+1: partial logits (independent of tile ti's softmax)
                // (after the last tile: products over a stale buffer, unused)
                logits_partial(ctile[nx1], n0, n1);
                __builtin_amdgcn_sched_barrier(0);
                c0[0] += q0.x; c0[1] += q0.y; c0[2] += q0.z; c0[3] += q0.w;
                c1[0] += q1.x; c1[1] += q1.y; c1[2] += q1.z; c1[3] += q1.w;
                finish_tile(tm, ctile[cur], c0, c1);
                zx0[par ^ 1][tid] = make_float4(n0[0], n0[1], n0[2], n0[3]);
                zx1[par ^ 1][tid] = make_float4(n1[0], n1[1], n1[2], n1[3]);
                __builtin_amdgcn_s_waitcnt(0xF70);  // tile ti+2 landed
                __syncthreads();
                cur = nx1;
            };
            v4f b0, b1;  // partial logits of the odd tiles
            for (int ti = 0; ti < ntl; ti += 2) {
                interval(ti, std::integral_constant<int, 0>{}, a0, a1, b0, b1);
                if (ti + 1 >= ntl) break;
                interval(ti + 1, std::integral_constant<int, 1>{}, b0, b1, a0, a1);
            }
        }
    }

    // ---- finish --------------------------------------------------------------
    const float l_tot = xor32_sum(xor16_sum(l_run));
    if (!hvalid) return;
    if (a.part_o) {
        // split: unnormalised partials of this wave's value dims
        const size_t pidx = (size_t)rs * a.H + h;
        float* po = a.part_o + pidx * DV + half * DVW;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
            *reinterpret_cast<float4*>(po + 16 * db + 4 * g) = make_float4(o[db][0], o[db][1], o[db][2], o[db][3]);
        if (g == 0 && half == 0) {
            a.part_ml[pidx * 2] = m_run;
            a.part_ml[pidx * 2 + 1] = l_tot;
        }
        return;
    }
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    unsigned char* op = a.out + (((size_t)qrow * a.H + h) * DV + half * DVW) * EB;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        const int d0 = 16 * db + 4 * g;
        if constexpr (EB == 2) {
            uint2 pk = make_uint2(pack_bf16x2(o[db][0] * inv, o[db][1] * inv), pack_bf16x2(o[db][2] * inv, o[db][3] * inv));
            *reinterpret_cast<uint2*>(op + d0 * 2) = pk;
        } else {
            *reinterpret_cast<float4*>(op + d0 * 4) = make_float4(o[db][0] * inv, o[db][1] * inv, o[db][2] * inv, o[db][3] * inv);
        }
    }
    if (a.lse && g == 0 && half == 0)
        a.lse[(size_t)qrow * a.H + h] = l_tot > 0.f ? (m_run + log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
}

// Merge the split partials of a decode row: o = sum_s 2^(m_s-M) o_s / sum_s 2^(m_s-M) l_s.
// One wave per (row, head), CB_NT/64 heads per workgroup; lane l owns value
// dims [l*DV/64, (l+1)*DV/64) (16-byte loads and stores).
constexpr int CB_NT = 256;

template <int DT, int DV>
__global__ __launch_bounds__(CB_NT) void attn_combine_kernel(const float* part_o, const float* part_ml, int rows, int H,
                                                             int nsplit, unsigned char* out, float* lse) {
    constexpr int EB = ElemBytes<DT>::v;
    constexpr int PER = DV / 64;
    static_assert(DV % 64 == 0 && (PER < 4 || PER % 4 == 0), "whole dims (or float4 groups) per lane");
    constexpr int VW = PER >= 4 ? 4 : 1;  // floats per load
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = lane_id();
    const int rh = blockIdx.x * (CB_NT / 64) + wv;  // row * H + head
    if (rh >= rows * H) return;
    const int row = rh / H, h = rh - row * H;
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
            const float* po = part_o + pidx * DV + l * PER;
#pragma unroll
            for (int j = 0; j < PER; j += VW) {
                if constexpr (VW == 4) {
                    const float4 v = *reinterpret_cast<const float4*>(po + j);
                    acc[j] += f * v.x;
                    acc[j + 1] += f * v.y;
                    acc[j + 2] += f * v.z;
                    acc[j + 3] += f * v.w;
                } else {
                    acc[j] += f * po[j];
                }
            }
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    unsigned char* op = out + (((size_t)row * H + h) * DV + l * PER) * EB;
#pragma unroll
    for (int j = 0; j < PER; j += VW) {
        if constexpr (VW == 4 && EB == 2)
            *reinterpret_cast<uint2*>(op + 2 * j) = make_uint2(pack_bf16x2(acc[j] * inv, acc[j + 1] * inv),
                                                               pack_bf16x2(acc[j + 2] * inv, acc[j + 3] * inv));
        else if constexpr (VW == 4)
            *reinterpret_cast<float4*>(op + 4 * j) =
                make_float4(acc[j] * inv, acc[j + 1] * inv, acc[j + 2] * inv, acc[j + 3] * inv);
        else if constexpr (EB == 2)
            reinterpret_cast<uint16_t*>(op)[j] = f32_to_bf16_rne(acc[j] * inv);
        else
            reinterpret_cast<float*>(op)[j] = acc[j] * inv;
    }
    if (lse && l == 0) lse[(size_t)row * H + h] = L > 0.f ? (M + log2f(L)) * 0.6931471805599453f : -INFINITY;
}

// ---------------------------------------------------------------------------
template <int DT, int HBW, int DSPLIT, int DQK, int DV, bool DEC>
static void launch_attn_t(AttnArgs a, int rows, hipStream_t st) {
    constexpr int HPW = 16 * HBW;
    const int hg = (a.H + HPW - 1) / HPW;
    a.rows = rows;
    const int grid = hg == 1 ? rows : (rows + 7) / 8 * 8 * hg;
    TLSL_TIMED_LAUNCH("sparse_attn_kernel", st,
                      hipLaunchKernelGGL((sparse_attn_kernel<DT, HBW, DSPLIT, DQK, DV, DEC>), dim3(grid),
                                         dim3(HBW * DSPLIT * 64), 0, st, a));
}

template <bool DEC>
static void dispatch_attn(const AttnShape& s, const AttnArgs& a, int rows, hipStream_t st) {
    if (s.dt == kBF16)
        launch_attn_t<kBF16, 4, 2, 576, 512, DEC>(a, rows, st);
    else
        launch_attn_t<kF32, 1, 1, 80, 64, DEC>(a, rows, st);
}

// S[row, i] = i for i <= t, -1 above: the selection TopK(min(k, t+1)) makes
// when every row keeps all of its history (t + 1 <= k)
__global__ __launch_bounds__(256) void fill_all_history_kernel(int32_t* S, int n, int k, size_t total) {
    for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (size_t)gridDim.x * 256) {
        const int i = (int)(e % k);
        const int t = (int)((e / k) % n);
        S[e] = i <= t ? i : -1;
    }
}

hipError_t launch_fill_all_history(int32_t* S, int B, int n, int k, hipStream_t st) {
    const size_t total = (size_t)B * n * k;
    const int grid = (int)std::min<size_t>((total + 255) / 256, (size_t)device_cu_count() * 8);
    TLSL_TIMED_LAUNCH("fill_all_history_kernel", st,
                      hipLaunchKernelGGL(fill_all_history_kernel, dim3(grid), dim3(256), 0, st, S, n, k, total));
    return hipGetLastError();
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
    const int ns = attn_decode_splits(s, B, k);
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
        const int grid = (B * s.H + CB_NT / 64 - 1) / (CB_NT / 64);
        if (s.dt == kBF16)
            TLSL_TIMED_LAUNCH("attn_combine_kernel", st,
                              hipLaunchKernelGGL((attn_combine_kernel<kBF16, 512>), dim3(grid), dim3(CB_NT), 0, st,
                                                 a.part_o, a.part_ml, B, s.H, ns, a.out, lse));
        else
            TLSL_TIMED_LAUNCH("attn_combine_kernel", st,
                              hipLaunchKernelGGL((attn_combine_kernel<kF32, 64>), dim3(grid), dim3(CB_NT), 0, st,
                                                 a.part_o, a.part_ml, B, s.H, ns, a.out, lse));
    }
    return hipGetLastError();
}

}  // namespace tlsl
