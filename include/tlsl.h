/*
 * tlsl.h -- C ABI of the DSA token-selection library for AMD Instinct MI355X
 * (gfx950).
 *
 * The library computes, for every query token t, the Lightning Indexer score
 * of the DSA page ("2.2.1 DSA 与索引器: 先召回 token, 再计算 Sparse MLA"),
 * section 1.1 eq.(1),
 *
 *     I[t,s] = sum_{j < H^I} w[t,j] * ReLU(q[t,j] . k[s]),   0 <= s <= t,
 *
 * keeps S_t = TopK({I[t,s]}, min(k, t+1)) (section 1.1 eq.(2)), and runs
 * softmax attention for all heads over only the gathered shared latent
 * entries c_s, s in S_t (section 1.1 eq.(3), in the weight-absorbed MQA form
 * of section 2 where every head reads the same entry).
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or synchronises.  Layouts are dense row-major with
 *    the last dimension contiguous.  Base pointers must be 16-byte aligned.
 *  - Every call is asynchronous on `stream` (NULL = the null stream).
 *  - Scratch memory comes from the caller.  index_prefill, topk_select and
 *    sparse_attn_decode take a workspace: pass workspace == NULL to query its
 *    size (written to *ws_bytes, nothing is launched, TLSL_OK is returned);
 *    otherwise *ws_bytes must hold the size of `workspace`, at least the
 *    queried size.  A workspace may be reused once the call that used it has
 *    completed on its stream; calls that overlap must not share one.
 *    index_decode, sparse_attn_prefill and dense_attn_prefill need no
 *    workspace:
 *    their workspace argument is ignored, and *ws_bytes (if ws_bytes is not
 *    NULL) receives 0.
 *  - Arguments are validated on the host before anything is launched; a
 *    negative return code means nothing ran and tlsl_last_error() describes
 *    why.  Shapes the library was not built for return TLSL_ERR_UNSUPPORTED;
 *    there is no fallback path.
 *  - Positions are 0-based and include the current token.  A selected row is
 *    written in ascending position order, followed by -1 in the unused slots.
 *    Ties in the score go to the lower position; -0.0 equals +0.0.  NaN or
 *    infinite inputs are not supported.
 *  - Results are bitwise reproducible for identical inputs and shapes.
 *  - fp8 means OCP e4m3 (e4m3fn: bias 7, max 448, no infinities), the format
 *    gfx950's matrix cores take, with one fp32 scale per token: a value is
 *    scale * code.
 */
#ifndef TLSL_H
#define TLSL_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TLSL_F32 = 0,      /* IEEE binary32 */
    TLSL_BF16 = 1,     /* bfloat16 */
    TLSL_FP8_E4M3 = 2  /* OCP e4m3fn + one fp32 scale per token */
} tlsl_dtype;

enum {
    TLSL_OK = 0,
    TLSL_ERR_NULL = -1,        /* a required pointer is NULL */
    TLSL_ERR_SHAPE = -2,       /* a size is out of range or inconsistent */
    TLSL_ERR_UNSUPPORTED = -3, /* dtype/shape combination not built */
    TLSL_ERR_WORKSPACE = -4,   /* workspace smaller than required */
    TLSL_ERR_HIP = -5,         /* the HIP runtime reported an error at launch */
    TLSL_ERR_ALIGN = -6        /* a pointer is not 16-byte aligned */
};

/*
 * index_prefill -- Lightning Indexer plus causal top-k for a prefill batch
 * (DSA page, section 1.1 eq.(1) and eq.(2); the tensors Q^I, K^I, W^I and S of
 * the paragraph after eq.(1)).  The B x n x n score matrix is never stored.
 *
 *   qI      [B,n,HI,dI]  dtype dt
 *   q_scale [B,n] fp32   per-token scale of qI (fp8 only; must be NULL otherwise)
 *   kI      [B,n,dI]     dtype dt, one shared key per token
 *   k_scale [B,n] fp32   per-token scale of kI (fp8 only; NULL otherwise)
 *   wI      [B,n,HI] fp32 per-head weights (may be negative)
 *   k       selection budget; row t keeps min(k, t+1) positions
 *   S       [B,n,k] int32 out: selected positions, ascending, then -1
 *   S_score [B,n,k] fp32 out (optional, may be NULL): I[t, S[t,i]] per slot,
 *           -inf for unused slots
 * Supported: dt=F32 with dI in {32,64}; dt=BF16 with dI in {32,64,128};
 * dt=FP8 with dI=128; 1 <= HI <= 64; 1 <= k <= 4096; B*n <= 2^30.  Scores are
 * accumulated in fp32.
 */
int index_prefill(const void* qI, const float* q_scale, const void* kI, const float* k_scale,
                  const float* wI, int B, int n, int HI, int dI, int k, tlsl_dtype dt,
                  int32_t* S, float* S_score, void* workspace, size_t* ws_bytes,
                  hipStream_t stream);

/*
 * index_decode -- Lightning Indexer score of each sequence's newest token
 * against its whole indexer key cache (DSA page, section 1.1 eq.(1); the decode
 * paragraph of section 2: one new query per step scans all cached K^I, which
 * is bandwidth-bound).  The caller has already appended the new token's key,
 * so sequence b has L_b = cu_seqlens[b+1]-cu_seqlens[b] >= 1 keys and its query
 * sits at position L_b - 1.
 *
 *   qI         [B,HI,dI] dtype dt        newest query of each sequence
 *   q_scale    [B] fp32                  (fp8 only; NULL otherwise)
 *   kI_cache   [sumL,dI] dtype dt        packed caches, sequence b at rows
 *                                        cu_seqlens[b] .. cu_seqlens[b+1]-1
 *   k_scale    [sumL] fp32               (fp8 only; NULL otherwise)
 *   wI         [B,HI] fp32
 *   cu_seqlens [B+1] int64 (device), non-decreasing, cu_seqlens[0] = 0
 *   max_len    >= every L_b (host value; sizes the launch)
 *   scores     [sumL] fp32 out, packed like the cache
 * Supported shapes as index_prefill.  Sequences with L_b = 0 are skipped.
 */
int index_decode(const void* qI, const float* q_scale, const void* kI_cache,
                 const float* k_scale, const float* wI, const int64_t* cu_seqlens, int B,
                 int HI, int dI, int max_len, tlsl_dtype dt, float* scores, void* workspace,
                 size_t* ws_bytes, hipStream_t stream);

/*
 * topk_select -- causal top-k over explicit score rows (DSA page, section 1.1
 * eq.(2); section 2 notes variable-length rows).  Row r is
 * scores[row_start[r] .. row_start[r]+row_len[r]-1]; it keeps
 * min(k, row_len[r]) positions, relative to the row start.
 *
 *   scores    fp32 (device)
 *   row_start [R] int64 (device), row_len [R] int32 (device, >= 0)
 *   max_len   >= every row_len (host value)
 *   S         [R,k] int32 out, S_score [R,k] fp32 out (optional)
 *   workspace about R*(2k+264)*8 bytes (query protocol above)
 * Supported: 1 <= k <= 4096, 0 <= row_len < 2^31.
 */
int topk_select(const float* scores, const int64_t* row_start, const int32_t* row_len, int R,
                int k, int max_len, int32_t* S, float* S_score, void* workspace,
                size_t* ws_bytes, hipStream_t stream);

/*
 * sparse_attn_prefill -- attention of every query over its selected shared
 * latent entries (DSA page, section 1.1 eq.(3); the Sparse MLA paragraph after
 * eq.(1) gathers the latent KV named by S[t,:]).  For query (b,t), head h and
 * valid slots i (0 <= S[b,t,i] <= t; other values are skipped, a repeated
 * position counts once per slot):
 *     z_i = softmax_scale * q[b,t,h,:] . kv[b,S[b,t,i],:]          (all Dqk)
 *     out[b,t,h,:] = sum_i softmax(z)_i * kv[b,S[b,t,i],0:Dv]
 *     lse[b,t,h]   = log sum_i exp(z_i)          (natural log)
 * A row without a valid slot gives out = 0 and lse = -inf.
 *
 *   q   [B,n,H,Dqk] dtype dt,  kv [B,n,Dqk] dtype dt,  S [B,n,k] int32
 *   out [B,n,H,Dv] dtype dt,   lse [B,n,H] fp32 (optional)
 * Supported: dt=BF16 with (Dqk,Dv) = (576,512) (the 512-dim latent plus the
 * 64-dim position part) and 1 <= H <= 128; dt=F32 with (Dqk,Dv) = (80,64) and
 * 1 <= H <= 16; 1 <= k <= 4096 (larger k: TLSL_ERR_UNSUPPORTED).  Products
 * and softmax run in fp32 (bf16 probabilities feed the value product);
 * softmax_scale must be positive and finite.
 */
int sparse_attn_prefill(const void* q, const void* kv, const int32_t* S, int B, int n, int H,
                        int Dqk, int Dv, int k, float softmax_scale, tlsl_dtype dt, void* out,
                        float* lse, void* workspace, size_t* ws_bytes, hipStream_t stream);

/*
 * dense_attn_prefill -- the short-prefill path: causal attention of every
 * query over all of its history.  When t + 1 <= k, TopK(min(k, t+1)) of the
 * DSA page, section 1.1 eq.(2) keeps every position 0..t, so eq.(3) over S_t
 * is plain masked attention; section 2 (the paragraph on short prefill) notes
 * that for short sequences the top-k, index materialisation and gather cost
 * more than the attention they save, and that serving picks the path by
 * length.  A caller with n <= k therefore skips index_prefill and calls this.
 * The result equals sparse_attn_prefill with k = n and S[b,t,i] = i for
 * i <= t (-1 above), bit for bit.
 *
 *   q   [B,n,H,Dqk] dtype dt,  kv [B,n,Dqk] dtype dt
 *   out [B,n,H,Dv] dtype dt,   lse [B,n,H] fp32 (optional)
 * Supported shapes as sparse_attn_prefill, with 1 <= n <= 4096 (longer
 * sequences: TLSL_ERR_UNSUPPORTED).
 */
int dense_attn_prefill(const void* q, const void* kv, int B, int n, int H, int Dqk, int Dv,
                       float softmax_scale, tlsl_dtype dt, void* out, float* lse,
                       void* workspace, size_t* ws_bytes, hipStream_t stream);

/*
 * sparse_attn_decode -- as sparse_attn_prefill for the newest token of each
 * sequence of a ragged decode batch (DSA page, section 2: Sparse MLA reads k
 * latent entries per step, shared by all heads).  S holds row-relative
 * positions; valid slots satisfy 0 <= S[b,i] <= L_b - 1.
 *
 *   q   [B,H,Dqk] dtype dt,  kv_cache [sumL,Dqk] dtype dt,
 *   cu_seqlens [B+1] int64 (device),  S [B,k] int32
 *   out [B,H,Dv] dtype dt,   lse [B,H] fp32 (optional)
 * Supported shapes as sparse_attn_prefill.
 */
int sparse_attn_decode(const void* q, const void* kv_cache, const int64_t* cu_seqlens,
                       const int32_t* S, int B, int H, int Dqk, int Dv, int k,
                       float softmax_scale, tlsl_dtype dt, void* out, float* lse,
                       void* workspace, size_t* ws_bytes, hipStream_t stream);

/* Message for the last non-OK return on the calling thread ("" if none). */
const char* tlsl_last_error(void);

/* Library version string. */
const char* tlsl_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TLSL_H */
