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
 *  - Results are bitwise reproducible for identical inputs and shapes (the
 *    one exception, indexer_loss_grad's dk, says so below).
 *  - fp8 means OCP e4m3 (e4m3fn: bias 7, max 448, no infinities), the format
 *    gfx950's matrix cores take, with one fp32 scale per token: a value is
 *    scale * code.  Scales must be finite and > 0: the kernels take them out
 *    of the ReLU and the head sum (w is multiplied by the query's scale, the
 *    head-summed score by the key's), which equals ReLU(scale_q * scale_k *
 *    q.k) only for positive scales.  The scales live in device memory and are
 *    not checked; a zero, negative or non-finite scale gives unspecified
 *    scores.
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
 * index_prefill_rerank -- coarse recall at fp8, then a high-precision re-rank
 * (DSA page, section 2, the paragraph on the quantised key cache: fp8 shifts
 * the order near the selection boundary; recall a larger candidate set, then
 * rank it with a higher-precision indexer).  For every row t:
 *     C_t = TopK over the fp8 inputs' scores, budget min(k_coarse, t+1)
 *           (index_prefill on qI8/kI8 with their scales)
 *     S_t = the min(k, |C_t|) best of C_t by the scores of the bf16 inputs
 *           qI/kI (eq.(1), the same weights wI), ties to the lower position,
 *           written in ascending position order, then -1.
 * With k_coarse >= n this is index_prefill on the bf16 inputs, bit for bit;
 * with k_coarse = k it keeps C_t.
 *
 *   qI8 [B,n,HI,dI] fp8 + q_scale [B,n];  kI8 [B,n,dI] fp8 + k_scale [B,n]
 *   qI  [B,n,HI,dI] bf16;  kI [B,n,dI] bf16;  wI [B,n,HI] fp32
 *   S [B,n,k] int32 out; S_score [B,n,k] fp32 out (optional): the bf16 scores
 *   C [B,n,k_coarse] int32 out (optional): the candidates; when NULL they are
 *     kept in the workspace
 *   workspace: query protocol (index_prefill's for k_coarse, plus C if NULL).
 * Supported: dI = 128, 1 <= HI <= 64, 1 <= k <= k_coarse <= 4096.
 */
int index_prefill_rerank(const void* qI8, const float* q_scale, const void* kI8,
                         const float* k_scale, const void* qI, const void* kI, const float* wI,
                         int B, int n, int HI, int dI, int k, int k_coarse, int32_t* S,
                         float* S_score, int32_t* C, void* workspace, size_t* ws_bytes,
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
 *   max_len    should be >= every L_b (host value; it sizes the launch and
 *              any staging; a longer sequence is still scored in full, only
 *              more slowly)
 *   scores     [sumL] fp32 out, packed like the cache
 * Supported shapes as index_prefill; L_b < 2^31 - 2^12.  Sequences with
 * L_b = 0 are skipped.
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
 *   max_len   should be >= every row_len (host value; it sizes the launch;
 *             a longer row is still selected exactly, only more slowly)
 *   S         [R,k] int32 out, S_score [R,k] fp32 out (optional)
 *   workspace about R*(2k+264)*8 bytes (query protocol above)
 * Supported: 1 <= k <= 4096, 0 <= row_len < 2^31 - 2^12.
 */
int topk_select(const float* scores, const int64_t* row_start, const int32_t* row_len, int R,
                int k, int max_len, int32_t* S, float* S_score, void* workspace,
                size_t* ws_bytes, hipStream_t stream);

/*
 * topk_select_noalloc -- topk_select for callers that cannot allocate memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, with the workspace taken from a
 * fixed device array inside the library instead of a caller's buffer.  The
 * call itself allocates nothing and clears nothing (every scratch byte it
 * reads is written earlier in the same call).
 *
 * Arguments as topk_select.  The scratch array holds TLSL_NOALLOC_SCRATCH_BYTES
 * bytes on each device the library runs on, from the first call on that device
 * until the process ends; a problem needing more (topk_select's queried
 * workspace size, about R*(2k+264)*8 bytes, e.g. more than ~480 rows at
 * k = 2048) returns TLSL_ERR_WORKSPACE without launching.  Calls that overlap
 * on one device (two streams, two threads) share the array and race: the
 * caller orders them.
 */
#define TLSL_NOALLOC_SCRATCH_BYTES (16u << 20)
int topk_select_noalloc(const float* scores, const int64_t* row_start, const int32_t* row_len, int R,
                        int k, int max_len, int32_t* S, float* S_score, hipStream_t stream);

/*
 * indexer_loss_grad -- one step of the indexer's sparse-stage training: the
 * loss of the DSA page, section 1.2 eq.(8), and its gradient.  For every row
 * (b, t) the valid slots i of S[b,t,:] (0 <= S[b,t,i] <= t) form S_t and
 *     I_i  = sum_j w[b,t,j] * ReLU(q[b,t,j,:] . k[b,S[b,t,i],:])   (eq.(1))
 *     P_i  = p[b,t,i] / sum_{valid} p[b,t,.]     (the teacher renormalised by
 *            its kept mass, as the page requires after eq.(8))
 *     R_i  = exp(I_i) / sum_{valid} exp(I)       (Softmax over S_t)
 *     loss[b,t] = sum_{valid} P_i (log P_i - log R_i),   0 log 0 = 0.
 * The indexer inputs are detached from the main model (section 1.2), so the
 * gradient of sum_{b,t} loss[b,t] is taken with respect to them only, with
 * ReLU'(0) = 0:
 *     dq [B,n,HI,dI], dw [B,n,HI]: per row;
 *     dk [B,n,dI]: summed over every query that selected the key (the call
 *         overwrites dk; keys no query selected get 0).
 * A row with no valid slot, or whose teacher has no mass on them, has loss 0
 * and contributes no gradient.  S is typically index_prefill's output and p
 * the main attention's probabilities on those slots summed over heads; any
 * p >= 0 is accepted.
 *
 *   qI [B,n,HI,dI] bf16, kI [B,n,dI] bf16, wI [B,n,HI] fp32,
 *   S [B,n,k] int32, p [B,n,k] fp32; outputs fp32.
 * Supported: dt = BF16 with dI = 128, 1 <= HI <= 64, 1 <= k <= 4096,
 * n < 2^22, B*n <= 2^30 (else TLSL_ERR_UNSUPPORTED / TLSL_ERR_SHAPE).  Scores, softmax and products accumulate in fp32 (the
 * coefficients of the backward products carry ~16 significant bits).  loss,
 * dq and dw are bitwise reproducible; dk is accumulated with atomic adds, so
 * its last bits may vary between runs.  Needs no workspace.
 */
int indexer_loss_grad(const void* qI, const void* kI, const float* wI, const int32_t* S,
                      const float* p, int B, int n, int HI, int dI, int k, tlsl_dtype dt,
                      float* loss, float* dq, float* dk, float* dw, hipStream_t stream);

/*
 * selection_quality -- how much of a teacher distribution each row's
 * selection covers (DSA page, section 1.2 eq.(9); section 3.1 eq.(14), (15)).
 * Row r of `teacher` holds masses a_0..a_{L-1} (L = row_len[r], at
 * row_start[r]; >= 0, not necessarily normalised), e.g. the main attention's
 * probabilities summed over heads.  With G = TopK(a, min(m, L)) by the rule of
 * eq.(2) (ties to the lower position):
 *     recall[r] = |G n S_r| / |G|          eq.(9); eq.(14) is m = k
 *     mass[r]   = sum_{s in S_r} a_s / sum_{s < L} a_s        eq.(15)
 * NaN where |G| = 0 or the row's total is not positive.
 *
 *   teacher, row_start, row_len, R, max_len: as topk_select's scores rows
 *   S      [R,k] int32 row-relative selections in the library's layout
 *          (ascending positions, then -1); positions >= L are ignored
 *   m      1..4096;  recall, mass [R] fp32 out
 *   workspace: query protocol (the teacher's top-m and topk_select's).
 * Sums run in fp64 (mass is the fp64 ratio rounded once to fp32).
 */
int selection_quality(const float* teacher, const int64_t* row_start, const int32_t* row_len,
                      int R, const int32_t* S, int k, int m, int max_len, float* recall,
                      float* mass, void* workspace, size_t* ws_bytes, hipStream_t stream);

/*
 * cutoff_margin -- the cutoff margin of each score row (DSA page, section 3.1
 * eq.(18)): margin[r] = s_(K) - s_(K+1), K = min(k, L), s_(1) >= s_(2) >= ...
 * the row's scores in descending order; +inf when the row has no (K+1)-th
 * score (L <= k).  A small margin means a small perturbation of the scores
 * (fp8 quantisation, rounding) can swap the selection's boundary keys.
 *
 *   scores, row_start, row_len, R, max_len: as topk_select
 *   margin [R] fp32 out (the fp32 difference of the two scores, rounded once)
 * Supported: 1 <= k <= 4095.  Workspace: query protocol.
 */
int cutoff_margin(const float* scores, const int64_t* row_start, const int32_t* row_len, int R,
                  int k, int max_len, float* margin, void* workspace, size_t* ws_bytes,
                  hipStream_t stream);

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
 * dsa_prefill -- the whole prefill path with the choice of kernels made by
 * length: the DSA page, section 2 (the short-prefill paragraph), notes that
 * for short sequences the top-k, index materialisation and gather cost more
 * than they save and that serving should pick the path by length and batch.
 * When n <= k, TopK(min(k, t+1)) (section 1.1 eq.(2)) keeps every position of
 * every row, so the indexer is skipped and the causal attention over all
 * history runs directly (dense_attn_prefill's path); otherwise index_prefill
 * and sparse_attn_prefill run back to back.  Both paths give the result of
 * the two-call sequence bit for bit (the same attention kernel and slot
 * order).
 *
 *   indexer inputs as index_prefill (qI, q_scale, kI, k_scale, wI, HI, dI,
 *   idx_dt); attention inputs as sparse_attn_prefill (q, kv, H, Dqk, Dv,
 *   softmax_scale, attn_dt); B, n, k.
 *   S    [B,n,k] int32 out, optional: the selection (on the dense path
 *        0..t then -1); when NULL the sparse path keeps it in the workspace
 *   out  [B,n,H,Dv], lse [B,n,H] (optional)
 *   workspace: query protocol; on the sparse path index_prefill's workspace
 *   (plus S when S is NULL), on the dense path 256 bytes.
 * Supported shapes: those of index_prefill and sparse_attn_prefill.
 */
int dsa_prefill(const void* qI, const float* q_scale, const void* kI, const float* k_scale,
                const float* wI, int HI, int dI, tlsl_dtype idx_dt, const void* q, const void* kv,
                int H, int Dqk, int Dv, float softmax_scale, tlsl_dtype attn_dt, int B, int n,
                int k, int32_t* S, void* out, float* lse, void* workspace, size_t* ws_bytes,
                hipStream_t stream);

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

/*
 * tlsl_set_debug -- device checks of the index metadata that callers pass in
 * device memory, which the host-side validation cannot read: on (on != 0),
 * index_decode checks cu_seqlens[0] == 0, sparse_attn_decode and
 * index_decode that cu_seqlens is non-decreasing with every length below
 * 2^31 - 2^12, and topk_select, topk_select_noalloc, selection_quality and
 * cutoff_margin that every row_start >= 0 and 0 <= row_len < 2^31 - 2^12.  A
 * violation returns TLSL_ERR_SHAPE (the message names the first offending
 * entry and its values) and launches nothing else.  Each check is one small
 * kernel followed by a synchronisation of the call's stream, so it is meant
 * for finding malformed batches, not for timed runs or graph capture.  Off
 * by default; the environment variable TLSL_DEBUG (any value but "0") turns
 * it on at the first call.  Returns the previous state (0 or 1).  Process-wide
 * (every thread and device).
 */
int tlsl_set_debug(int on);

#ifdef __cplusplus
}
#endif

#endif /* TLSL_H */
