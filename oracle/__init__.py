"""CPU oracle of the DSA token-selection path -- TEST INFRASTRUCTURE ONLY.

A plain double-precision C implementation (``tlsl_oracle.c``) of the DSA page's
section 1.1 eq.(1) (Lightning Indexer score), eq.(2) (causal top-k) and eq.(3)
(attention over the selected shared latent entries), driven through ctypes on
numpy arrays.  Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import this package; the HIP library never does.

Every function here is pinned by ``tests/test_oracle_pins.py`` against the
page's worked example, closed forms, special cases that reduce to library
routines, invariants and brute force.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tlsl_oracle.c")
_LIB = os.path.join(_HERE, "libtlsl_oracle.so")

F32, BF16, FP8 = 0, 1, 2

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (OpenMP, no fp contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off",
                               "-fno-fast-math", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.ora_decode_fp8_e4m3.restype = ctypes.c_double
        lib.ora_decode_fp8_e4m3.argtypes = [ctypes.c_uint8]
        lib.ora_decode_bf16.restype = ctypes.c_double
        lib.ora_decode_bf16.argtypes = [ctypes.c_uint16]
        lib.ora_topk_rows.argtypes = [P, P, P, I, I, P, P]
        lib.ora_index_prefill_rows.argtypes = [I, P, P, P, P, P, I, I, I, I, I, P, I, P, P, P, P]
        lib.ora_index_decode.argtypes = [I, P, P, P, P, P, P, I, I, I, P, I, P, P]
        lib.ora_sparse_attn_prefill_rows.argtypes = [I, P, P, P, I, I, I, I, I, I,
                                                     ctypes.c_double, P, I, P, P]
        lib.ora_sparse_attn_decode.argtypes = [I, P, P, P, P, I, I, I, I, I, ctypes.c_double,
                                               P, I, P, P]
        lib.ora_sparse_attn_rows.argtypes = [I, P, P, P, P, I, I, I, I, I, ctypes.c_double, P, P]
        lib.ora_indexer_kl.argtypes = [I, P, P, P, P, P, I, I, I, I, I, P, P, P, P, P, P]
        lib.ora_indexer_kl_mag.argtypes = [I, P, P, P, P, P, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P, P]
        lib.ora_selection_quality.argtypes = [P, P, P, I, P, I, I, P, P]
        lib.ora_rerank_rows.argtypes = [I, P, P, P, I, I, I, I, P, I, P, I, I, P, P]
        lib.ora_cutoff_margin.argtypes = [P, P, P, I, I, P]
        lib.ora_num_threads.restype = I
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype=None):
    if a is None:
        return None
    a = np.asarray(a)
    if dtype is not None:
        a = a.astype(dtype, copy=False)
    return np.ascontiguousarray(a)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: bad arguments (rc={rc})")


def num_threads() -> int:
    return _load().ora_num_threads()


def decode_fp8_e4m3(code: int) -> float:
    return _load().ora_decode_fp8_e4m3(int(code))


def decode_bf16(bits: int) -> float:
    return _load().ora_decode_bf16(int(bits))


def topk_rows(scores, row_start, row_len, k):
    """eq.(2) on explicit score rows; returns (S[R,k] int32 row-relative, S_score[R,k])."""
    lib = _load()
    scores = _c(scores, np.float32)
    row_start = _c(row_start, np.int64)
    row_len = _c(row_len, np.int32)
    R = len(row_len)
    S = np.empty((R, k), np.int32)
    Ss = np.empty((R, k), np.float32)
    _check(lib.ora_topk_rows(_ptr(scores), _ptr(row_start), _ptr(row_len), R, k, _ptr(S),
                             _ptr(Ss)), "topk_rows")
    return S, Ss


def index_prefill_rows(dt, q, q_scale, k_in, k_scale, w, k, rows, want_scores=False):
    """eq.(1)+(2) for the listed flattened rows b*n+t of a prefill batch.

    q [B,n,HI,DI], k_in [B,n,DI] storage arrays (f32, bf16 as uint16, fp8 as
    uint8), scales [B,n] f32 or None, w [B,n,HI] f32.  Returns
    (S[nrows,k], S_score[nrows,k], scores[nrows,n] or None, mags[nrows,n] or None).
    """
    lib = _load()
    q = _c(q)
    k_in = _c(k_in)
    w = _c(w, np.float32)
    q_scale = _c(q_scale, np.float32)
    k_scale = _c(k_scale, np.float32)
    B, n, HI, DI = q.shape
    rows = _c(rows, np.int64)
    nr = len(rows)
    S = np.empty((nr, k), np.int32)
    Ss = np.empty((nr, k), np.float32)
    sc = np.empty((nr, n), np.float32) if want_scores else None
    mg = np.empty((nr, n), np.float32) if want_scores else None
    _check(lib.ora_index_prefill_rows(dt, _ptr(q), _ptr(q_scale), _ptr(k_in), _ptr(k_scale),
                                      _ptr(w), B, n, HI, DI, k, _ptr(rows), nr, _ptr(S),
                                      _ptr(Ss), _ptr(sc), _ptr(mg)), "index_prefill_rows")
    return S, Ss, sc, mg


def index_decode(dt, q, q_scale, k_cache, k_scale, w, cu_seqlens, seqs=None):
    """eq.(1) for the newest token of each listed sequence against its cache slice.

    Returns (scores[sumL] f32, mags[sumL] f32); entries of unlisted sequences are NaN.
    """
    lib = _load()
    q = _c(q)
    k_cache = _c(k_cache)
    w = _c(w, np.float32)
    q_scale = _c(q_scale, np.float32)
    k_scale = _c(k_scale, np.float32)
    cu = _c(cu_seqlens, np.int64)
    B, HI, DI = q.shape
    if seqs is None:
        seqs = np.arange(B)
    seqs = _c(seqs, np.int32)
    total = int(cu[-1])
    scores = np.full(total, np.nan, np.float32)
    mags = np.full(total, np.nan, np.float32)
    _check(lib.ora_index_decode(dt, _ptr(q), _ptr(q_scale), _ptr(k_cache), _ptr(k_scale),
                                _ptr(w), _ptr(cu), B, HI, DI, _ptr(seqs), len(seqs),
                                _ptr(scores), _ptr(mags)), "index_decode")
    return scores, mags


def sparse_attn_prefill_rows(dt, q, kv, S, scale, rows, Dv):
    """eq.(3) for the listed flattened rows; returns (out[nrows,H,Dv] f64, lse[nrows,H])."""
    lib = _load()
    q = _c(q)
    kv = _c(kv)
    S = _c(S, np.int32)
    B, n, H, Dqk = q.shape
    k = S.shape[-1]
    rows = _c(rows, np.int64)
    nr = len(rows)
    out = np.empty((nr, H, Dv), np.float64)
    lse = np.empty((nr, H), np.float64)
    _check(lib.ora_sparse_attn_prefill_rows(dt, _ptr(q), _ptr(kv), _ptr(S), B, n, H, Dqk, Dv,
                                            k, float(scale), _ptr(rows), nr, _ptr(out),
                                            _ptr(lse)), "sparse_attn_prefill_rows")
    return out, lse


def sparse_attn_decode(dt, q, kv, cu_seqlens, S, scale, Dv, seqs=None):
    """eq.(3) for the newest token of each listed sequence; S is [B,k] row-relative."""
    lib = _load()
    q = _c(q)
    kv = _c(kv)
    S = _c(S, np.int32)
    cu = _c(cu_seqlens, np.int64)
    B, H, Dqk = q.shape
    k = S.shape[-1]
    if seqs is None:
        seqs = np.arange(B)
    seqs = _c(seqs, np.int32)
    out = np.empty((len(seqs), H, Dv), np.float64)
    lse = np.empty((len(seqs), H), np.float64)
    _check(lib.ora_sparse_attn_decode(dt, _ptr(q), _ptr(kv), _ptr(cu), _ptr(S), B, H, Dqk, Dv,
                                      k, float(scale), _ptr(seqs), len(seqs), _ptr(out),
                                      _ptr(lse)), "sparse_attn_decode")
    return out, lse


def sparse_attn_rows(dt, q_rows, kv, S_rows, limits, scale, Dv):
    """eq.(3) for query rows given one by one: q_rows [R,H,Dqk], their slots
    S_rows [R,k] into the entries kv [m,Dqk], valid slots 0 <= s <= limits[r].
    Returns (out[R,H,Dv] f64, lse[R,H])."""
    lib = _load()
    q_rows = _c(q_rows)
    kv = _c(kv)
    S_rows = _c(S_rows, np.int32)
    limits = _c(limits, np.int64)
    R, H, Dqk = q_rows.shape
    k = S_rows.shape[-1]
    if S_rows.shape[0] != R or len(limits) != R or kv.shape[-1] != Dqk:
        raise ValueError("oracle sparse_attn_rows: inconsistent shapes")
    out = np.empty((R, H, Dv), np.float64)
    lse = np.empty((R, H), np.float64)
    _check(lib.ora_sparse_attn_rows(dt, _ptr(q_rows), _ptr(kv), _ptr(S_rows), _ptr(limits), R, H, Dqk,
                                    Dv, k, float(scale), _ptr(out), _ptr(lse)), "sparse_attn_rows")
    return out, lse


def indexer_kl(dt, q, q_scale, k_in, k_scale, w, S, p, want_mags=False):
    """Sparse-stage indexer loss (DSA page section 1.2 eq.(8), both sides
    normalised over S_t) and its gradient, for every row of a batch.

    q [B,n,HI,DI], k_in [B,n,DI] storage arrays, scales [B,n] or None,
    w [B,n,HI] f32, S [B,n,k] int32 (slots outside [0,t] are not selected),
    p [B,n,k] f32 teacher masses per slot (normalised over the valid slots).
    Returns (loss [B,n], dq [B,n,HI,DI], dk [B,n,DI], dw [B,n,HI]), float64;
    with ``want_mags`` also their magnitude sums (the same shapes; the sums of
    the terms' absolute values with |g_i| replaced by R_i + P_i) and the kink
    bands of dq and dk (the terms whose dot product lies within fp32
    accumulation rounding of ReLU's kink), which tests use to bound the
    difference of a result computed in fp32.
    """
    lib = _load()
    q = _c(q)
    k_in = _c(k_in)
    w = _c(w, np.float32)
    q_scale = _c(q_scale, np.float32)
    k_scale = _c(k_scale, np.float32)
    S = _c(S, np.int32)
    p = _c(p, np.float32)
    B, n, HI, DI = q.shape
    k = S.shape[-1]
    if S.shape != (B, n, k) or p.shape != (B, n, k) or k_in.shape != (B, n, DI) or w.shape != (B, n, HI):
        raise ValueError("oracle indexer_kl: inconsistent shapes")
    loss = np.empty((B, n), np.float64)
    dq = np.empty((B, n, HI, DI), np.float64)
    dk = np.empty((B, n, DI), np.float64)
    dw = np.empty((B, n, HI), np.float64)
    if not want_mags:
        _check(lib.ora_indexer_kl(dt, _ptr(q), _ptr(q_scale), _ptr(k_in), _ptr(k_scale), _ptr(w), B, n, HI, DI, k,
                                  _ptr(S), _ptr(p), _ptr(loss), _ptr(dq), _ptr(dk), _ptr(dw)), "indexer_kl")
        return loss, dq, dk, dw
    mags = (np.empty_like(loss), np.empty_like(dq), np.empty_like(dk), np.empty_like(dw), np.empty_like(dq),
            np.empty_like(dk))
    _check(lib.ora_indexer_kl_mag(dt, _ptr(q), _ptr(q_scale), _ptr(k_in), _ptr(k_scale), _ptr(w), B, n, HI, DI, k,
                                  _ptr(S), _ptr(p), _ptr(loss), _ptr(dq), _ptr(dk), _ptr(dw), *(_ptr(m) for m in mags)),
           "indexer_kl")
    return (loss, dq, dk, dw) + mags


def selection_quality(teacher, row_start, row_len, S, m):
    """Recall of the teacher's top-m (DSA page eq.(9); eq.(14) is m = k) and
    teacher mass coverage (eq.(15), teacher normalised over the row) of the
    selections S [R,k] (row-relative).  Returns (recall [R], mass [R])."""
    lib = _load()
    teacher = _c(teacher, np.float32)
    row_start = _c(row_start, np.int64)
    row_len = _c(row_len, np.int32)
    S = _c(S, np.int32)
    R, k = S.shape
    recall = np.empty(R, np.float64)
    mass = np.empty(R, np.float64)
    _check(lib.ora_selection_quality(_ptr(teacher), _ptr(row_start), _ptr(row_len), R, _ptr(S), k, int(m),
                                     _ptr(recall), _ptr(mass)), "selection_quality")
    return recall, mass


def cutoff_margin(scores, row_start, row_len, k):
    """Cutoff margin s_(K) - s_(K+1) of each score row (eq.(18)), +inf when
    the row has no (K+1)-th score."""
    lib = _load()
    scores = _c(scores, np.float32)
    row_start = _c(row_start, np.int64)
    row_len = _c(row_len, np.int32)
    R = len(row_len)
    margin = np.empty(R, np.float64)
    _check(lib.ora_cutoff_margin(_ptr(scores), _ptr(row_start), _ptr(row_len), R, int(k), _ptr(margin)),
           "cutoff_margin")
    return margin


def rerank_rows(dt_fine, q, k_in, w, rows, C, k):
    """Re-rank (DSA page section 2, the quantised-cache paragraph): the listed
    rows' candidates C [nrows, kc] (positions; entries outside [0, t] skipped)
    scored with eq.(1) on the fine inputs (f32 or bf16 storage), the min(k,
    #candidates) best by (score desc, position asc), ascending, then -1.
    Returns (S [nrows,k], S_score [nrows,k])."""
    lib = _load()
    q = _c(q)
    k_in = _c(k_in)
    w = _c(w, np.float32)
    rows = _c(rows, np.int64)
    C = _c(C, np.int32)
    B, n, HI, DI = q.shape
    nr, kc = C.shape
    if len(rows) != nr:
        raise ValueError("oracle rerank_rows: one candidate row per listed row")
    S = np.empty((nr, k), np.int32)
    Ss = np.empty((nr, k), np.float32)
    _check(lib.ora_rerank_rows(dt_fine, _ptr(q), _ptr(k_in), _ptr(w), B, n, HI, DI, _ptr(rows), nr, _ptr(C), kc, k,
                               _ptr(S), _ptr(Ss)), "rerank_rows")
    return S, Ss


def index_prefill_rerank_rows(dt_coarse, q_c, q_scale, k_c, k_scale, dt_fine, q_f, k_f, w, k, k_coarse, rows):
    """Coarse recall then re-rank: C = TopK over the coarse inputs' scores with
    budget k_coarse (eq.(1)-(2)), then the k best of C by the fine inputs'
    scores.  Returns (S, S_score, C)."""
    C, _, _, _ = index_prefill_rows(dt_coarse, q_c, q_scale, k_c, k_scale, w, k_coarse, rows)
    S, Ss = rerank_rows(dt_fine, q_f, k_f, w, rows, C, k)
    return S, Ss, C
