"""ctypes binding of libtlsl.so (the C ABI in include/tlsl.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream, every step of the computation runs in the library's kernels.  There
is no CPU path: if the library is missing the call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtlsl.so")

F32, BF16, FP8_E4M3 = 0, 1, 2

EXPORTS = ("index_prefill", "index_prefill_rerank", "index_decode", "topk_select", "topk_select_noalloc", "sparse_attn_prefill",
           "dense_attn_prefill", "dsa_prefill", "sparse_attn_decode", "indexer_loss_grad", "selection_quality", "cutoff_margin",
           "tlsl_last_error", "tlsl_version", "tlsl_set_debug",
           # measurement aids (include/tlsl_measure.h)
           "tlsl_timer_arm", "tlsl_timer_collect", "tlsl_calib_copy", "tlsl_calib_mfma")

_lib = None


class TlslError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn} failed ({code}): {msg}")
        self.code = code


def load():
    """Load libtlsl.so (built by ``token_level_sparse_lightning_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m token_level_sparse_lightning_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)
    F = ctypes.c_float
    lib.index_prefill.argtypes = [P, P, P, P, P, I, I, I, I, I, I, P, P, P, SZ, P]
    lib.index_decode.argtypes = [P, P, P, P, P, P, I, I, I, I, I, P, P, SZ, P]
    lib.topk_select.argtypes = [P, P, P, I, I, I, P, P, P, SZ, P]
    lib.topk_select_noalloc.argtypes = [P, P, P, I, I, I, P, P, P]
    lib.sparse_attn_prefill.argtypes = [P, P, P, I, I, I, I, I, I, F, I, P, P, P, SZ, P]
    lib.dense_attn_prefill.argtypes = [P, P, I, I, I, I, I, F, I, P, P, P, SZ, P]
    lib.sparse_attn_decode.argtypes = [P, P, P, P, I, I, I, I, I, F, I, P, P, P, SZ, P]
    lib.indexer_loss_grad.argtypes = [P, P, P, P, P, I, I, I, I, I, I, P, P, P, P, P]
    lib.dsa_prefill.argtypes = [P, P, P, P, P, I, I, I, P, P, I, I, I, F, I, I, I, I, P, P, P, P, SZ, P]
    lib.selection_quality.argtypes = [P, P, P, I, P, I, I, I, P, P, P, SZ, P]
    lib.index_prefill_rerank.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, P, P, P, P, SZ, P]
    lib.cutoff_margin.argtypes = [P, P, P, I, I, I, P, P, SZ, P]
    for fn in ("index_prefill", "index_decode", "topk_select", "topk_select_noalloc", "sparse_attn_prefill",
               "dense_attn_prefill",
               "sparse_attn_decode", "indexer_loss_grad", "dsa_prefill", "selection_quality", "cutoff_margin",
               "index_prefill_rerank"):
        getattr(lib, fn).restype = I
    lib.tlsl_last_error.restype = ctypes.c_char_p
    lib.tlsl_version.restype = ctypes.c_char_p
    lib.tlsl_set_debug.argtypes = [I]
    lib.tlsl_set_debug.restype = I
    D = ctypes.POINTER(ctypes.c_double)
    lib.tlsl_timer_arm.argtypes = [ctypes.c_char_p, I]
    lib.tlsl_timer_collect.argtypes = [ctypes.POINTER(I), D, D, D]
    lib.tlsl_calib_copy.argtypes = [P, P, ctypes.c_size_t, P]
    lib.tlsl_calib_mfma.argtypes = [I, I, I, P, D, P]
    for fn in ("tlsl_timer_arm", "tlsl_timer_collect", "tlsl_calib_copy", "tlsl_calib_mfma"):
        getattr(lib, fn).restype = I
    _lib = lib
    return lib


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn, rc):
    if rc != 0:
        raise TlslError(fn, rc, _lib.tlsl_last_error().decode())


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return FP8_E4M3
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def _need(t, name):
    if t is not None and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


# ---------------------------------------------------------------------------
def index_prefill_workspace_bytes(qI, kI, wI, k, q_scale=None, k_scale=None) -> int:
    lib = load()
    B, n, HI, DI = qI.shape
    size = ctypes.c_size_t(0)
    dummy = ctypes.c_void_p(16)  # never dereferenced by a size query
    rc = lib.index_prefill(dummy, dummy if q_scale is not None else None, dummy,
                           dummy if k_scale is not None else None, dummy, B, n, HI, DI, k,
                           dtype_code(qI), dummy, None, None, ctypes.byref(size), None)
    _check("index_prefill", rc)
    return size.value


def index_prefill(qI, kI, wI, k, q_scale=None, k_scale=None, S=None, S_score=None,
                  want_scores=False, workspace=None, stream=None):
    """Lightning Indexer + causal top-k: returns (S [B,n,k] int32, S_score or None)."""
    lib = load()
    for t, nm in ((qI, "qI"), (kI, "kI"), (wI, "wI"), (q_scale, "q_scale"), (k_scale, "k_scale")):
        _need(t, nm)
    B, n, HI, DI = qI.shape
    if S is None:
        S = torch.empty((B, n, k), dtype=torch.int32, device=qI.device)
    if S_score is None and want_scores:
        S_score = torch.empty((B, n, k), dtype=torch.float32, device=qI.device)
    if workspace is None:
        workspace = torch.empty(index_prefill_workspace_bytes(qI, kI, wI, k, q_scale, k_scale),
                                dtype=torch.uint8, device=qI.device)
    size = ctypes.c_size_t(workspace.numel())
    rc = lib.index_prefill(_ptr(qI), _ptr(q_scale), _ptr(kI), _ptr(k_scale), _ptr(wI), B, n, HI,
                           DI, k, dtype_code(qI), _ptr(S), _ptr(S_score), _ptr(workspace),
                           ctypes.byref(size), _stream(stream))
    _check("index_prefill", rc)
    return S, S_score


def index_prefill_rerank(qI8, q_scale, kI8, k_scale, qI, kI, wI, k, k_coarse, S=None, S_score=None,
                         want_scores=False, C=None, want_C=False, workspace=None, stream=None):
    """fp8 coarse recall (budget k_coarse), then the k best candidates by the
    bf16 inputs' scores: returns (S [B,n,k], S_score or None, C or None)."""
    lib = load()
    for t, nm in ((qI8, "qI8"), (kI8, "kI8"), (qI, "qI"), (kI, "kI"), (wI, "wI")):
        _need(t, nm)
    B, n, HI, DI = qI.shape
    dev = qI.device
    if S is None:
        S = torch.empty((B, n, k), dtype=torch.int32, device=dev)
    if S_score is None and want_scores:
        S_score = torch.empty((B, n, k), dtype=torch.float32, device=dev)
    if C is None and want_C:
        C = torch.empty((B, n, k_coarse), dtype=torch.int32, device=dev)
    args = [_ptr(qI8), _ptr(q_scale), _ptr(kI8), _ptr(k_scale), _ptr(qI), _ptr(kI), _ptr(wI), B, n, HI, DI, int(k),
            int(k_coarse), _ptr(S), _ptr(S_score), _ptr(C)]
    _with_workspace("index_prefill_rerank", args, dev, workspace, stream)
    return S, S_score, C


def index_decode(qI, kI_cache, wI, cu_seqlens, max_len, q_scale=None, k_scale=None,
                 scores=None, stream=None):
    """Decode indexer scan: returns scores [sumL] fp32, packed like the cache."""
    lib = load()
    B, HI, DI = qI.shape
    total = kI_cache.shape[0]
    if scores is None:
        scores = torch.empty(total, dtype=torch.float32, device=qI.device)
    rc = lib.index_decode(_ptr(qI), _ptr(q_scale), _ptr(kI_cache), _ptr(k_scale), _ptr(wI),
                          _ptr(cu_seqlens), B, HI, DI, int(max_len), dtype_code(qI), _ptr(scores),
                          None, None, _stream(stream))
    _check("index_decode", rc)
    return scores


def topk_select_workspace_bytes(R, k, max_len) -> int:
    lib = load()
    size = ctypes.c_size_t(0)
    dummy = ctypes.c_void_p(16)
    rc = lib.topk_select(dummy, dummy, dummy, int(R), int(k), int(max_len), dummy, None, None,
                         ctypes.byref(size), None)
    _check("topk_select", rc)
    return size.value


def topk_select(scores, row_start, row_len, k, max_len, S=None, S_score=None, want_scores=False,
                workspace=None, stream=None):
    """Row top-k: returns (S [R,k] int32 row-relative, S_score or None)."""
    lib = load()
    R = row_len.shape[0]
    if S is None:
        S = torch.empty((R, k), dtype=torch.int32, device=scores.device)
    if S_score is None and want_scores:
        S_score = torch.empty((R, k), dtype=torch.float32, device=scores.device)
    if workspace is None:
        workspace = torch.empty(topk_select_workspace_bytes(R, k, max_len), dtype=torch.uint8,
                                device=scores.device)
    size = ctypes.c_size_t(workspace.numel())
    rc = lib.topk_select(_ptr(scores), _ptr(row_start), _ptr(row_len), R, k, int(max_len), _ptr(S),
                         _ptr(S_score), _ptr(workspace), ctypes.byref(size), _stream(stream))
    _check("topk_select", rc)
    return S, S_score


def topk_select_noalloc(scores, row_start, row_len, k, max_len, S=None, S_score=None, want_scores=False,
                        stream=None):
    """topk_select with the library's fixed device scratch instead of a
    workspace (the call allocates nothing; the outputs are the caller's)."""
    lib = load()
    R = row_len.shape[0]
    if S is None:
        S = torch.empty((R, k), dtype=torch.int32, device=scores.device)
    if S_score is None and want_scores:
        S_score = torch.empty((R, k), dtype=torch.float32, device=scores.device)
    rc = lib.topk_select_noalloc(_ptr(scores), _ptr(row_start), _ptr(row_len), R, k, int(max_len), _ptr(S),
                                 _ptr(S_score), _stream(stream))
    _check("topk_select_noalloc", rc)
    return S, S_score


def sparse_attn_prefill(q, kv, S, softmax_scale, Dv, out=None, lse=None, want_lse=False,
                        stream=None):
    """Sparse attention for a prefill batch: returns (out [B,n,H,Dv], lse or None)."""
    lib = load()
    B, n, H, Dqk = q.shape
    k = S.shape[-1]
    if out is None:
        out = torch.empty((B, n, H, Dv), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, n, H), dtype=torch.float32, device=q.device)
    rc = lib.sparse_attn_prefill(_ptr(q), _ptr(kv), _ptr(S), B, n, H, Dqk, Dv, k,
                                 float(softmax_scale), dtype_code(q), _ptr(out), _ptr(lse), None,
                                 None, _stream(stream))
    _check("sparse_attn_prefill", rc)
    return out, lse


def dense_attn_prefill(q, kv, softmax_scale, Dv, out=None, lse=None, want_lse=False, stream=None):
    """Causal attention over all history (short prefill, n <= k): (out [B,n,H,Dv], lse or None)."""
    lib = load()
    B, n, H, Dqk = q.shape
    if out is None:
        out = torch.empty((B, n, H, Dv), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, n, H), dtype=torch.float32, device=q.device)
    rc = lib.dense_attn_prefill(_ptr(q), _ptr(kv), B, n, H, Dqk, Dv, float(softmax_scale),
                                dtype_code(q), _ptr(out), _ptr(lse), None, None, _stream(stream))
    _check("dense_attn_prefill", rc)
    return out, lse


def dsa_prefill(qI, kI, wI, q, kv, k, softmax_scale, Dv, q_scale=None, k_scale=None, S=None, want_S=False,
                out=None, lse=None, want_lse=False, workspace=None, stream=None):
    """The whole prefill path, dense when n <= k (every row keeps all of its
    history), indexer + top-k + sparse attention otherwise:
    returns (out [B,n,H,Dv], lse or None, S or None)."""
    lib = load()
    for t, nm in ((qI, "qI"), (kI, "kI"), (wI, "wI"), (q, "q"), (kv, "kv")):
        _need(t, nm)
    B, n, HI, DI = qI.shape
    H, Dqk = q.shape[2], q.shape[3]
    dev = q.device
    if S is None and want_S:
        S = torch.empty((B, n, k), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty((B, n, H, Dv), dtype=q.dtype, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, n, H), dtype=torch.float32, device=dev)
    args = [_ptr(qI), _ptr(q_scale), _ptr(kI), _ptr(k_scale), _ptr(wI), HI, DI, dtype_code(qI), _ptr(q), _ptr(kv), H,
            Dqk, Dv, float(softmax_scale), dtype_code(q), B, n, k, _ptr(S), _ptr(out), _ptr(lse)]
    if workspace is None:
        size = ctypes.c_size_t(0)
        _check("dsa_prefill", lib.dsa_prefill(*args, None, ctypes.byref(size), None))
        workspace = torch.empty(size.value, dtype=torch.uint8, device=dev)
    size = ctypes.c_size_t(workspace.numel())
    _check("dsa_prefill", lib.dsa_prefill(*args, _ptr(workspace), ctypes.byref(size), _stream(stream)))
    return out, lse, S


def _with_workspace(fn, args, device, workspace, stream):
    """Call a workspace-protocol entry point: size query, then the call."""
    lib = load()
    if workspace is None:
        size = ctypes.c_size_t(0)
        _check(fn, getattr(lib, fn)(*args, None, ctypes.byref(size), None))
        workspace = torch.empty(max(size.value, 1), dtype=torch.uint8, device=device)
    size = ctypes.c_size_t(workspace.numel())
    _check(fn, getattr(lib, fn)(*args, _ptr(workspace), ctypes.byref(size), _stream(stream)))


def selection_quality(teacher, row_start, row_len, S, m, max_len, recall=None, mass=None, workspace=None,
                      stream=None):
    """Recall of the teacher's top-m and teacher mass coverage of the
    selections S [R,k]: returns (recall [R], mass [R]) fp32."""
    R, k = S.shape
    dev = S.device
    recall = torch.empty(R, dtype=torch.float32, device=dev) if recall is None else recall
    mass = torch.empty(R, dtype=torch.float32, device=dev) if mass is None else mass
    _with_workspace("selection_quality", [_ptr(teacher), _ptr(row_start), _ptr(row_len), R, _ptr(S), k, int(m),
                                          int(max_len), _ptr(recall), _ptr(mass)], dev, workspace, stream)
    return recall, mass


def cutoff_margin(scores, row_start, row_len, k, max_len, margin=None, workspace=None, stream=None):
    """Cutoff margin s_(K) - s_(K+1) of each score row: returns margin [R] fp32."""
    R = row_len.shape[0]
    dev = scores.device
    margin = torch.empty(R, dtype=torch.float32, device=dev) if margin is None else margin
    _with_workspace("cutoff_margin", [_ptr(scores), _ptr(row_start), _ptr(row_len), R, int(k), int(max_len),
                                      _ptr(margin)], dev, workspace, stream)
    return margin


def sparse_attn_decode_workspace_bytes(q, kv_cache, S, Dv) -> int:
    lib = load()
    B, H, Dqk = q.shape
    size = ctypes.c_size_t(0)
    dummy = ctypes.c_void_p(16)
    rc = lib.sparse_attn_decode(dummy, dummy, dummy, dummy, B, H, Dqk, Dv, S.shape[-1], 1.0,
                                dtype_code(q), dummy, None, None, ctypes.byref(size), None)
    _check("sparse_attn_decode", rc)
    return size.value


def sparse_attn_decode(q, kv_cache, cu_seqlens, S, softmax_scale, Dv, out=None, lse=None,
                       want_lse=False, workspace=None, stream=None):
    """Sparse attention for the newest token of each sequence: (out [B,H,Dv], lse or None)."""
    lib = load()
    B, H, Dqk = q.shape
    k = S.shape[-1]
    if out is None:
        out = torch.empty((B, H, Dv), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(sparse_attn_decode_workspace_bytes(q, kv_cache, S, Dv),
                                dtype=torch.uint8, device=q.device)
    size = ctypes.c_size_t(workspace.numel())
    rc = lib.sparse_attn_decode(_ptr(q), _ptr(kv_cache), _ptr(cu_seqlens), _ptr(S), B, H, Dqk, Dv,
                                k, float(softmax_scale), dtype_code(q), _ptr(out), _ptr(lse),
                                _ptr(workspace), ctypes.byref(size), _stream(stream))
    _check("sparse_attn_decode", rc)
    return out, lse


def indexer_loss_grad(qI, kI, wI, S, p, loss=None, dq=None, dk=None, dw=None, stream=None):
    """Sparse-stage indexer loss (KL over the selected set) and its gradient:
    returns (loss [B,n], dq [B,n,HI,dI], dk [B,n,dI], dw [B,n,HI]), fp32."""
    lib = load()
    for t, nm in ((qI, "qI"), (kI, "kI"), (wI, "wI"), (S, "S"), (p, "p")):
        _need(t, nm)
    B, n, HI, DI = qI.shape
    k = S.shape[-1]
    dev = qI.device
    f32 = torch.float32
    loss = torch.empty((B, n), dtype=f32, device=dev) if loss is None else loss
    dq = torch.empty((B, n, HI, DI), dtype=f32, device=dev) if dq is None else dq
    dk = torch.empty((B, n, DI), dtype=f32, device=dev) if dk is None else dk
    dw = torch.empty((B, n, HI), dtype=f32, device=dev) if dw is None else dw
    rc = lib.indexer_loss_grad(_ptr(qI), _ptr(kI), _ptr(wI), _ptr(S), _ptr(p), B, n, HI, DI, k, dtype_code(qI),
                               _ptr(loss), _ptr(dq), _ptr(dk), _ptr(dw), _stream(stream))
    _check("indexer_loss_grad", rc)
    return loss, dq, dk, dw


# ---- measurement aids (include/tlsl_measure.h) --------------------------------
def set_debug(on: bool) -> bool:
    """Switch the device checks of cu_seqlens / row_start / row_len on or off
    (tlsl_set_debug); returns the previous state."""
    return bool(load().tlsl_set_debug(1 if on else 0))


def timer_arm(kernel: str, max_launches: int = 4096) -> None:
    """Bracket every following launch of ``kernel`` with HIP events on its stream."""
    lib = load()
    _check("tlsl_timer_arm", lib.tlsl_timer_arm(kernel.encode(), int(max_launches)))


def timer_collect():
    """Disarm the kernel timer: (launches, total_ms, min_ms, max_ms)."""
    lib = load()
    n = ctypes.c_int(0)
    tot, mn, mx = ctypes.c_double(0), ctypes.c_double(0), ctypes.c_double(0)
    _check("tlsl_timer_collect", lib.tlsl_timer_collect(ctypes.byref(n), ctypes.byref(tot), ctypes.byref(mn),
                                                        ctypes.byref(mx)))
    return n.value, tot.value, mn.value, mx.value


def calib_copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    """Streaming copy of src's bytes into dst (the HBM-bandwidth calibration kernel)."""
    lib = load()
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst is smaller than src")
    _check("tlsl_calib_copy", lib.tlsl_calib_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)))


def calib_mfma(dt: int, blocks: int, iters: int, sink: torch.Tensor, stream=None) -> float:
    """Matrix-core loop (the MFMA-rate calibration kernel); returns its flop count."""
    lib = load()
    if sink.dtype != torch.float32 or sink.numel() < blocks * 256:
        raise ValueError("sink must hold blocks*256 float32")
    fl = ctypes.c_double(0)
    _check("tlsl_calib_mfma", lib.tlsl_calib_mfma(int(dt), int(blocks), int(iters), _ptr(sink), ctypes.byref(fl),
                                                  _stream(stream)))
    return fl.value
