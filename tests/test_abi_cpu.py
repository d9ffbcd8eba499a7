"""The C ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before anything is launched (CPU only: no call here
reaches a kernel launch)."""
import ctypes
import os
import re

import pytest
import torch

import token_level_sparse_lightning_amd as tl
from token_level_sparse_lightning_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tlsl.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUP, ERR_WS, ERR_HIP, ERR_ALIGN = 0, -1, -2, -3, -4, -5, -6


def _lib():
    if not os.path.exists(binding.LIB_PATH):
        from token_level_sparse_lightning_amd import build
        build.build()
    return tl.load()


def _declared(headers=None):
    names = set()
    for h in headers or HEADERS:
        text = open(h).read()
        names |= set(re.findall(r"^(?:int|const char\*)\s+(\w+)\s*\(", text, flags=re.M))
    return sorted(names)


def test_header_declares_the_five_calls():
    names = _declared([HEADER])
    for fn in ("index_prefill", "index_decode", "topk_select", "sparse_attn_prefill",
               "sparse_attn_decode", "tlsl_last_error", "tlsl_version"):
        assert fn in names


def test_every_declared_symbol_is_exported():
    lib = _lib()
    names = _declared()
    assert "tlsl_timer_arm" in names and "tlsl_calib_copy" in names
    for fn in names:
        assert hasattr(lib, fn), fn
    assert set(binding.EXPORTS) == set(names)
    assert lib.tlsl_version().startswith(b"tlsl")


def test_measurement_validation():
    """Host-side checks of the measurement aids (no event or launch is made)."""
    lib = _lib()
    assert lib.tlsl_timer_arm(None, 4) == ERR_NULL
    assert lib.tlsl_timer_arm(b"prefill_score_kernel", 0) == ERR_SHAPE
    assert lib.tlsl_timer_arm(b"prefill_score_kernel", 70000) == ERR_SHAPE
    assert lib.tlsl_timer_collect(None, None, None, None) == ERR_SHAPE      # not armed
    assert lib.tlsl_calib_copy(None, P, 16, None) == ERR_NULL
    assert lib.tlsl_calib_copy(P, P, 17, None) == ERR_SHAPE
    assert lib.tlsl_calib_copy(MIS, P, 16, None) == ERR_ALIGN
    d = ctypes.c_double(0)
    assert lib.tlsl_calib_mfma(1, 0, 4, P, ctypes.byref(d), None) == ERR_SHAPE
    assert lib.tlsl_calib_mfma(0, 4, 4, P, ctypes.byref(d), None) == ERR_UNSUP
    assert b"bf16" in lib.tlsl_last_error()


P = ctypes.c_void_p(256)      # aligned dummy device pointer: never dereferenced here
MIS = ctypes.c_void_p(257)    # misaligned dummy


def _ws():
    return ctypes.c_size_t(0)


def _prefill(lib, q=P, qs=None, k=P, ks=None, w=P, B=1, n=64, HI=64, DI=128, kk=16, dt=1, S=P,
             Ss=None, ws=None, size=None):
    size = size if size is not None else _ws()
    return lib.index_prefill(q, qs, k, ks, w, B, n, HI, DI, kk, dt, S, Ss, ws, ctypes.byref(size), None), size


def test_index_prefill_validation():
    lib = _lib()
    assert _prefill(lib, q=None)[0] == ERR_NULL
    assert b"non-NULL" in lib.tlsl_last_error()
    assert _prefill(lib, S=None)[0] == ERR_NULL
    assert _prefill(lib, dt=7)[0] == ERR_UNSUP
    assert _prefill(lib, dt=2)[0] == ERR_NULL                    # fp8 needs both scales
    assert _prefill(lib, dt=1, qs=P, ks=P)[0] == ERR_SHAPE        # scales only for fp8
    assert _prefill(lib, DI=96)[0] == ERR_UNSUP
    assert _prefill(lib, HI=65)[0] == ERR_UNSUP
    assert _prefill(lib, dt=2, qs=P, ks=P, DI=64)[0] == ERR_UNSUP
    assert _prefill(lib, n=0)[0] == ERR_SHAPE
    assert _prefill(lib, kk=0)[0] == ERR_SHAPE
    assert _prefill(lib, kk=5000)[0] == ERR_UNSUP
    assert _prefill(lib, q=MIS)[0] == ERR_ALIGN
    # size query: nothing launches, a positive size comes back
    rc, size = _prefill(lib)
    assert rc == OK and size.value > 0
    # too small a workspace is refused before any launch
    small = ctypes.c_size_t(size.value - 1)
    rc, _ = _prefill(lib, ws=P, size=small)
    assert rc == ERR_WS
    assert _prefill(lib, ws=MIS, size=ctypes.c_size_t(size.value))[0] == ERR_ALIGN


def test_workspace_grows_with_the_problem():
    a = tl.index_prefill_workspace_bytes(torch.empty(1, 1024, 64, 128, dtype=torch.bfloat16), None, None, 256)
    b = tl.index_prefill_workspace_bytes(torch.empty(1, 4096, 64, 128, dtype=torch.bfloat16), None, None, 256)
    c = tl.index_prefill_workspace_bytes(torch.empty(1, 4096, 64, 128, dtype=torch.bfloat16), None, None, 2048)
    assert 0 < a < b < c


def test_index_decode_validation():
    lib = _lib()
    f = lib.index_decode
    s = _ws()
    assert f(None, None, P, None, P, P, 4, 64, 128, 100, 1, P, None, ctypes.byref(s), None) == ERR_NULL
    assert f(P, None, P, None, P, None, 4, 64, 128, 100, 1, P, None, ctypes.byref(s), None) == ERR_NULL
    assert f(P, None, P, None, P, P, 0, 64, 128, 100, 1, P, None, ctypes.byref(s), None) == ERR_SHAPE
    assert f(P, None, P, None, P, P, 4, 64, 128, 0, 1, P, None, ctypes.byref(s), None) == ERR_SHAPE
    assert f(P, None, P, None, P, P, 4, 64, 100, 10, 1, P, None, ctypes.byref(s), None) == ERR_UNSUP
    assert f(P, None, P, None, P, P, 4, 64, 128, 10, 2, P, None, ctypes.byref(s), None) == ERR_NULL


def test_topk_select_validation():
    lib = _lib()
    f = lib.topk_select
    s = _ws()
    assert f(None, P, P, 4, 16, 100, P, None, None, ctypes.byref(s), None) == ERR_NULL
    assert f(P, P, P, 0, 16, 100, P, None, None, ctypes.byref(s), None) == ERR_SHAPE
    assert f(P, P, P, 4, 0, 100, P, None, None, ctypes.byref(s), None) == ERR_SHAPE
    assert f(P, P, P, 4, 4097, 100, P, None, None, ctypes.byref(s), None) == ERR_UNSUP
    assert f(P, P, P, 4, 16, -1, P, None, None, ctypes.byref(s), None) == ERR_SHAPE
    assert f(P, P, P, 4, 16, 100, MIS, None, None, ctypes.byref(s), None) == ERR_ALIGN
    size = _ws()
    assert f(P, P, P, 64, 2048, 131072, P, None, None, ctypes.byref(size), None) == OK   # size query
    assert size.value > 64 * 2048 * 8
    assert f(P, P, P, 64, 2048, 131072, P, None, P, ctypes.byref(ctypes.c_size_t(size.value - 1)),
             None) == ERR_WS


def test_attention_validation():
    lib = _lib()
    f = lib.sparse_attn_prefill
    s = _ws()
    args = lambda **kw: dict(dict(q=P, kv=P, S=P, B=1, n=8, H=128, Dqk=576, Dv=512, k=16, sc=0.1, dt=1, out=P), **kw)

    def call(**kw):
        a = args(**kw)
        return f(a["q"], a["kv"], a["S"], a["B"], a["n"], a["H"], a["Dqk"], a["Dv"], a["k"], a["sc"], a["dt"],
                 a["out"], None, None, ctypes.byref(s), None)

    assert call(q=None) == ERR_NULL
    assert call(n=0) == ERR_SHAPE
    assert call(dt=2) == ERR_UNSUP
    assert call(Dqk=512) == ERR_UNSUP
    assert call(H=129) == ERR_UNSUP
    assert call(k=4097) == ERR_UNSUP                                # one workgroup stages at most 4096 slots
    assert call(sc=0.0) == ERR_SHAPE
    assert call(sc=float("nan")) == ERR_SHAPE
    assert call(sc=float("inf")) == ERR_SHAPE
    assert call(out=MIS) == ERR_ALIGN
    d = lib.dense_attn_prefill

    def dcall(**kw):
        a = args(**kw)
        return d(a["q"], a["kv"], a["B"], a["n"], a["H"], a["Dqk"], a["Dv"], a["sc"], a["dt"], a["out"], None,
                 None, ctypes.byref(s), None)

    assert dcall(kv=None) == ERR_NULL
    assert dcall(B=0) == ERR_SHAPE
    assert dcall(n=4097) == ERR_UNSUP                               # every row's history fits one workgroup
    assert dcall(H=17, Dqk=80, Dv=64, dt=0) == ERR_UNSUP
    assert dcall(sc=float("inf")) == ERR_SHAPE
    assert dcall(q=MIS) == ERR_ALIGN
    g = lib.sparse_attn_decode
    size = _ws()
    assert g(P, P, P, P, 64, 128, 576, 512, 2048, 0.04, 1, P, None, None, ctypes.byref(size), None) == OK
    assert size.value > 0                                           # the split partials
    assert g(P, P, P, P, 64, 128, 576, 512, 2048, 0.04, 1, P, None, P,
             ctypes.byref(ctypes.c_size_t(size.value - 1)), None) == ERR_WS
    assert g(P, P, None, P, 64, 128, 576, 512, 2048, 0.04, 1, P, None, None, ctypes.byref(size), None) == ERR_NULL
    assert g(P, P, P, P, 64, 128, 576, 512, 4097, 0.04, 1, P, None, None, ctypes.byref(size), None) == ERR_UNSUP


def test_indexer_loss_grad_validation():
    lib = _lib()
    f = lib.indexer_loss_grad
    args = lambda **kw: dict(dict(q=P, k=P, w=P, S=P, p=P, B=1, n=64, HI=64, dI=128, topk=16, dt=1,
                                  loss=P, dq=P, dk=P, dw=P), **kw)

    def call(**kw):
        a = args(**kw)
        return f(a["q"], a["k"], a["w"], a["S"], a["p"], a["B"], a["n"], a["HI"], a["dI"], a["topk"], a["dt"],
                 a["loss"], a["dq"], a["dk"], a["dw"], None)

    assert call(p=None) == ERR_NULL
    assert call(dk=None) == ERR_NULL
    assert call(n=0) == ERR_SHAPE
    assert call(B=1 << 10, n=(1 << 20) + 1) == ERR_SHAPE            # B*n above 2^30
    assert call(dt=2) == ERR_UNSUP
    assert call(dI=64) == ERR_UNSUP
    assert call(HI=65) == ERR_UNSUP
    assert call(topk=4097) == ERR_UNSUP
    assert call(n=1 << 22) == ERR_UNSUP                             # dK rows take 32-bit byte offsets
    assert call(dq=MIS) == ERR_ALIGN


def test_debug_switch(monkeypatch):
    """tlsl_set_debug returns the previous state; the device checks it
    switches on run only where a launch would follow (a size query returns
    before them, so it stays valid on a host without a GPU)."""
    lib = _lib()
    prev = lib.tlsl_set_debug(1)
    try:
        assert prev in (0, 1)
        assert lib.tlsl_set_debug(1) == 1
        need = ctypes.c_size_t(0)
        assert lib.topk_select(P, P, P, 64, 2048, 131072, P, None, None, ctypes.byref(need), None) == OK
        assert need.value > 0
        assert lib.tlsl_set_debug(0) == 1
        assert lib.tlsl_set_debug(0) == 0
    finally:
        lib.tlsl_set_debug(prev)


def test_binding_refuses_when_library_missing(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        binding.load()
