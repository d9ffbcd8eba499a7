"""The debug switch (tlsl_set_debug): with it on, the calls that take index
metadata in device memory check it on the device before launching anything,
and return TLSL_ERR_SHAPE for a malformed batch; on well-formed input the
results are the same as with it off.

Every malformed input used here would stay in bounds even if it reached the
kernels (the cache and score buffers are padded past the shifted sequence
boundaries; a negative row length is clamped to an empty row by the kernels),
so the tests exercise the checks without risking an out-of-bounds access."""
import numpy as np
import pytest
import torch

import token_level_sparse_lightning_amd as tl
from token_level_sparse_lightning_amd import synth
from tests.gpu_util import DEV, announce, to_dev

pytestmark = pytest.mark.gpu

SHAPE_ERR = -2
FP8 = synth.DT_FP8


@pytest.fixture
def debug_on():
    prev = tl.set_debug(True)
    try:
        yield
    finally:
        tl.set_debug(prev)


def _decode_inputs():
    lengths = [300, 0, 2049, 77]
    inp = synth.indexer_decode(lengths, 64, 128, FP8, seed=11, planted=False)
    return lengths, inp


def test_debug_switch_reports_previous_state():
    prev = tl.set_debug(True)
    try:
        assert tl.set_debug(True) is True
    finally:
        tl.set_debug(prev)
    assert tl.set_debug(prev) is prev


def test_index_decode_same_scores_with_checks(debug_on):
    lengths, inp = _decode_inputs()
    args = (to_dev(inp.q), to_dev(inp.k), to_dev(inp.w), to_dev(inp.cu_seqlens), max(lengths))
    kw = dict(q_scale=to_dev(inp.q_scale), k_scale=to_dev(inp.k_scale))
    announce("index_decode with the device checks on")
    on = tl.index_decode(*args, **kw)
    tl.set_debug(False)
    off = tl.index_decode(*args, **kw)
    torch.cuda.synchronize()
    assert torch.equal(on, off)


def test_index_decode_rejects_nonzero_first_boundary(debug_on):
    lengths, inp = _decode_inputs()
    pad = 64
    total = int(sum(lengths))
    kpad = torch.cat([inp.k, torch.zeros((pad, 128), dtype=inp.k.dtype)])
    spad = torch.cat([inp.k_scale, torch.ones(pad, dtype=torch.float32)])
    cu_bad = inp.cu_seqlens + pad  # every boundary shifted: in bounds of the padded cache
    scores = torch.full((total + pad,), float("nan"), device=DEV)
    announce("index_decode with cu_seqlens[0] = 64 and the device checks on")
    with pytest.raises(tl.TlslError) as ei:
        tl.index_decode(to_dev(inp.q), to_dev(kpad), to_dev(inp.w), to_dev(cu_bad), max(lengths),
                        q_scale=to_dev(inp.q_scale), k_scale=to_dev(spad), scores=scores)
    assert ei.value.code == SHAPE_ERR and "cu_seqlens[0] = 64" in str(ei.value)
    torch.cuda.synchronize()
    assert torch.isnan(scores).all()  # nothing was launched


def test_sparse_attn_decode_rejects_decreasing_boundaries(debug_on):
    lengths = np.array([40, 70, 33], dtype=np.int64)
    q, kv = synth.attn_decode(lengths, 128, 576, synth.DT_BF16, seed=5)
    cu = np.zeros(4, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    S = torch.arange(32, dtype=torch.int32).repeat(3, 1)
    out_ok, _ = tl.sparse_attn_decode(to_dev(q), to_dev(kv), torch.from_numpy(cu).to(DEV), to_dev(S),
                                      1 / 24, 512)
    bad = cu.copy()
    bad[2] = bad[1] - 5  # sequence 1 has a negative length (the kernel would see no valid slot)
    out = torch.full((3, 128, 512), float("nan"), dtype=torch.bfloat16, device=DEV)
    announce("sparse_attn_decode with a decreasing cu_seqlens and the device checks on")
    with pytest.raises(tl.TlslError) as ei:
        tl.sparse_attn_decode(to_dev(q), to_dev(kv), torch.from_numpy(bad).to(DEV), to_dev(S), 1 / 24, 512, out=out)
    assert ei.value.code == SHAPE_ERR and "cu_seqlens[2]" in str(ei.value)
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()
    assert torch.isfinite(out_ok.float()).all()


def test_topk_select_rejects_negative_row_length(debug_on):
    g = torch.Generator(device=DEV)
    g.manual_seed(4)
    scores = torch.randn(5000, generator=g, device=DEV)
    row_start = torch.tensor([0, 1000, 3000], dtype=torch.int64, device=DEV)
    row_len = torch.tensor([1000, 2000, 2000], dtype=torch.int32, device=DEV)
    S_on, _ = tl.topk_select(scores, row_start, row_len, 64, 2000)
    tl.set_debug(False)
    S_off, _ = tl.topk_select(scores, row_start, row_len, 64, 2000)
    torch.cuda.synchronize()
    assert torch.equal(S_on, S_off)
    tl.set_debug(True)
    bad_len = torch.tensor([1000, -5, 2000], dtype=torch.int32, device=DEV)
    announce("topk_select and topk_select_noalloc with a negative row length and the device checks on")
    for fn in (tl.topk_select, tl.topk_select_noalloc):
        with pytest.raises(tl.TlslError) as ei:
            fn(scores, row_start, bad_len, 64, 2000)
        assert ei.value.code == SHAPE_ERR and "row_len[1] = -5" in str(ei.value)
