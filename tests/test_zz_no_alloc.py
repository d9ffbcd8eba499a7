"""topk_select_noalloc (the allocation-free variant of topk_select, for callers
that cannot allocate: graph capture, tight serving loops) against
topk_select, through the C ABI, on two calls in a row -- the second with a
smaller input, so stale scratch contents from the first would show -- and
against the oracle.  Sizes beyond the fixed scratch are refused."""
import numpy as np
import pytest
import torch

import oracle
import token_level_sparse_lightning_amd as tl
from tests.gpu_util import DEV, announce

pytestmark = pytest.mark.gpu


def _rows(R, lo, hi, seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi + 1, size=R).astype(np.int32)
    lens[0] = 0
    flat = rng.standard_normal(int(lens.sum())).astype(np.float32)
    flat[rng.random(flat.size) < 0.02] = 0.25  # ties
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    return flat, starts, lens


def test_noalloc_equals_topk_select_on_two_calls():
    for R, lo, hi, k, seed in ((64, 16384, 131072, 2048, 1), (9, 1, 5000, 256, 2)):
        flat, starts, lens = _rows(R, lo, hi, seed)
        announce(f"topk_select_noalloc R={R} k={k} sumL={int(lens.sum())}")
        sc, st, ln = (torch.from_numpy(x).to(DEV) for x in (flat, starts, lens))
        max_len = int(lens.max())
        S_na, Ss_na = tl.topk_select_noalloc(sc, st, ln, k, max_len, want_scores=True)
        S_ws, Ss_ws = tl.topk_select(sc, st, ln, k, max_len, want_scores=True)
        torch.cuda.synchronize()
        assert torch.equal(S_na, S_ws)
        assert torch.equal(Ss_na, Ss_ws)
        S_o, Ss_o = oracle.topk_rows(flat, starts, lens, k)
        np.testing.assert_array_equal(S_na.cpu().numpy(), S_o)
        np.testing.assert_array_equal(Ss_na.cpu().numpy(), Ss_o)


def test_noalloc_refuses_more_than_its_scratch():
    flat, starts, lens = _rows(600, 1, 100, 3)
    sc, st, ln = (torch.from_numpy(x).to(DEV) for x in (flat, starts, lens))
    announce("topk_select_noalloc beyond its scratch")
    with pytest.raises(tl.TlslError) as e:
        tl.topk_select_noalloc(sc, st, ln, 2048, int(lens.max()))
    assert e.value.code == -4  # TLSL_ERR_WORKSPACE
