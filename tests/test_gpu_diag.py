"""GPU parity of the selection-quality diagnostics (DSA page, section 1.2
eq.(9); section 3.1 eq.(14), (15), (18)) against the oracle: recall of the
teacher's top-m and the cutoff margin are exact (ratios of counts, and the
fp32 difference of two fp32 scores, each rounded once); the mass coverage is
a ratio of fp64 sums rounded once to fp32, equal to the oracle's up to one
unit in the last place (the two sums run in different orders)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import token_level_sparse_lightning_amd as tl
from tests.gpu_util import DEV, announce

pytestmark = pytest.mark.gpu


def _rows(seed):
    rng = np.random.default_rng(seed)
    lens = [0, 1, 5, 64, 65, 2049, 5000, 20000, 140001]
    teach, scores = [], []
    for L in lens:
        a = rng.random(L).astype(np.float32) ** 4
        a[rng.random(L) < 0.05] = 0.25            # tied teacher masses
        teach.append(a)
        s = rng.standard_normal(L).astype(np.float32)
        s[rng.random(L) < 0.05] = 0.5             # tied scores (margin 0 where they meet the cutoff)
        scores.append(s)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    return np.concatenate(teach), np.concatenate(scores), starts, np.array(lens, np.int32)


@pytest.mark.parametrize("k,m", [(64, 16), (2048, 2048), (2048, 64)])
def test_selection_quality(k, m):
    teach, scores, starts, lens = _rows(k + m)
    announce(f"selection_quality k={k} m={m}")
    d = lambda x: torch.from_numpy(x).to(DEV)
    S, _ = tl.topk_select(d(scores), d(starts), d(lens), k, int(lens.max()))
    recall, mass = tl.selection_quality(d(teach), d(starts), d(lens), S, m, int(lens.max()))
    torch.cuda.synchronize()
    r_o, m_o = oracle.selection_quality(teach, starts, lens, S.cpu().numpy(), m)
    np.testing.assert_array_equal(recall.cpu().numpy(), r_o.astype(np.float32))
    got = mass.cpu().numpy()
    ref = m_o.astype(np.float32)
    assert (np.isnan(got) == np.isnan(ref)).all()
    ok = ~np.isnan(ref)
    assert (np.abs(got[ok] - ref[ok]) <= np.spacing(ref[ok])).all(), (got, ref)
    print(f"[parity] selection_quality k={k} m={m}: recall exact, mass within 1 ulp; recall {recall.cpu().numpy()}",
          flush=True)


@pytest.mark.parametrize("k", [1, 64, 2048])
def test_cutoff_margin(k):
    _, scores, starts, lens = _rows(7 + k)
    announce(f"cutoff_margin k={k}")
    d = lambda x: torch.from_numpy(x).to(DEV)
    mg = tl.cutoff_margin(d(scores), d(starts), d(lens), k, int(lens.max()))
    torch.cuda.synchronize()
    ref = oracle.cutoff_margin(scores, starts, lens, k).astype(np.float32)
    np.testing.assert_array_equal(mg.cpu().numpy(), ref)


def test_cutoff_margin_worked_example():
    with open(os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")) as f:
        sc = np.array(json.load(f)["indexer"]["scores"], np.float32)
    d = lambda x: torch.from_numpy(x).to(DEV)
    announce("cutoff_margin worked example")
    out = [float(tl.cutoff_margin(d(sc), d(np.array([0], np.int64)), d(np.array([3], np.int32)), k, 3)[0])
           for k in (1, 2, 3)]
    assert out == [0.0, 0.5, float("inf")]
