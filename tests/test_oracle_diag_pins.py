"""Pins of the oracle's selection-quality diagnostics (CPU only).

DSA page, section 1.2 eq.(9) (recall of the teacher's top-m) and section 3.1
eq.(14) (the same at m = k), eq.(15) (teacher mass coverage) and eq.(18) (the
cutoff margin).  Each is tied to something the oracle does not compute
itself: values worked out by hand from the page's 3-token example and from
the page's three-head example, brute force with Python sets and numpy sorts,
and invariances of the definitions.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def test_cutoff_margin_on_the_worked_example():
    """Scores 1.5, 1.5, 1.0 (the page's example): Delta_1 = 1.5 - 1.5 = 0 (the
    tie the k=1 selection breaks by position), Delta_2 = 1.5 - 1.0 = 0.5, and
    no third-ranked competitor at k = 3."""
    with open(GOLDEN) as f:
        sc = np.array(json.load(f)["indexer"]["scores"], np.float32)
    m = oracle.cutoff_margin(np.tile(sc, 3), [0, 3, 6], [3, 3, 3], 1)
    assert m.tolist() == [0.0, 0.0, 0.0]
    assert oracle.cutoff_margin(sc, [0], [3], 2).tolist() == [0.5]
    assert oracle.cutoff_margin(sc, [0], [3], 3).tolist() == [np.inf]


def test_three_head_example_recall_and_mass():
    """The page's three-head example: heads put 0.9 on positions 10, 20 and 30
    (the rest spread evenly over 40 positions); the averaged teacher has its
    three peaks at 0.3 + 0.1/40 each.  A shared set of k = 2 can hold two
    peaks: recall of the teacher's top-3 is 2/3 and the covered mass is
    2 * (0.3 + 0.1/40)."""
    L = 40
    heads = np.full((3, L), 0.1 / (L - 1))
    for h, pos in enumerate((10, 20, 30)):
        heads[h, pos] = 0.9
    a = heads.mean(0).astype(np.float32)
    S = np.array([[10, 30]], np.int32)
    recall, mass = oracle.selection_quality(a, [0], [L], S, 3)
    assert recall[0] == 2 / 3
    np.testing.assert_allclose(mass[0], 2 * float(a[10]) / float(a.astype(np.float64).sum()), rtol=1e-12)
    # with m = k = 2 (eq.(14)) the teacher's top-2 are 10 and 20 (equal peaks:
    # lower positions win), of which the set holds one
    recall2, _ = oracle.selection_quality(a, [0], [L], S, 2)
    assert recall2[0] == 0.5


@pytest.mark.parametrize("seed", [0, 1])
def test_recall_mass_margin_brute_force(seed):
    rng = np.random.default_rng(seed)
    lens = [0, 1, 7, 64, 65, 300, 1000]
    k, m = 64, 16
    rows, starts, Ss = [], [], []
    off = 0
    for L in lens:
        a = rng.random(L).astype(np.float32) ** 4
        a[rng.random(L) < 0.1] = 0.5                       # ties
        rows.append(a)
        starts.append(off)
        off += L
        S = np.full(k, -1, np.int32)
        K = min(k, L)
        S[:K] = np.sort(rng.choice(L, K, replace=False)) if L else []
        Ss.append(S)
    flat = np.concatenate(rows) if off else np.zeros(0, np.float32)
    S = np.stack(Ss)
    recall, mass = oracle.selection_quality(flat, starts, lens, S, m)
    margin = oracle.cutoff_margin(flat, starts, lens, k)
    for r, (a, L) in enumerate(zip(rows, lens)):
        sel = set(int(x) for x in S[r] if 0 <= x < L)
        order = sorted(range(L), key=lambda s: (-float(a[s]), s))   # eq.(2)'s order
        G = set(order[: min(m, L)])
        if G:
            assert recall[r] == len(G & sel) / len(G)
        else:
            assert np.isnan(recall[r])
        tot = float(a.astype(np.float64).sum())
        if tot > 0:
            np.testing.assert_allclose(mass[r], sum(float(a[s]) for s in sel) / tot, rtol=1e-12)
        else:
            assert np.isnan(mass[r])
        if L > k:
            desc = np.sort(a.astype(np.float64))[::-1]
            assert margin[r] == desc[k - 1] - desc[k]
            assert margin[r] >= 0
        else:
            assert margin[r] == np.inf


def test_diagnostics_invariances():
    """A selection equal to the teacher's top-k has recall 1 at m = k
    (eq.(14)); mass coverage is invariant to scaling the teacher; the margin
    scales with the scores; a repeated or out-of-range entry adds nothing."""
    rng = np.random.default_rng(3)
    L, k = 500, 32
    a = rng.random(L).astype(np.float32)
    top = np.sort(np.argsort(-a, kind="stable")[:k]).astype(np.int32)[None]
    r, mass = oracle.selection_quality(a, [0], [L], top, k)
    assert r[0] == 1.0
    _, mass2 = oracle.selection_quality(a * np.float32(4.0), [0], [L], top, k)
    assert mass2[0] == mass[0]
    m1 = oracle.cutoff_margin(a, [0], [L], k)
    m2 = oracle.cutoff_margin(a * np.float32(2.0), [0], [L], k)
    assert m2[0] == 2 * m1[0]
    messy = top.copy()
    messy[0, 0] = messy[0, 1]
    messy[0, 2] = L + 5
    clean = np.delete(top, [0, 2], axis=1)
    clean = np.concatenate([clean, np.full((1, 2), -1, np.int32)], axis=1)
    assert oracle.selection_quality(a, [0], [L], messy, k)[1][0] == oracle.selection_quality(a, [0], [L], clean, k)[1][0]
