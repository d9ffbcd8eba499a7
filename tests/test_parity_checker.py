"""Fault injection into the parity checker (CPU only).

Every bf16 / fp8 GPU verdict goes through ``oracle/parity.py``.  Following the
NSA page's correctness advice (section 6: a checker must catch a corrupted
index, a dropped tail or swapped indices), each test here starts from a
selection the checker accepts, plants one mistake, and asserts that the
checker now rejects it -- or, for a swap inside the tie margin that the DSA
page (section 3.1, the discussion of ties and the cutoff margin) allows, that
it still accepts it.
"""
import numpy as np
import pytest

import oracle
from oracle import parity

K = 64


def _rows(nrows=200, n=600, seed=0):
    """Distinct random fp32 score rows and the oracle's selection of each
    (query t = n - 1 - i for row i, so every row has t + 1 > K)."""
    rng = np.random.default_rng(seed)
    ts = np.array([n - 1 - i for i in range(nrows)], np.int64)
    sc = rng.standard_normal((nrows, n)).astype(np.float32)
    for i, t in enumerate(ts):
        sc[i, t + 1:] = np.nan
    starts = np.arange(nrows, dtype=np.int64) * n
    S, Ss = oracle.topk_rows(sc.reshape(-1), starts, (ts + 1).astype(np.int32), K)
    return ts, sc, S, Ss


def test_clean_selection_is_accepted():
    ts, sc, S, Ss = _rows()
    rep = parity.check_selection(S, S, ts, K, sc)
    assert rep.ok() and rep.match == 1.0, rep.summary()
    assert parity.check_selection(S, S, ts, K, exact=True).ok(exact=True)
    worst, _ = parity.check_scores(S, Ss, ts, K, sc, None, lowp=True)
    assert worst == 0.0


def _swap_in(row_sel, scores_row, t, pick):
    """Replace the selected position with the lowest score by `pick` (an
    unselected position), keeping the row ascending."""
    sel = row_sel[:K].copy()
    worst = sel[np.argmin(scores_row[sel])]
    sel[sel == worst] = pick
    out = row_sel.copy()
    out[:K] = np.sort(sel)
    return out


def test_loser_far_from_the_cutoff_is_rejected():
    ts, sc, S, _ = _rows()
    bad = S.copy()
    i = 7
    t = int(ts[i])
    unselected = np.setdiff1d(np.arange(t + 1), S[i, :K])
    loser = unselected[np.argmin(sc[i, unselected])]   # the worst key of the row
    bad[i] = _swap_in(S[i], sc[i], t, loser)
    rep = parity.check_selection(bad, S, ts, K, sc)
    assert not rep.ok() and rep.margin_errors, rep.summary()
    assert rep.margin_errors[0][0] == t


def test_swap_inside_the_margin_is_accepted_and_outside_rejected():
    ts, sc, S, _ = _rows()
    i = 3
    t = int(ts[i])
    c = parity.kth_score(sc[i], t, K)
    tol = parity.MARGIN_RTOL * max(abs(c), 1e-6 * float(np.abs(sc[i, : t + 1]).max()))
    unselected = np.setdiff1d(np.arange(t + 1), S[i, :K])
    for factor, accepted in ((0.5, True), (2.0, False)):
        sc2 = sc.copy()
        near = unselected[0]
        sc2[i, near] = np.float32(c - factor * tol)  # just below the K-th score
        bad = S.copy()
        bad[i] = _swap_in(S[i], sc2[i], t, near)
        rep = parity.check_selection(bad, S, ts, K, sc2)
        assert not rep.structure_errors
        assert (not rep.margin_errors) == accepted, (factor, rep.summary())
        # one swapped slot in 200 rows of 64 keeps the match above 99.9%
        assert rep.match > parity.SET_MATCH_MIN
        assert rep.ok() == accepted


def test_too_many_margin_swaps_fail_the_match_fraction():
    ts, sc, S, _ = _rows(nrows=4)
    bad = S.copy()
    sc2 = sc.copy()
    for i in range(4):
        t = int(ts[i])
        c = parity.kth_score(sc[i], t, K)
        near = np.setdiff1d(np.arange(t + 1), S[i, :K])[0]
        sc2[i, near] = c  # an exact tie at the cutoff: a legal alternative
        bad[i] = _swap_in(S[i], sc2[i], t, near)
    rep = parity.check_selection(bad, S, ts, K, sc2)
    assert not rep.margin_errors and not rep.structure_errors
    assert rep.match < parity.SET_MATCH_MIN and not rep.ok()


@pytest.mark.parametrize("fault", ["pad_to_position", "position_to_pad", "unsorted", "duplicate",
                                   "beyond_t", "negative", "dropped_padding"])
def test_structure_faults_are_rejected(fault):
    n = 600
    ts = np.array([30, 599], np.int64)           # one short row (padding), one full
    rng = np.random.default_rng(1)
    sc = rng.standard_normal((2, n)).astype(np.float32)
    S, _ = oracle.topk_rows(sc.reshape(-1), np.array([0, n], np.int64), (ts + 1).astype(np.int32), K)
    bad = S.copy()
    if fault == "pad_to_position":
        bad[0, 40] = 5                           # a -1 slot turned into a position
    elif fault == "position_to_pad":
        bad[0, 10] = -1                          # a selected slot dropped
    elif fault == "unsorted":
        bad[1, [3, 4]] = bad[1, [4, 3]]
    elif fault == "duplicate":
        bad[1, 4] = bad[1, 3]
    elif fault == "beyond_t":
        bad[0, 30] = 31                          # row 0 holds 0..30 = every position
    elif fault == "negative":
        bad[1, 0] = -2
    elif fault == "dropped_padding":
        bad[0, 31:] = 0                          # no -1 after the valid slots
    rep = parity.check_selection(bad, S, ts, K, sc)
    assert rep.structure_errors and not rep.ok(), (fault, rep.summary())


def test_two_swapped_rows_are_rejected():
    ts, sc, S, _ = _rows()
    bad = S.copy()
    bad[[10, 11]] = bad[[11, 10]]
    rep = parity.check_selection(bad, S, ts, K, sc)
    assert not rep.ok(), rep.summary()
    assert rep.structure_errors or rep.margin_errors


def test_exact_mode_flags_any_difference():
    ts, sc, S, _ = _rows()
    bad = S.copy()
    i = 5
    t = int(ts[i])
    near = np.setdiff1d(np.arange(t + 1), S[i, :K])[0]
    sc2 = sc.copy()
    sc2[i, near] = parity.kth_score(sc[i], t, K)   # a tie: fine for the margin rule
    bad[i] = _swap_in(S[i], sc2[i], t, near)
    rep = parity.check_selection(bad, S, ts, K, exact=True)
    assert rep.exact_errors and not rep.ok(exact=True)


def test_score_faults_are_rejected():
    ts, sc, S, Ss = _rows()
    # a score perturbed beyond the low-precision tolerance
    bad = Ss.copy()
    bad[9, 17] += 0.05
    worst, wt = parity.check_scores(S, bad, ts, K, sc, None, lowp=True)
    assert worst > 1.0 and wt == int(ts[9])
    # within it
    ok = Ss.copy()
    ok[9, 17] += 0.5 * parity.SCORE_ATOL_LOWP
    assert parity.check_scores(S, ok, ts, K, sc, None, lowp=True)[0] <= 1.0
    # a padding slot that is not -inf
    ts2 = np.array([20], np.int64)
    sc2 = sc[:1].copy()
    S2, Ss2 = oracle.topk_rows(sc2.reshape(-1), np.array([0], np.int64), np.array([21], np.int32), K)
    Ss2[0, 30] = 0.0
    assert parity.check_scores(S2, Ss2, ts2, K, sc2, None, lowp=True)[0] == float("inf")
    # fp32 inputs: relative bound 1e-5 * max(|I|, A)
    mag = np.abs(sc).astype(np.float32)
    bad = Ss.copy()
    bad[2, 5] = Ss[2, 5] * (1 + 1e-4) + 1e-4
    assert parity.check_scores(S, bad, ts, K, sc, mag, lowp=False)[0] > 1.0
    assert parity.check_scores(S, Ss, ts, K, sc, mag, lowp=False)[0] == 0.0


def test_score_vector_faults_are_rejected():
    rng = np.random.default_rng(3)
    ref = rng.standard_normal(1000).astype(np.float32)
    mag = np.abs(ref) + 1.0
    got = ref.copy()
    assert parity.check_score_vector(got, ref, mag, lowp=True) == 0.0
    got[123] += 0.05
    assert parity.check_score_vector(got, ref, mag, lowp=True) > 1.0
    got = ref.copy()
    got[5] += 1e-3 * mag[5]
    assert parity.check_score_vector(got, ref, mag, lowp=False) > 1.0
    got = ref.copy()
    got[5] += 1e-6 * mag[5]
    assert parity.check_score_vector(got, ref, mag, lowp=False) <= 1.0
