"""Parity rules between the HIP library and the oracle -- TEST INFRASTRUCTURE.

Selection (DSA page, section 1.1 eq.(2); the tie discussion of section 3.1
says two correct implementations may return different indices when scores
tie, so compare the cutoff value, the set strictly above it, then the ties):

* structure, always exact: row t holds K_t = min(k, t+1) positions, strictly
  ascending, inside [0, t], then exactly k - K_t entries of -1;
* ``exact=True`` (dyadic inputs, every score exact in fp32): identical rows;
* otherwise the selected sets may differ only at the margin: every position
  in the symmetric difference must have an oracle score within
  ``1e-3 * max(|c_t|, 1e-6 * max_s |I(t,s)|)`` of the oracle's K_t-th score
  c_t, and at least 99.9% of the selected slots must agree overall.

Scores: fp32 inputs |dI| <= 1e-5 * max(|I|, A) with A the magnitude sum
sum_j |w_j| ReLU(q_j . k) (cancellation between heads of opposite weight makes
a plain relative bound meaningless); bf16 / fp8 inputs |dI| <= 2e-2.

Attention: max |out_gpu - out_oracle| <= 2e-2 (bf16) or 1e-5 (fp32), with the
oracle run on the GPU's own selection (two-layer check).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SCORE_RTOL_F32 = 1e-5
SCORE_ATOL_LOWP = 2e-2
MARGIN_RTOL = 1e-3
SET_MATCH_MIN = 0.999
ATTN_ATOL_BF16 = 2e-2
ATTN_ATOL_F32 = 1e-5


@dataclass
class SelectionReport:
    rows: int = 0
    slots: int = 0
    matched: int = 0
    structure_errors: list = field(default_factory=list)
    margin_errors: list = field(default_factory=list)
    exact_errors: list = field(default_factory=list)
    mismatched_rows: int = 0
    worst_margin_ratio: float = 0.0   # max over mismatches of |I(t,s) - c_t| / tolerance

    @property
    def match(self) -> float:
        return 1.0 if self.slots == 0 else self.matched / self.slots

    def ok(self, exact=False) -> bool:
        if self.structure_errors or self.margin_errors:
            return False
        if exact:
            return not self.exact_errors
        return self.match >= SET_MATCH_MIN

    def summary(self) -> str:
        return (f"rows={self.rows} slots={self.slots} match={self.match:.6f} "
                f"mismatched_rows={self.mismatched_rows} worst_margin_ratio={self.worst_margin_ratio:.3g} "
                f"structure={self.structure_errors[:3]} margin={self.margin_errors[:3]} "
                f"exact={self.exact_errors[:3]}")


def check_structure(row: np.ndarray, t: int, k: int):
    """Return None if row is a well-formed selection for query t, else a message."""
    K = min(k, t + 1)
    valid, pad = row[:K], row[K:]
    if len(row) != k:
        return f"width {len(row)} != {k}"
    if (pad != -1).any():
        return f"padding is not -1 ({int((pad != -1).sum())} bad slots)"
    if (valid < 0).any() or (valid > t).any():
        return "position outside [0, t]"
    if K > 1 and not (np.diff(valid) > 0).all():
        return "positions not strictly ascending"
    return None


def kth_score(scores_row: np.ndarray, t: int, K: int) -> float:
    """The K-th largest fp32 score among positions 0..t."""
    return float(np.sort(scores_row[: t + 1])[::-1][K - 1])


def check_selection(S_gpu, S_ora, ts, k, score_rows=None, exact=False) -> SelectionReport:
    """Compare selections row by row.  ``score_rows[i]`` are the oracle's fp32
    scores of row i (positions 0..t); needed unless ``exact``."""
    rep = SelectionReport()
    S_gpu = np.asarray(S_gpu)
    S_ora = np.asarray(S_ora)
    for i, t in enumerate(ts):
        t = int(t)
        K = min(k, t + 1)
        rep.rows += 1
        rep.slots += K
        g, o = S_gpu[i], S_ora[i]
        msg = check_structure(g, t, k)
        if msg:
            rep.structure_errors.append((t, msg))
            continue
        if exact and not np.array_equal(g, o):
            rep.exact_errors.append((t, int((g != o).sum())))
        gs, os_ = set(g[:K].tolist()), set(o[:K].tolist())
        rep.matched += len(gs & os_)
        diff = gs ^ os_
        rep.mismatched_rows += bool(diff)
        if diff and score_rows is not None:
            sr = np.asarray(score_rows[i], dtype=np.float64)
            c = kth_score(sr, t, K)
            floor = 1e-6 * float(np.abs(sr[: t + 1]).max())
            tol = MARGIN_RTOL * max(abs(c), floor)
            worst = max(abs(sr[s] - c) for s in diff)
            rep.worst_margin_ratio = max(rep.worst_margin_ratio, worst / tol if tol > 0 else float("inf"))
            if worst > tol:
                rep.margin_errors.append((t, len(diff), worst, tol))
        elif diff and not exact:
            rep.margin_errors.append((t, len(diff), float("nan"), 0.0))
    return rep


def check_scores(S_gpu, Ss_gpu, ts, k, score_rows, mag_rows, lowp: bool):
    """Check the per-slot scores the GPU reports for its own selection.
    Returns (max violation ratio, worst row); ratio <= 1 passes."""
    worst, worst_t = 0.0, None
    for i, t in enumerate(ts):
        K = min(k, int(t) + 1)
        pos = np.asarray(S_gpu[i][:K])
        got = np.asarray(Ss_gpu[i][:K], dtype=np.float64)
        ref = np.asarray(score_rows[i], dtype=np.float64)[pos]
        if lowp:
            tol = np.full(K, SCORE_ATOL_LOWP)
        else:
            mag = np.asarray(mag_rows[i], dtype=np.float64)[pos]
            tol = SCORE_RTOL_F32 * np.maximum(np.abs(ref), mag)
            tol = np.maximum(tol, 1e-30)
        r = float((np.abs(got - ref) / tol).max()) if K else 0.0
        if not np.isneginf(np.asarray(Ss_gpu[i][K:])).all():
            r = float("inf")
        if r > worst:
            worst, worst_t = r, int(t)
    return worst, worst_t


def check_score_vector(got, ref, mag, lowp: bool):
    """Elementwise score check for a decode scan; returns the max violation ratio."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if lowp:
        return float((np.abs(got - ref) / SCORE_ATOL_LOWP).max())
    tol = np.maximum(SCORE_RTOL_F32 * np.maximum(np.abs(ref), np.asarray(mag, dtype=np.float64)), 1e-30)
    return float((np.abs(got - ref) / tol).max())
