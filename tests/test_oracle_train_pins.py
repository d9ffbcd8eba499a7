"""Pins of the oracle's sparse-stage indexer loss and gradient (CPU only).

DSA page, section 1.2 eq.(8): per query, KL(p_{t,S_t} || Softmax(I_{t,S_t}))
with both sides normalised over the selected set (a teacher cut from a dense
distribution is divided by its kept mass); eq.(7) is the dense warm-up form.
Each test ties ``oracle.indexer_kl`` to something it does not compute itself:
a closed form derived by hand on the page's worked example, central finite
differences of the oracle's own loss (a check of the gradient, not of the
loss), scipy's relative entropy and softmax on the case where the selection
keeps all history (eq.(8) = eq.(7)), and invariances of the definition.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import softmax
from scipy.stats import entropy

import oracle
from token_level_sparse_lightning_amd import synth

F32 = synth.DT_F32
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def _example():
    """The page's 3-token example: query at t=2 (H^I=2, d^I=2), keys at 0..2;
    rows 0 and 1 have zero queries and weights."""
    with open(GOLDEN) as f:
        ex = json.load(f)["indexer"]
    q = np.zeros((1, 3, 2, 2), np.float32)
    q[0, 2] = ex["q"]
    k = np.array(ex["keys"], np.float32)[None]
    w = np.zeros((1, 3, 2), np.float32)
    w[0, 2] = ex["w"]
    return q, k, w


def test_worked_example_closed_form():
    """S_2 = {0, 1} (scores 1.5, 1.5), teacher masses (1, 3): P = (1/4, 3/4),
    the student is uniform, so L = 1/4 ln(1/2) + 3/4 ln(3/2) and
    g = R - P = (1/4, -1/4).  With X = q_j . k_s = [[2, -1], [1, 3]] (keys 0, 1;
    heads 0, 1) the chain rule through eq.(1) gives, by hand:
      dw = 1/4 (2, 0) - 1/4 (1, 3)                 = (1/4, -3/4)
      dq_0 = w_0 (1/4 k_0 - 1/4 k_1)               = (3/16, -3/4)
      dq_1 = w_1 (-1/4) k_1  (X_01 = -1 is cut)    = (-1/16, -3/16)
      dk_0 = 1/4 w_0 q_0                           = (3/16, 0)
      dk_1 = -1/4 (w_0 q_0 + w_1 q_1)              = (-3/16, -1/16)
    Row 0 has one slot (L = 0); row 1 has zero scores and a uniform teacher
    (L = 0)."""
    q, k, w = _example()
    S = np.array([[[0, -1], [0, 1], [0, 1]]], np.int32)
    p = np.array([[[5.0, 0.0], [2.0, 2.0], [1.0, 3.0]]], np.float32)
    loss, dq, dk, dw = oracle.indexer_kl(F32, q, None, k, None, w, S, p)
    assert loss[0, 0] == 0.0 and abs(loss[0, 1]) < 1e-15
    assert math.isclose(loss[0, 2], 0.25 * math.log(0.5) + 0.75 * math.log(1.5), rel_tol=1e-14)
    np.testing.assert_allclose(dw[0, 2], [0.25, -0.75], rtol=0, atol=1e-15)
    np.testing.assert_allclose(dq[0, 2], [[0.1875, -0.75], [-0.0625, -0.1875]], rtol=0, atol=1e-15)
    np.testing.assert_allclose(dk[0], [[0.1875, 0.0], [-0.1875, -0.0625], [0.0, 0.0]], rtol=0, atol=1e-15)
    assert not dq[0, :2].any() and not dw[0, :2].any()


def _random_problem(seed, B=1, n=24, HI=3, DI=5, k=6, holes=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, n, HI, DI)).astype(np.float32)
    kk = rng.standard_normal((B, n, DI)).astype(np.float32)
    w = rng.standard_normal((B, n, HI)).astype(np.float32)
    S = np.full((B, n, k), -1, np.int32)
    for b in range(B):
        for t in range(n):
            K = min(k, t + 1)
            S[b, t, :K] = np.sort(rng.choice(t + 1, K, replace=False))
            if holes and t % 5 == 4 and K > 2:
                S[b, t, 1] = -1          # an invalid slot
                S[b, t, 0] = t + 3       # beyond the causal limit: not selected
    p = rng.random((B, n, k)).astype(np.float32) + 0.05
    return q, kk, w, S, p


def _total_loss(q, kk, w, S, p):
    return float(oracle.indexer_kl(F32, q, None, kk, None, w, S, p)[0].sum())


@pytest.mark.parametrize("seed", [0, 1])
def test_gradient_matches_central_differences(seed):
    """Each checked coordinate is perturbed by +-h in float32; coordinates whose
    perturbation would flip the sign of some q_j . k_s (a ReLU kink) are
    skipped, so the loss is smooth in between."""
    q, kk, w, S, p = _random_problem(seed)
    loss, dq, dk, dw = oracle.indexer_kl(F32, q, None, kk, None, w, S, p)
    X = np.einsum("bthd,bsd->bths", q.astype(np.float64), kk.astype(np.float64))
    rng = np.random.default_rng(100 + seed)
    h = 1e-3
    checked = 0
    for name, arr, grad in (("q", q, dq), ("k", kk, dk), ("w", w, dw)):
        for _ in range(25):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            if name == "q":
                b, t, j, d = idx
                if (np.abs(X[b, t, j]) <= 2 * h * np.abs(kk[b, :, d])).any():
                    continue
            if name == "k":
                b, s, d = idx
                if (np.abs(X[b, :, :, s]) <= 2 * h * np.abs(q[b, :, :, d])).any():
                    continue
            plus, minus = arr.copy(), arr.copy()
            plus[idx] = np.float32(arr[idx] + h)
            minus[idx] = np.float32(arr[idx] - h)
            args = {"q": q, "k": kk, "w": w}
            lp = _total_loss(*(plus if nm == name else args[nm] for nm in ("q", "k", "w")), S, p)
            lm = _total_loss(*(minus if nm == name else args[nm] for nm in ("q", "k", "w")), S, p)
            fd = (lp - lm) / (float(plus[idx]) - float(minus[idx]))
            assert abs(fd - grad[idx]) <= 1e-5 * max(1.0, abs(grad[idx])), (name, idx, fd, grad[idx])
            checked += 1
    assert checked >= 40


def test_all_history_selection_is_the_dense_warmup_kl():
    """When S_t keeps every position 0..t, eq.(8) is eq.(7): the KL between the
    dense teacher and Softmax(I_t), here with one head, unit weight and
    non-negative inputs so that I = Q K^T (numpy), against scipy's relative
    entropy and softmax."""
    rng = np.random.default_rng(3)
    n, DI = 30, 7
    q = rng.random((1, n, 1, DI)).astype(np.float32)
    kk = rng.random((1, n, DI)).astype(np.float32)
    w = np.ones((1, n, 1), np.float32)
    S = np.full((1, n, n), -1, np.int32)
    p = np.zeros((1, n, n), np.float32)
    for t in range(n):
        S[0, t, : t + 1] = np.arange(t + 1)
        p[0, t, : t + 1] = rng.random(t + 1).astype(np.float32) + 0.01
    loss, _, _, _ = oracle.indexer_kl(F32, q, None, kk, None, w, S, p)
    I = q[0, :, 0].astype(np.float64) @ kk[0].astype(np.float64).T
    for t in range(n):
        P = p[0, t, : t + 1].astype(np.float64)
        ref = entropy(P / P.sum(), softmax(I[t, : t + 1]))
        assert math.isclose(loss[0, t], ref, rel_tol=1e-12, abs_tol=1e-15), t


def test_teacher_is_renormalised_by_its_kept_mass():
    """A teacher cut from a dense distribution (mass < 1 on S_t) gives the same
    loss and gradient as the same sub-vector renormalised to one, and scaling
    the teacher by a power of two changes nothing at all."""
    q, kk, w, S, p = _random_problem(4)
    base = oracle.indexer_kl(F32, q, None, kk, None, w, S, p)
    valid = (S >= 0) & (S <= np.arange(S.shape[1])[None, :, None])
    mass = np.where(valid, p, 0).sum(-1, keepdims=True)
    renorm = oracle.indexer_kl(F32, q, None, kk, None, w, S, (p / mass).astype(np.float32))
    scaled = oracle.indexer_kl(F32, q, None, kk, None, w, S, p * np.float32(8.0))
    for a, b, c in zip(base, renorm, scaled):
        # (p / mass rounded to float32: 1e-7 relative per entry)
        np.testing.assert_allclose(a, b, rtol=1e-5, atol=1e-7)
        np.testing.assert_array_equal(a, c)


def test_student_equal_to_teacher_gives_zero():
    """p = Softmax(I_{S_t}) (I from numpy with one head and non-negative
    inputs): the loss and every gradient vanish; otherwise the loss is
    positive (Gibbs' inequality)."""
    rng = np.random.default_rng(5)
    n, DI, k = 20, 4, 5
    q = rng.random((1, n, 1, DI)).astype(np.float32)
    kk = rng.random((1, n, DI)).astype(np.float32)
    w = np.ones((1, n, 1), np.float32)
    I = q[0, :, 0].astype(np.float64) @ kk[0].astype(np.float64).T
    S = np.full((1, n, k), -1, np.int32)
    p = np.zeros((1, n, k), np.float32)
    for t in range(n):
        K = min(k, t + 1)
        S[0, t, :K] = np.sort(rng.choice(t + 1, K, replace=False))
        p[0, t, :K] = softmax(I[t, S[0, t, :K]])
    loss, dq, dk, dw = oracle.indexer_kl(F32, q, None, kk, None, w, S, p)
    assert np.abs(loss).max() < 1e-7
    for g in (dq, dk, dw):
        assert np.abs(g).max() < 1e-6
    p2 = p.copy()
    p2[0, :, 0] *= 3.0
    loss2 = oracle.indexer_kl(F32, q, None, kk, None, w, S, p2)[0]
    assert (loss2[0, 1:] > 0).all()


def test_invalid_slots_and_relu_kink():
    """Slots that are -1 or beyond t are not part of S_t: the result equals
    that of the compacted selection.  A dot product of exactly zero takes
    ReLU'(0) = 0 (dyadic inputs make it exact)."""
    q, kk, w, S, p = _random_problem(6)
    base = oracle.indexer_kl(F32, q, None, kk, None, w, S, p)
    n, k = S.shape[1], S.shape[2]
    S2 = np.full_like(S, -1)
    p2 = np.zeros_like(p)
    for t in range(n):
        keep = (S[0, t] >= 0) & (S[0, t] <= t)
        m = int(keep.sum())
        S2[0, t, :m] = S[0, t][keep]
        p2[0, t, :m] = p[0, t][keep]
        p2[0, t, m:] = 123.0  # mass on slots that are not selected is ignored
    comp = oracle.indexer_kl(F32, q, None, kk, None, w, S2, p2)
    for a, b in zip(base, comp):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-15)
    # kink: key 1 is orthogonal to the only head's query
    q = np.zeros((1, 2, 1, 2), np.float32)
    q[0, 1, 0] = [1.0, 0.0]
    kk = np.array([[[1.0, 0.0], [0.0, 2.0]]], np.float32)
    w = np.ones((1, 2, 1), np.float32)
    S = np.array([[[0, -1], [0, 1]]], np.int32)
    p = np.array([[[1, 0], [1, 1]]], np.float32)
    loss, dq, dk, dw = oracle.indexer_kl(F32, q, None, kk, None, w, S, p)
    # I = (1, 0): R = (e, 1)/(e + 1), P = (1/2, 1/2), g_0 = R_0 - 1/2
    g0 = math.e / (math.e + 1) - 0.5
    np.testing.assert_allclose(dq[0, 1, 0], [g0, 0.0], rtol=1e-14)  # no term from key 1
    np.testing.assert_allclose(dk[0, 1], [0.0, 0.0])
    np.testing.assert_allclose(dw[0, 1], [g0 * 1.0], rtol=1e-14)


def test_quantised_inputs_use_the_decoded_values():
    """fp8 (unit scales) and bf16 storage give exactly the result of the same
    decoded values passed as float32 (the decoders are pinned to torch's casts
    elsewhere)."""
    q, kk, w, S, p = _random_problem(7, DI=8)
    for dt in (synth.DT_BF16, synth.DT_FP8):
        if dt == synth.DT_FP8:
            qs = torch.from_numpy(q).to(torch.float8_e4m3fn)
            ks = torch.from_numpy(kk).to(torch.float8_e4m3fn)
            qsc, ksc = np.ones(q.shape[:2], np.float32), np.ones(kk.shape[:2], np.float32)
            q_store, k_store = qs.view(torch.uint8).numpy(), ks.view(torch.uint8).numpy()
        else:
            qs = torch.from_numpy(q).to(torch.bfloat16)
            ks = torch.from_numpy(kk).to(torch.bfloat16)
            qsc = ksc = None
            q_store, k_store = synth.storage_to_numpy(qs), synth.storage_to_numpy(ks)
        got = oracle.indexer_kl(dt, q_store, qsc, k_store, ksc, w, S, p)
        ref = oracle.indexer_kl(F32, qs.float().numpy(), None, ks.float().numpy(), None, w, S, p)
        for a, b in zip(got, ref):
            np.testing.assert_array_equal(a, b)


def test_magnitude_sums_bound_the_results():
    """The optional magnitude sums (used to scale test tolerances) change no
    result and bound each result's absolute value; on non-negative inputs with
    one head and unit weight every mask is open and the dq magnitude is
    sum_i (R_i + P_i) |k_i| exactly."""
    q, kk, w, S, p = _random_problem(8)
    base = oracle.indexer_kl(F32, q, None, kk, None, w, S, p)
    res = oracle.indexer_kl(F32, q, None, kk, None, w, S, p, want_mags=True)
    for a, b in zip(base, res[:4]):
        np.testing.assert_array_equal(a, b)
    for val, mag in zip(res[:4], res[4:8]):
        assert (np.abs(val) <= mag * (1 + 1e-12) + 1e-300).all()
    rng = np.random.default_rng(9)
    n, DI, k = 12, 3, 4
    q = rng.random((1, n, 1, DI)).astype(np.float32) + 0.1
    kk = rng.random((1, n, DI)).astype(np.float32) + 0.1
    w = np.ones((1, n, 1), np.float32)
    S = np.full((1, n, k), -1, np.int32)
    for t in range(n):
        K = min(k, t + 1)
        S[0, t, :K] = np.sort(rng.choice(t + 1, K, replace=False))
    p = rng.random((1, n, k)).astype(np.float32) + 0.1
    _, _, _, _, _, dqm, _, _, dqk, dkk = oracle.indexer_kl(F32, q, None, kk, None, w, S, p, want_mags=True)
    assert not dqk.any() and not dkk.any()   # positive inputs: every dot product is far from the kink
    I = q[0, :, 0].astype(np.float64) @ kk[0].astype(np.float64).T
    t = n - 1
    sel = S[0, t]
    R = softmax(I[t, sel])
    P = p[0, t].astype(np.float64) / p[0, t].astype(np.float64).sum()
    np.testing.assert_allclose(dqm[0, t, 0], ((R + P)[:, None] * np.abs(kk[0, sel].astype(np.float64))).sum(0),
                               rtol=1e-12)


def test_kink_band_holds_exactly_the_near_zero_terms():
    """A dot product that is exactly zero lies in the band (its term is
    reported at full weight there and not counted in dq); one far from zero
    does not."""
    q = np.zeros((1, 2, 1, 2), np.float32)
    q[0, 1, 0] = [1.0, 0.0]
    kk = np.array([[[1.0, 0.0], [0.0, 2.0]]], np.float32)
    w = np.full((1, 2, 1), 0.5, np.float32)
    S = np.array([[[0, -1], [0, 1]]], np.int32)
    p = np.array([[[1, 0], [1, 1]]], np.float32)
    res = oracle.indexer_kl(F32, q, None, kk, None, w, S, p, want_mags=True)
    dq, dqk, dkk = res[1], res[8], res[9]
    # row 1: I = (0.5, 0), R = (e^.5, 1)/(e^.5 + 1), P = (1/2, 1/2); key 1 is orthogonal to q
    R1 = 1.0 / (math.exp(0.5) + 1.0)
    np.testing.assert_allclose(dqk[0, 1, 0], [0.0, (R1 + 0.5) * 0.5 * 2.0], rtol=1e-14)
    np.testing.assert_allclose(dkk[0, 1], [(R1 + 0.5) * 0.5 * 1.0, 0.0], rtol=1e-14)
    assert dq[0, 1, 0, 1] == 0.0
    assert not dkk[0, 0].any()
