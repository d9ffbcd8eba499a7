"""Pins of the oracle's coarse-recall-then-re-rank selection (CPU only).

DSA page, section 2 (the paragraph on the quantised key cache): recall a
larger candidate set with the FP8 indexer, then rank it with a
higher-precision indexer.  ``oracle.rerank_rows`` is tied to: the plain fine
selection (when the candidates are all of the history), the coarse selection
(when the candidate budget equals k, re-ranking cannot change the set),
brute force with numpy matmul scores and Python's sort, and the page's worked
example.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from token_level_sparse_lightning_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")
F32, BF16, FP8 = synth.DT_F32, synth.DT_BF16, synth.DT_FP8
sn = synth.storage_to_numpy


def _two_precisions(n, HI, DI, seed):
    """Fine inputs in bf16 and their fp8 quantisation (per-token scales)."""
    inp = synth.indexer_prefill(1, n, HI, DI, BF16, seed)
    qf = inp.q.float()
    kf = inp.k.float()
    q8, qs = synth.quantize_fp8_rows(qf, 2)
    k8, ks = synth.quantize_fp8_rows(kf, 1)
    return inp, (sn(q8), sn(qs), sn(k8), sn(ks))


def test_all_history_candidates_give_the_fine_selection():
    n, k = 300, 16
    inp, (q8, qs, k8, ks) = _two_precisions(n, 8, 128, 1)
    rows = np.arange(n)
    S, Ss, C = oracle.index_prefill_rerank_rows(FP8, q8, qs, k8, ks, BF16, sn(inp.q), sn(inp.k), sn(inp.w), k, n,
                                                rows)
    S_f, Ss_f, _, _ = oracle.index_prefill_rows(BF16, sn(inp.q), None, sn(inp.k), None, sn(inp.w), k, rows)
    np.testing.assert_array_equal(S, S_f)
    np.testing.assert_array_equal(Ss, Ss_f)


def test_candidate_budget_k_keeps_the_coarse_set():
    n, k = 300, 16
    inp, (q8, qs, k8, ks) = _two_precisions(n, 8, 128, 2)
    rows = np.arange(n)
    S, Ss, C = oracle.index_prefill_rerank_rows(FP8, q8, qs, k8, ks, BF16, sn(inp.q), sn(inp.k), sn(inp.w), k, k,
                                                rows)
    np.testing.assert_array_equal(S, C)
    # and the slots carry the fine scores
    _, _, sc, _ = oracle.index_prefill_rows(BF16, sn(inp.q), None, sn(inp.k), None, sn(inp.w), n, rows,
                                            want_scores=True)
    for r in range(n):
        K = min(k, r + 1)
        np.testing.assert_array_equal(Ss[r, :K], sc[r, S[r, :K]])


@pytest.mark.parametrize("seed", [3, 4])
def test_rerank_brute_force(seed):
    """One head, unit weight, non-negative inputs: fine scores are Q K^T
    (numpy); candidates with holes, out-of-range and repeated entries."""
    rng = np.random.default_rng(seed)
    n, DI, k, kc = 40, 6, 5, 12
    q = rng.random((1, n, 1, DI)).astype(np.float32)
    kk = rng.random((1, n, DI)).astype(np.float32)
    kk[0, 7] = kk[0, 3]                          # a tie between positions 3 and 7
    w = np.ones((1, n, 1), np.float32)
    rows = np.arange(n)
    C = np.full((n, kc), -1, np.int32)
    for t in range(n):
        m = min(kc, t + 1)
        C[t, :m] = rng.choice(t + 1, m, replace=False)
        if t > 10:
            C[t, 0] = t + 4                      # beyond t: not a candidate
            C[t, 1] = C[t, 2]                    # repeated
    S, Ss = oracle.rerank_rows(F32, q, kk, w, rows, C, k)
    I = q[0, :, 0].astype(np.float64) @ kk[0].astype(np.float64).T
    for t in range(n):
        cand = sorted({int(c) for c in C[t] if 0 <= c <= t})
        order = sorted(cand, key=lambda s: (-float(np.float32(I[t, s])), s))
        want = sorted(order[:k])
        assert S[t, :len(want)].tolist() == want
        assert (S[t, len(want):] == -1).all()
        np.testing.assert_array_equal(Ss[t, :len(want)], I[t, want].astype(np.float32))


def test_worked_example_rerank():
    """The page's example with equal coarse and fine inputs (small integers,
    exact in fp8 at unit scale): candidates k' = 3 re-ranked to k = 2 give
    positions {0, 1}; k = 1 gives {0} (the 1.5 / 1.5 tie)."""
    with open(GOLDEN) as f:
        ex = json.load(f)["indexer"]
    q = np.zeros((1, 3, 2, 2), np.float32)
    q[0, 2] = ex["q"]
    kk = np.array(ex["keys"], np.float32)[None]
    w = np.zeros((1, 3, 2), np.float32)
    w[0, 2] = ex["w"]
    q8 = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    k8 = torch.from_numpy(kk).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    one = np.ones((1, 3), np.float32)
    for k, want in ((2, [0, 1]), (1, [0])):
        S, Ss, C = oracle.index_prefill_rerank_rows(FP8, q8, one, k8, one, F32, q, kk, w, k, 3, [2])
        assert S[0].tolist() == want
        assert C[0].tolist() == [0, 1, 2]
