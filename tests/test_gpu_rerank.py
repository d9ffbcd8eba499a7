"""GPU parity of index_prefill_rerank (fp8 coarse recall, then a bf16 re-rank;
DSA page section 2, the quantised key cache paragraph) against the oracle.

* Integer-valued inputs (bf16 integers in [-20, 20], their fp8 quantisation at
  unit scale, weights in quarters): every coarse and fine score is exact in
  fp32 on both sides, so candidates, selection and scores must match bit for
  bit -- and since fp8 rounds 17 and 19, the two precisions differ.
* All-history candidates (k_coarse >= n): the result is index_prefill on the
  bf16 inputs, bit for bit.
* Normal inputs with planted keys: the candidates follow the selection rule's
  margin against the oracle's coarse scores, and the re-ranked selection
  follows it against the oracle's fine scores over the GPU's own candidates.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import parity
import token_level_sparse_lightning_amd as tl
from token_level_sparse_lightning_amd import synth
from tests.gpu_util import DEV, announce, host, sample_rows, to_dev

pytestmark = pytest.mark.gpu
BF16, FP8 = synth.DT_BF16, synth.DT_FP8


def _integer_inputs(n, HI, DI, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randint(-20, 21, (1, n, HI, DI), generator=g).float()
    k = torch.randint(-20, 21, (1, n, DI), generator=g).float()
    w = (torch.randint(-4, 5, (1, n, HI), generator=g).float() * 0.25).contiguous()
    q8 = q.to(torch.float8_e4m3fn).view(torch.uint8).contiguous()
    k8 = k.to(torch.float8_e4m3fn).view(torch.uint8).contiguous()
    one = torch.ones(1, n)
    return q8, one, k8, one.clone(), q.to(torch.bfloat16).contiguous(), k.to(torch.bfloat16).contiguous(), w


def test_rerank_exact_on_integer_inputs():
    n, HI, DI, k, kc = 600, 8, 128, 32, 128
    q8, qs, k8, ks, qb, kb, w = _integer_inputs(n, HI, DI, 61)
    announce("index_prefill_rerank integer inputs")
    S, Ss, C = tl.index_prefill_rerank(to_dev(q8), to_dev(qs), to_dev(k8), to_dev(ks), to_dev(qb), to_dev(kb),
                                       to_dev(w), k, kc, want_scores=True, want_C=True)
    torch.cuda.synchronize()
    rows = np.arange(n)
    S_o, Ss_o, C_o = oracle.index_prefill_rerank_rows(FP8, host(q8), host(qs), host(k8), host(ks), BF16, host(qb),
                                                      host(kb), host(w), k, kc, rows)
    np.testing.assert_array_equal(C[0].cpu().numpy(), C_o)
    np.testing.assert_array_equal(S[0].cpu().numpy(), S_o)
    np.testing.assert_array_equal(Ss[0].cpu().numpy(), Ss_o)
    # the two precisions really differ: re-ranking changed the selection of
    # some rows against the fp8 selection with budget k
    S8, _, _, _ = oracle.index_prefill_rows(FP8, host(q8), host(qs), host(k8), host(ks), host(w), k, rows)
    assert (S_o != S8).any()


def test_rerank_with_all_history_candidates_is_the_bf16_selection():
    n, k = 1000, 64
    inp = synth.indexer_prefill(1, n, 64, 128, BF16, seed=62, planted=True)
    q8, qs = synth.quantize_fp8_rows(inp.q.float(), 2)
    k8, ks = synth.quantize_fp8_rows(inp.k.float(), 1)
    announce("index_prefill_rerank all-history candidates")
    S, Ss, _ = tl.index_prefill_rerank(to_dev(q8), to_dev(qs), to_dev(k8), to_dev(ks), to_dev(inp.q), to_dev(inp.k),
                                       to_dev(inp.w), k, n, want_scores=True)
    S_b, Ss_b = tl.index_prefill(to_dev(inp.q), to_dev(inp.k), to_dev(inp.w), k, want_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(S, S_b) and torch.equal(Ss, Ss_b)


def test_rerank_normal_inputs_margin_rule():
    n, k, kc = 3000, 256, 512
    inp = synth.indexer_prefill(1, n, 64, 128, BF16, seed=63, planted=True)
    q8, qs = synth.quantize_fp8_rows(inp.q.float(), 2)
    k8, ks = synth.quantize_fp8_rows(inp.k.float(), 1)
    announce("index_prefill_rerank normal inputs")
    S, Ss, C = tl.index_prefill_rerank(to_dev(q8), to_dev(qs), to_dev(k8), to_dev(ks), to_dev(inp.q), to_dev(inp.k),
                                       to_dev(inp.w), k, kc, want_scores=True, want_C=True)
    torch.cuda.synchronize()
    S, Ss, C = S[0].cpu().numpy(), Ss[0].cpu().numpy(), C[0].cpu().numpy()
    rows = sample_rows(n, kc, 40, seed=6, extra=[255, 511, 767, 2999])
    # candidates: the coarse selection, within the margin of the oracle's fp8 scores
    C_o, _, sc8, _ = oracle.index_prefill_rows(FP8, host(q8), host(qs), host(k8), host(ks), host(inp.w), kc, rows,
                                               want_scores=True)
    rep_c = parity.check_selection(C[rows], C_o, rows, kc, sc8)
    # re-rank over the GPU's own candidates, against the oracle's bf16 scores
    S_o, Ss_o = oracle.rerank_rows(BF16, host(inp.q), host(inp.k), host(inp.w), rows, C[rows], k)
    _, _, scb, mgb = oracle.index_prefill_rows(BF16, host(inp.q), None, host(inp.k), None, host(inp.w), 1, rows,
                                               want_scores=True)
    cand_scores = np.full_like(scb, -np.inf)
    for i, t in enumerate(rows):
        valid = C[t][C[t] >= 0]
        cand_scores[i, valid] = scb[i, valid]
    rep_s = parity.check_selection(S[rows], S_o, rows, k, cand_scores)
    worst, wt = parity.check_scores(S[rows], Ss[rows], rows, k, scb, mgb, lowp=True)
    print(f"[parity] rerank candidates: {rep_c.summary()}; re-ranked: {rep_s.summary()}; score ratio {worst:.3g}",
          flush=True)
    assert rep_c.ok(), rep_c.summary()
    assert rep_s.ok(), rep_s.summary()
    assert worst <= 1.0
    # every selected position is a candidate
    for t in rows:
        assert set(S[t][S[t] >= 0].tolist()) <= set(C[t][C[t] >= 0].tolist())
