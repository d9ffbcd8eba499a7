"""Parity at the full benchmark sizes, in the launch configuration bench.py
times, on sampled outputs the oracle computes one by one.

Workloads: prefill indexer + top-k at n=8192 (bf16), n=32768 and n=131072
(fp8); sparse attention prefill at n=32768 (H=128, 576/512, bf16) on the GPU's
own selection; one ragged decode step of 64 sequences with L ~ U[16384,131072].
Inputs are drawn on the GPU from the seeded generators and copied to the host
for the oracle.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import parity
import token_level_sparse_lightning_amd as tl
from token_level_sparse_lightning_amd import synth
from tests.gpu_util import DEV, announce, host, sample_rows

pytestmark = pytest.mark.gpu

K = 2048


def _prefill(n, dt, seed, plant_max_dist=None):
    inp = synth.indexer_prefill(1, n, 64, 128, dt, seed, planted=True, plant_max_dist=plant_max_dist, device=DEV)
    ws = torch.empty(tl.index_prefill_workspace_bytes(inp.q, inp.k, inp.w, K, inp.q_scale, inp.k_scale),
                     dtype=torch.uint8, device=DEV)
    S, Ss = tl.index_prefill(inp.q, inp.k, inp.w, K, q_scale=inp.q_scale, k_scale=inp.k_scale,
                             want_scores=True, workspace=ws)
    torch.cuda.synchronize()
    return inp, S, Ss


def _check_prefill(inp, S, Ss, n, rows):
    Sh = S[0].cpu().numpy()
    Ssh = Ss[0].cpu().numpy()
    # structure of every row (host-side, exact)
    bad = [t for t in range(0, n, max(1, n // 4096)) if parity.check_structure(Sh[t], t, K)]
    assert not bad, bad[:5]
    S_o, _, sc, mg = oracle.index_prefill_rows(inp.dt, host(inp.q), host(inp.q_scale), host(inp.k),
                                               host(inp.k_scale), host(inp.w), K, rows, want_scores=True)
    rep = parity.check_selection(Sh[rows], S_o, rows, K, sc)
    assert rep.ok(), rep.summary()
    worst, wt = parity.check_scores(Sh[rows], Ssh[rows], rows, K, sc, mg, lowp=True)
    assert worst <= 1.0, (worst, wt)
    # planted keys are found at the probes
    hit = tot = 0
    for (_, t), pos in inp.probes.items():
        sel = set(Sh[t][Sh[t] >= 0].tolist())
        hit += sum(p in sel for p in pos)
        tot += len(pos)
    return rep, hit / max(tot, 1)


def test_fullsize_prefill_bf16_8192():
    n = 8192
    announce(f"full-size prefill bf16 n={n}")
    inp, S, Ss = _prefill(n, synth.DT_BF16, 2)
    rows = sample_rows(n, K, 24, seed=1, extra=[255, 4351, 4352, 8191])
    rep, recall = _check_prefill(inp, S, Ss, n, rows)
    print(f"planted-key recall {recall:.3f} (diagnostic)", flush=True)


def test_fullsize_prefill_fp8_32768_and_attention():
    n = 32768
    announce(f"full-size prefill fp8 n={n}")
    inp, S, Ss = _prefill(n, synth.DT_FP8, 3)
    rows = sample_rows(n, K, 16, seed=2, extra=[4351, 4352, 32767])
    _check_prefill(inp, S, Ss, n, rows)
    del Ss
    announce(f"full-size sparse attention prefill n={n}")
    H, Dqk, Dv = 128, 576, 512
    q, kv = synth.attn_prefill(1, n, H, Dqk, synth.DT_BF16, 3, device=DEV)
    scale = 1.0 / math.sqrt(Dqk)
    out, lse = tl.sparse_attn_prefill(q, kv, S, scale, Dv, want_lse=True)
    torch.cuda.synchronize()
    # row t of a prefill batch sees keys 0..t: the decode form of the oracle with
    # a cache of length t+1 evaluates exactly that row
    for t in [0, 1, 2047, 2048, 16000, 32767]:
        cu1 = np.array([0, t + 1])
        r, rl = oracle.sparse_attn_decode(1, host(q[0, t:t + 1]), host(kv[0, : t + 1]), cu1,
                                          S[0, t:t + 1].cpu().numpy(), scale, Dv)
        got = out[0, t].float().cpu().numpy()
        assert np.abs(got - r[0]).max() <= parity.ATTN_ATOL_BF16, (t, np.abs(got - r[0]).max())
        np.testing.assert_allclose(lse[0, t].cpu().numpy(), rl[0], rtol=1e-4, atol=1e-4)


def test_fullsize_prefill_fp8_131072():
    n = 131072
    announce(f"full-size prefill fp8 n={n}")
    inp, S, Ss = _prefill(n, synth.DT_FP8, 5, plant_max_dist=100000)
    rows = sample_rows(n, K, 8, seed=3, extra=[4352, 131071])
    _, recall = _check_prefill(inp, S, Ss, n, rows)
    print(f"planted-key recall {recall:.3f} (diagnostic)", flush=True)


def test_fullsize_decode_step():
    B, HI, DI, H, Dqk, Dv = 64, 64, 128, 128, 576, 512
    lengths = synth.decode_lengths(B, 16384, 131072, 5)
    announce(f"full-size decode step sumL={int(lengths.sum())}")
    di = synth.indexer_decode(lengths, HI, DI, synth.DT_FP8, 5, device=DEV)
    qa, kva = synth.attn_decode(lengths, H, Dqk, synth.DT_BF16, 5, device=DEV)
    cu = di.cu_seqlens
    max_len = int(lengths.max())
    sc = tl.index_decode(di.q, di.k, di.w, cu, max_len, q_scale=di.q_scale, k_scale=di.k_scale)
    row_len = torch.as_tensor(lengths, dtype=torch.int32, device=DEV)
    S, Ss = tl.topk_select(sc, cu[:-1].contiguous(), row_len, K, max_len, want_scores=True)
    scale = 1.0 / math.sqrt(Dqk)
    out, lse = tl.sparse_attn_decode(qa, kva, cu, S, scale, Dv, want_lse=True)
    torch.cuda.synchronize()
    cuh = cu.cpu().numpy()
    seqs = [0, 17, 42, 63]
    Sh, Ssh, sch = S.cpu().numpy(), Ss.cpu().numpy(), sc.cpu().numpy()
    for b in seqs:
        lo, hi = int(cuh[b]), int(cuh[b + 1])
        cu1 = np.array([0, hi - lo])
        ref, mag = oracle.index_decode(2, host(di.q[b:b + 1]), host(di.q_scale[b:b + 1]), host(di.k[lo:hi]),
                                       host(di.k_scale[lo:hi]), host(di.w[b:b + 1]), cu1)
        assert parity.check_score_vector(sch[lo:hi], ref, mag, lowp=True) <= 1.0
        # selection from the GPU's own scores must be exact (topk_select is exact on its input)
        S_o, Ss_o = oracle.topk_rows(sch[lo:hi], [0], [hi - lo], K)
        np.testing.assert_array_equal(Sh[b], S_o[0])
        np.testing.assert_array_equal(Ssh[b], Ss_o[0])
        # and the oracle's own selection agrees at the margin
        rep = parity.check_selection(Sh[b:b + 1], oracle.topk_rows(ref, [0], [hi - lo], K)[0], [hi - lo - 1], K,
                                     [ref])
        assert rep.ok(), rep.summary()
        # attention on the GPU's selection
        r, rl = oracle.sparse_attn_decode(1, host(qa[b:b + 1]), host(kva[lo:hi]), cu1, Sh[b:b + 1], scale, Dv)
        assert np.abs(out[b].float().cpu().numpy() - r[0]).max() <= parity.ATTN_ATOL_BF16
        np.testing.assert_allclose(lse[b].cpu().numpy(), rl[0], rtol=1e-4, atol=1e-4)
    hit = tot = 0
    for b, pos in di.planted.items():
        sel = set(Sh[b][Sh[b] >= 0].tolist())
        hit += sum(p in sel for p in pos)
        tot += len(pos)
    print(f"planted-key recall {hit / tot:.3f} (diagnostic)", flush=True)
