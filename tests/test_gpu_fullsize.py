"""Parity at the full benchmark sizes, in the launch configuration bench.py
times, against the oracle.

Workloads (seeded, synthetic, the shapes of the five benchmark
configurations):
  * prefill indexer + top-k, B=1, n=8192, H^I=64, d^I=128, k=2048, bf16:
    EVERY query row against the oracle;
  * n=32768 and n=131072, fp8 e4m3 with per-token scales: the stratified
    sample t in {0, k-2, k-1, k, n-1}, every probe row (the queries with
    planted keys) and uniform rows up to 512 rows or more;
  * sparse attention prefill (H=128, Dqk=576, Dv=512, bf16) at n=32768 and
    n=131072 on the GPU's own selection (two-layer check), sampled rows;
  * one decode step of 64 ragged sequences, L ~ U[16384, 131072]: EVERY
    sequence (scores, the exact selection on the GPU's scores, the margin
    rule against the oracle's own selection, attention).

Every check prints the statistics of the selection rule: the fraction of
identical slots, the number of rows that differ, the worst distance of a
differing position from the K-th score relative to the tolerance, the worst
score error relative to its tolerance, and the attention error next to the
RMS of the output.  Inputs are drawn on the GPU from the seeded generators and
copied to the host for the oracle.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import parity
import token_level_sparse_lightning_amd as tl
from token_level_sparse_lightning_amd import synth
from tests.gpu_util import DEV, announce, host, stratified_rows

pytestmark = pytest.mark.gpu

K = 2048


def stat(msg):
    print(f"[parity] {msg}", flush=True)


def _prefill(n, dt, seed, plant_max_dist=None):
    inp = synth.indexer_prefill(1, n, 64, 128, dt, seed, planted=True, plant_max_dist=plant_max_dist, device=DEV)
    ws = torch.empty(tl.index_prefill_workspace_bytes(inp.q, inp.k, inp.w, K, inp.q_scale, inp.k_scale),
                     dtype=torch.uint8, device=DEV)
    S, Ss = tl.index_prefill(inp.q, inp.k, inp.w, K, q_scale=inp.q_scale, k_scale=inp.k_scale,
                             want_scores=True, workspace=ws)
    torch.cuda.synchronize()
    del ws
    return inp, S, Ss


def _structure_every_row(Sh, k):
    """Row t holds min(k, t+1) strictly ascending positions in [0, t], then -1
    (checked for every row, in blocks)."""
    n = Sh.shape[0]
    col = np.arange(k)[None, :]
    for a in range(0, n, 4096):
        blk = Sh[a:a + 4096]
        t = np.arange(a, a + len(blk))[:, None]
        valid = col < np.minimum(k, t + 1)
        assert (~valid | ((blk >= 0) & (blk <= t))).all(), "position outside [0, t]"
        assert (valid | (blk == -1)).all(), "padding is not -1"
        assert (~valid[:, 1:] | (np.diff(blk, axis=1) > 0)).all(), "positions not strictly ascending"


def _check_prefill(name, inp, S, Ss, n, rows):
    Sh = S[0].cpu().numpy()
    Ssh = Ss[0].cpu().numpy()
    _structure_every_row(Sh, K)
    S_o, _, sc, mg = oracle.index_prefill_rows(inp.dt, host(inp.q), host(inp.q_scale), host(inp.k),
                                               host(inp.k_scale), host(inp.w), K, rows, want_scores=True)
    rep = parity.check_selection(Sh[rows], S_o, rows, K, sc)
    worst, wt = parity.check_scores(Sh[rows], Ssh[rows], rows, K, sc, mg, lowp=True)
    hit = tot = 0
    for (_, t), pos in inp.probes.items():
        sel = set(Sh[t][Sh[t] >= 0].tolist())
        hit += sum(p in sel for p in pos)
        tot += len(pos)
    stat(f"{name}: {rep.summary()} score_violation_ratio={worst:.3g} (row {wt}); "
         f"planted-key recall {hit / max(tot, 1):.4f} (diagnostic)")
    assert rep.ok(), rep.summary()
    assert worst <= 1.0, (worst, wt)
    return Sh


def _check_attention_rows(name, q, kv, S, rows, scale, Dv):
    """Attention on the GPU's own selection S for the listed rows of batch row
    0; q, kv and S stay on the device, only the sampled rows (and the entries)
    are copied."""
    out, lse = tl.sparse_attn_prefill(q, kv, S, scale, Dv, want_lse=True)
    torch.cuda.synchronize()
    ridx = torch.as_tensor(rows, device=DEV)
    got = out[0].index_select(0, ridx).float().cpu().numpy()
    got_lse = lse[0].index_select(0, ridx).cpu().numpy()
    q_rows = host(q[0].index_select(0, ridx))
    S_rows = S[0].index_select(0, ridx).cpu().numpy()
    del out, lse
    ref, ref_lse = oracle.sparse_attn_rows(synth.DT_BF16, q_rows, host(kv[0]), S_rows, rows, scale, Dv)
    err = float(np.abs(got - ref).max())
    rms = float(np.sqrt((ref ** 2).mean()))
    lse_err = float(np.abs(got_lse - ref_lse).max())
    stat(f"{name}: rows={len(rows)} max_abs_err={err:.3g} (bound {parity.ATTN_ATOL_BF16}) "
         f"output_rms={rms:.3g} err/rms={err / rms:.3g} lse_max_abs_err={lse_err:.3g}")
    assert err <= parity.ATTN_ATOL_BF16, err
    np.testing.assert_allclose(got_lse, ref_lse, rtol=1e-4, atol=1e-4)


def test_fullsize_prefill_bf16_8192_every_row():
    n = 8192
    announce(f"full-size prefill bf16 n={n}, every row")
    inp, S, Ss = _prefill(n, synth.DT_BF16, 2)
    _check_prefill(f"prefill bf16 n={n} (all rows)", inp, S, Ss, n, np.arange(n, dtype=np.int64))


def test_fullsize_prefill_fp8_32768_and_attention():
    n = 32768
    announce(f"full-size prefill fp8 n={n}")
    inp, S, Ss = _prefill(n, synth.DT_FP8, 3)
    probes = [t for (_, t) in inp.probes]
    rows = stratified_rows(n, K, probes, uniform=512 - 5 - len(probes), seed=2)
    _check_prefill(f"prefill fp8 n={n} (stratified)", inp, S, Ss, n, rows)
    del Ss, inp
    torch.cuda.empty_cache()
    announce(f"full-size sparse attention prefill n={n}")
    H, Dqk, Dv = 128, 576, 512
    q, kv = synth.attn_prefill(1, n, H, Dqk, synth.DT_BF16, 3, device=DEV)
    arows = stratified_rows(n, K, probes[::4], uniform=96, seed=4)
    _check_attention_rows(f"attention prefill n={n}", q, kv, S, arows, 1.0 / math.sqrt(Dqk), Dv)


def test_fullsize_prefill_fp8_131072_and_attention():
    n = 131072
    announce(f"full-size prefill fp8 n={n}")
    inp, S, Ss = _prefill(n, synth.DT_FP8, 5, plant_max_dist=100000)
    probes = [t for (_, t) in inp.probes]
    rows = stratified_rows(n, K, probes, uniform=64, seed=3)
    assert len(rows) >= 512
    _check_prefill(f"prefill fp8 n={n} (stratified)", inp, S, Ss, n, rows)
    del Ss, inp
    torch.cuda.empty_cache()
    announce(f"full-size sparse attention prefill n={n}")
    H, Dqk, Dv = 128, 576, 512
    q, kv = synth.attn_prefill(1, n, H, Dqk, synth.DT_BF16, 5, device=DEV)
    arows = stratified_rows(n, K, probes[::16], uniform=24, seed=5)
    _check_attention_rows(f"attention prefill n={n}", q, kv, S, arows, 1.0 / math.sqrt(Dqk), Dv)


def test_fullsize_decode_step_every_sequence():
    B, HI, DI, H, Dqk, Dv = 64, 64, 128, 128, 576, 512
    lengths = synth.decode_lengths(B, 16384, 131072, 5)
    announce(f"full-size decode step sumL={int(lengths.sum())}, every sequence")
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
    Sh, Ssh, sch = S.cpu().numpy(), Ss.cpu().numpy(), sc.cpu().numpy()
    # scores of every cached key of every sequence
    ref, mag = oracle.index_decode(2, host(di.q), host(di.q_scale), host(di.k), host(di.k_scale), host(di.w), cuh)
    sv = parity.check_score_vector(sch, ref, mag, lowp=True)
    # the selection on the GPU's own scores is exact (topk_select is exact on its input)
    S_g, Ss_g = oracle.topk_rows(sch, cuh[:-1], lengths, K)
    exact_rows = int((S_g == Sh).all(axis=1).sum())
    # and the oracle's own selection agrees at the margin
    S_o, _ = oracle.topk_rows(ref, cuh[:-1], lengths, K)
    rep = parity.check_selection(Sh, S_o, lengths - 1, K, [ref[cuh[b]:cuh[b + 1]] for b in range(B)])
    stat(f"decode scores: violation_ratio={sv:.3g}; selection on the GPU scores: {exact_rows}/{B} rows "
         f"identical; vs the oracle's selection: {rep.summary()}")
    assert sv <= 1.0
    np.testing.assert_array_equal(Sh, S_g)
    np.testing.assert_array_equal(Ssh, Ss_g)
    assert rep.ok(), rep.summary()
    del di, sc, Ss
    # attention on the GPU's selection, every sequence
    r, rl = oracle.sparse_attn_decode(1, host(qa), host(kva), cuh, Sh, scale, Dv)
    got = out.float().cpu().numpy()
    err = float(np.abs(got - r).max())
    rms = float(np.sqrt((r ** 2).mean()))
    lerr = float(np.abs(lse.cpu().numpy() - rl).max())
    stat(f"decode attention: max_abs_err={err:.3g} (bound {parity.ATTN_ATOL_BF16}) output_rms={rms:.3g} "
         f"err/rms={err / rms:.3g} lse_max_abs_err={lerr:.3g}")
    assert err <= parity.ATTN_ATOL_BF16
    np.testing.assert_allclose(lse.cpu().numpy(), rl, rtol=1e-4, atol=1e-4)
