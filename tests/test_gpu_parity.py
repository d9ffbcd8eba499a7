"""GPU parity of every entry point of the C ABI against the CPU oracle.

Sizes are small enough for the oracle to finish in seconds while spanning
several tiles and a ragged tail; full-size configurations are covered by
tests/test_gpu_fullsize.py on sampled rows.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import parity
import token_level_sparse_lightning_amd as tl
from token_level_sparse_lightning_amd import synth
from tests.gpu_util import DEV, announce, host, sample_rows, to_dev

pytestmark = pytest.mark.gpu

F32, BF16, FP8 = synth.DT_F32, synth.DT_BF16, synth.DT_FP8


# ---------------------------------------------------------------------------
# topk_select
# ---------------------------------------------------------------------------
def _score_rows(seed):
    rng = np.random.default_rng(seed)
    # (140001: several load batches per row, and past the position bitmap of the
    # in-LDS path, so it is selected from the full row)
    lens = [0, 1, 5, 63, 64, 65, 100, 1000, 2047, 2048, 2049, 140001, 5000, 4000, 3500, 20000, 20000, 9000]
    rows = []
    for i, L in enumerate(lens):
        if i in (len(lens) - 5, len(lens) - 4):
            # fits the candidate buffer whole: 1500 distinct high scores over a
            # block of exact ties (+0 and -0 mixed in the second row), so the
            # selection boundary falls inside a bin of thousands of equal keys
            r = np.zeros(L, np.float32)
            hi = rng.choice(L, 1500, replace=False)
            r[hi] = 5.0 + rng.standard_normal(1500).astype(np.float32)
            if i == len(lens) - 4:
                r[r == 0] = np.where(rng.random((r == 0).sum()) < 0.5, -0.0, 0.0)
        elif i == len(lens) - 3:
            r = np.zeros(L, np.float32)                       # one giant tie
        elif i == len(lens) - 2:
            r = rng.integers(-3, 4, L).astype(np.float32)     # 7 values, huge ties
            r[r == 0] = np.where(rng.random((r == 0).sum()) < 0.5, -0.0, 0.0)
        else:
            r = rng.standard_normal(L).astype(np.float32)
            r[rng.random(L) < 0.05] = 0.5                     # a few ties
        rows.append(r)
    starts = np.concatenate([[0], np.cumsum([len(r) for r in rows])[:-1]]).astype(np.int64)
    # 16-element alignment is not required for scores; offset rows by one to check that
    starts += 1
    flat = np.concatenate([np.zeros(1, np.float32)] + rows)
    return flat, starts, np.array([len(r) for r in rows], np.int32)


@pytest.mark.parametrize("k", [1, 64, 2048, 4096])
def test_topk_select_exact(k):
    flat, starts, lens = _score_rows(k)
    announce(f"topk_select k={k} rows={len(lens)}")
    S, Ss = tl.topk_select(torch.from_numpy(flat).to(DEV), torch.from_numpy(starts).to(DEV),
                           torch.from_numpy(lens).to(DEV), k, int(lens.max()), want_scores=True)
    torch.cuda.synchronize()
    S_o, Ss_o = oracle.topk_rows(flat, starts, lens, k)
    np.testing.assert_array_equal(S.cpu().numpy(), S_o)
    np.testing.assert_array_equal(Ss.cpu().numpy(), Ss_o)


# ---------------------------------------------------------------------------
# index_decode
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dt,max_len", [(F32, None), (BF16, None), (FP8, None), (FP8, 4_000_000)])
def test_index_decode(dt, max_len):
    """max_len far above the lengths (allowed: it only has to bound them) sizes
    the launch for long sequences, so each wave stages its own scores instead
    of the workgroup staging its whole range."""
    HI, DI = (4, 32) if dt == F32 else (64, 128)
    lengths = [1, 0, 17, 64, 65, 300, 0, 2048, 2049, 5000]  # empty sequences are skipped
    dist = "dyadic" if dt == F32 else "normal"
    # planted keys carry N(0,1) noise, so the exact (dyadic) case plants none
    inp = synth.indexer_decode(lengths, HI, DI, dt, seed=3, dist=dist, planted=dt != F32)
    announce(f"index_decode dt={dt} max_len={max_len}")
    sc = tl.index_decode(to_dev(inp.q), to_dev(inp.k), to_dev(inp.w), to_dev(inp.cu_seqlens),
                         max_len or max(lengths), q_scale=to_dev(inp.q_scale), k_scale=to_dev(inp.k_scale))
    torch.cuda.synchronize()
    ref, mag = oracle.index_decode(dt, host(inp.q), host(inp.q_scale), host(inp.k), host(inp.k_scale),
                                   host(inp.w), host(inp.cu_seqlens))
    got = sc.cpu().numpy()
    if dt == F32:
        np.testing.assert_array_equal(got, ref)
    else:
        assert parity.check_score_vector(got, ref, mag, lowp=True) <= 1.0


# ---------------------------------------------------------------------------
# index_prefill
# ---------------------------------------------------------------------------
def _prefill_gpu(inp, k, want_scores=True):
    S, Ss = tl.index_prefill(to_dev(inp.q), to_dev(inp.k), to_dev(inp.w), k,
                             q_scale=to_dev(inp.q_scale), k_scale=to_dev(inp.k_scale),
                             want_scores=want_scores)
    torch.cuda.synchronize()
    return S.cpu().numpy(), (Ss.cpu().numpy() if Ss is not None else None)


def _oracle_rows(inp, k, rows):
    return oracle.index_prefill_rows(inp.dt, host(inp.q), host(inp.q_scale), host(inp.k),
                                     host(inp.k_scale), host(inp.w), k, rows, want_scores=True)


@pytest.mark.parametrize("B,n,HI,DI,k", [(1, 512, 4, 32, 64), (2, 1000, 16, 64, 128), (1, 700, 64, 32, 300)])
def test_index_prefill_dyadic_exact(B, n, HI, DI, k):
    """Dyadic inputs: every score is exact in fp32, so rows must match bit for bit."""
    inp = synth.indexer_prefill(B, n, HI, DI, F32, seed=1, dist="dyadic")
    announce(f"index_prefill dyadic B={B} n={n} HI={HI} DI={DI} k={k}")
    S, Ss = _prefill_gpu(inp, k)
    rows = np.arange(B * n)
    S_o, Ss_o, _, _ = _oracle_rows(inp, k, rows)
    np.testing.assert_array_equal(S.reshape(B * n, k), S_o)
    np.testing.assert_array_equal(Ss.reshape(B * n, k), Ss_o)


@pytest.mark.parametrize("dt,n,k", [(BF16, 3000, 256), (FP8, 3000, 256), (BF16, 2500, 2048),
                                    (FP8, 6000, 2048), (BF16, 9000, 4096), (FP8, 7000, 3000)])
def test_index_prefill_lowp(dt, n, k):
    HI, DI = 64, 128
    inp = synth.indexer_prefill(1, n, HI, DI, dt, seed=2, planted=True)
    announce(f"index_prefill dt={dt} n={n} k={k}")
    S, Ss = _prefill_gpu(inp, k)
    S, Ss = S[0], Ss[0]
    for t in range(n):
        msg = parity.check_structure(S[t], t, k)
        assert msg is None, (t, msg)
    rows = sample_rows(n, k, 40, seed=dt, extra=[255, 767, 768, 4351, 4352, 8447, 8448])
    S_o, _, sc, mg = _oracle_rows(inp, k, rows)
    rep = parity.check_selection(S[rows], S_o, rows, k, sc)
    assert rep.ok(), rep.summary()
    worst, wt = parity.check_scores(S[rows], Ss[rows], rows, k, sc, mg, lowp=True)
    assert worst <= 1.0, (worst, wt)


def test_index_prefill_all_ties_fallback():
    """Every score equal: the candidate buffers overflow and rows are recomputed;
    the lowest positions win every tie."""
    B, n, HI, DI, k = 1, 3000, 4, 32, 256
    inp = synth.indexer_prefill(B, n, HI, DI, BF16, seed=5, dist="normal")
    inp.w.zero_()
    announce("index_prefill all-ties fallback")
    S, Ss = _prefill_gpu(inp, k)
    for t in range(n):
        K = min(k, t + 1)
        assert S[0, t, :K].tolist() == list(range(K)), t
        assert (S[0, t, K:] == -1).all()
        assert (Ss[0, t, :K] == 0).all()


def test_index_prefill_sample_miss_fallback():
    """Keys of the strided threshold sample score high but are fewer than k, so
    the sample threshold overshoots and the affected rows are recomputed."""
    n, HI, DI, k = 2000, 4, 32, 256
    q = torch.zeros(1, n, HI, DI)
    q[..., 0] = 1.0
    kk = torch.zeros(1, n, DI)
    kk[0, :, 0] = 1.0
    even_low = torch.arange(n) % 2 == 0
    # 200 high keys at even positions below 400: over-represented in the
    # strided sample (every 2nd or 4th key), so its threshold overshoots
    kk[0, even_low & (torch.arange(n) < 400), 0] = 3.0
    w = torch.ones(1, n, HI)
    inp = synth.IndexerPrefill(F32, q.contiguous(), None, kk.contiguous(), None, w.contiguous())
    announce("index_prefill sample-miss fallback")
    S, Ss = _prefill_gpu(inp, k)
    S_o, Ss_o, _, _ = _oracle_rows(inp, k, np.arange(n))
    np.testing.assert_array_equal(S[0], S_o)
    np.testing.assert_array_equal(Ss[0], Ss_o)


def test_prefill_decode_consistency():
    """Prefill row t equals index_decode + topk_select at length t+1, bit for bit."""
    n, HI, DI, k = 1500, 64, 128, 256
    inp = synth.indexer_prefill(1, n, HI, DI, FP8, seed=7, planted=True)
    announce("prefill/decode consistency")
    S, Ss = _prefill_gpu(inp, k)
    ts = [0, 100, 255, 767, 768, 1499]
    qd = torch.stack([inp.q[0, t] for t in ts])
    qs = torch.stack([inp.q_scale[0, t] for t in ts])
    wd = torch.stack([inp.w[0, t] for t in ts])
    kc = torch.cat([inp.k[0, : t + 1] for t in ts])
    ksc = torch.cat([inp.k_scale[0, : t + 1] for t in ts])
    cu = torch.tensor(np.concatenate([[0], np.cumsum([t + 1 for t in ts])]), dtype=torch.int64)
    sc = tl.index_decode(to_dev(qd), to_dev(kc), to_dev(wd), to_dev(cu), n, q_scale=to_dev(qs),
                         k_scale=to_dev(ksc))
    lens = torch.tensor([t + 1 for t in ts], dtype=torch.int32)
    Sd, Ssd = tl.topk_select(sc, to_dev(cu[:-1]), to_dev(lens), k, n, want_scores=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(Sd.cpu().numpy(), S[0, ts])
    np.testing.assert_array_equal(Ssd.cpu().numpy(), Ss[0, ts])


def test_index_prefill_deterministic():
    inp = synth.indexer_prefill(1, 2000, 64, 128, FP8, seed=8, planted=True)
    announce("index_prefill determinism")
    a = _prefill_gpu(inp, 512)
    b = _prefill_gpu(inp, 512)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_index_prefill_without_scores():
    inp = synth.indexer_prefill(1, 1200, 64, 128, BF16, seed=9)
    announce("index_prefill S only")
    S1, _ = _prefill_gpu(inp, 300, want_scores=False)
    S2, _ = _prefill_gpu(inp, 300, want_scores=True)
    np.testing.assert_array_equal(S1, S2)


# ---------------------------------------------------------------------------
# sparse attention
# ---------------------------------------------------------------------------
def _random_selection(n, k, seed, messy=False):
    rng = np.random.default_rng(seed)
    S = np.full((n, k), -1, np.int32)
    for t in range(n):
        K = min(k, t + 1)
        S[t, :K] = np.sort(rng.choice(t + 1, size=K, replace=False))
        if messy and t % 7 == 3 and K > 2:
            S[t, 1] = -1              # hole
            S[t, 0] = t + 5           # beyond the causal limit: skipped
            S[t, K - 1] = S[t, K - 2]  # duplicate: counted twice
    return S


@pytest.mark.parametrize("dt,H,Dqk,Dv,n,k", [(BF16, 128, 576, 512, 150, 64), (BF16, 16, 576, 512, 300, 256),
                                             (F32, 4, 80, 64, 512, 64), (BF16, 128, 576, 512, 40, 2048)])
def test_sparse_attn_prefill(dt, H, Dqk, Dv, n, k):
    q, kv = synth.attn_prefill(1, n, H, Dqk, dt, seed=11)
    S = _random_selection(n, k, seed=n, messy=True)[None]
    scale = 1.0 / math.sqrt(Dqk)
    announce(f"sparse_attn_prefill dt={dt} H={H} n={n} k={k}")
    out, lse = tl.sparse_attn_prefill(to_dev(q), to_dev(kv), torch.from_numpy(S).to(DEV), scale, Dv,
                                      want_lse=True)
    torch.cuda.synchronize()
    rows = sample_rows(n, k, 24, seed=3)
    ref, ref_lse = oracle.sparse_attn_prefill_rows(dt, host(q), host(kv), S, scale, rows, Dv)
    got = out.float().cpu().numpy()[0][rows]
    tol = parity.ATTN_ATOL_F32 if dt == F32 else parity.ATTN_ATOL_BF16
    err = np.abs(got - ref).max()
    assert err <= tol, err
    np.testing.assert_allclose(lse.cpu().numpy()[0][rows], ref_lse, rtol=1e-4, atol=1e-4)


def test_sparse_attn_prefill_tile_pipeline():
    # many tiles per row (every rotation of the tile buffers), whole tiles
    # without a valid slot in the middle of a row, a ragged last tile (k=300)
    # and a partial second head group (H=100)
    n, H, k = 700, 100, 300
    q, kv = synth.attn_prefill(1, n, H, 576, BF16, seed=14)
    S = _random_selection(n, k, seed=7, messy=True)
    S[::3, 32:96] = -1
    S[1::5, 200:264] = -1
    S = S[None]
    scale = 1.0 / math.sqrt(576)
    announce("sparse_attn_prefill tile pipeline")
    out, lse = tl.sparse_attn_prefill(to_dev(q), to_dev(kv), torch.from_numpy(S).to(DEV), scale, 512,
                                      want_lse=True)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([sample_rows(n, k, 20, seed=5), [0, 1, 31, 32, 33, 95, 96, 299, 300, 699]]))
    ref, ref_lse = oracle.sparse_attn_prefill_rows(BF16, host(q), host(kv), S, scale, rows, 512)
    got = out.float().cpu().numpy()[0][rows]
    err = np.abs(got - ref).max()
    assert err <= parity.ATTN_ATOL_BF16, err
    np.testing.assert_allclose(lse.cpu().numpy()[0][rows], ref_lse, rtol=1e-4, atol=1e-4)


def test_sparse_attn_prefill_empty_rows():
    n, H, k = 20, 16, 64
    q, kv = synth.attn_prefill(1, n, H, 576, BF16, seed=12)
    S = np.full((1, n, k), -1, np.int32)
    S[0, 5, 3] = 2
    announce("sparse_attn_prefill empty rows")
    out, lse = tl.sparse_attn_prefill(to_dev(q), to_dev(kv), torch.from_numpy(S).to(DEV), 0.05, 512,
                                      want_lse=True)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()[0]
    l = lse.cpu().numpy()[0]
    assert (o[np.arange(n) != 5] == 0).all()
    assert np.isneginf(l[np.arange(n) != 5]).all()
    np.testing.assert_array_equal(o[5], np.repeat(kv[0, 2:3, :512].float().numpy(), H, 0))


# ---------------------------------------------------------------------------
# dense_attn_prefill (short prefill, n <= k)
# ---------------------------------------------------------------------------
def _all_history(B, n):
    """What TopK(min(k, t+1)) keeps when t+1 <= k: every position 0..t."""
    S = np.full((B, n, n), -1, np.int32)
    for t in range(n):
        S[:, t, : t + 1] = np.arange(t + 1, dtype=np.int32)
    return S


@pytest.mark.parametrize("dt,B,H,Dqk,Dv,n", [(F32, 2, 4, 80, 64, 300), (BF16, 1, 128, 576, 512, 200),
                                             (BF16, 2, 16, 576, 512, 1000), (BF16, 1, 8, 576, 512, 4096),
                                             (BF16, 1, 100, 576, 512, 1)])
def test_dense_attn_prefill(dt, B, H, Dqk, Dv, n):
    q, kv = synth.attn_prefill(B, n, H, Dqk, dt, seed=15)
    scale = 1.0 / math.sqrt(Dqk)
    announce(f"dense_attn_prefill dt={dt} B={B} H={H} n={n}")
    out, lse = tl.dense_attn_prefill(to_dev(q), to_dev(kv), scale, Dv, want_lse=True)
    torch.cuda.synchronize()
    # rows around the 32-slot tiles and both ends of every batch row
    per = sample_rows(n, 32, 12, seed=n, extra=(31, 33, 63, 64, 65))
    rows = np.unique(np.concatenate([b * n + per for b in range(B)]))
    ref, ref_lse = oracle.sparse_attn_prefill_rows(dt, host(q), host(kv), _all_history(B, n), scale, rows, Dv)
    got = out.float().cpu().numpy().reshape(B * n, H, Dv)[rows]
    tol = parity.ATTN_ATOL_F32 if dt == F32 else parity.ATTN_ATOL_BF16
    err = np.abs(got - ref).max()
    assert err <= tol, err
    np.testing.assert_allclose(lse.cpu().numpy().reshape(B * n, H)[rows], ref_lse, rtol=1e-4, atol=1e-4)


def test_short_prefill_path_equals_selected_path():
    """With k >= n the indexer keeps every position, and the dense path gives
    the sparse path's result over that selection bit for bit."""
    n, H = 333, 32
    ix = synth.indexer_prefill(1, n, 16, 64, BF16, seed=16, device=DEV)
    announce("short prefill: index_prefill k=n, sparse vs dense attention")
    S, _ = tl.index_prefill(ix.q, ix.k, ix.w, n, q_scale=ix.q_scale, k_scale=ix.k_scale)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(S.cpu().numpy(), _all_history(1, n))
    q, kv = synth.attn_prefill(1, n, H, 576, BF16, seed=17)
    qd, kvd = to_dev(q), to_dev(kv)
    o_s, l_s = tl.sparse_attn_prefill(qd, kvd, S, 0.05, 512, want_lse=True)
    o_d, l_d = tl.dense_attn_prefill(qd, kvd, 0.05, 512, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o_d)
    assert torch.equal(l_s, l_d)


@pytest.mark.parametrize("dt,H,Dqk,Dv", [(BF16, 128, 576, 512), (F32, 4, 80, 64)])
def test_sparse_attn_decode(dt, H, Dqk, Dv):
    lengths = [1, 0, 5, 64, 2048, 3000, 5000]  # an empty sequence: zero output, lse -inf
    k = 2048
    q, kv = synth.attn_decode(lengths, H, Dqk, dt, seed=13)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    rng = np.random.default_rng(1)
    S = np.full((len(lengths), k), -1, np.int32)
    for b, L in enumerate(lengths):
        K = min(k, L)
        S[b, :K] = np.sort(rng.choice(L, size=K, replace=False))
    scale = 1.0 / math.sqrt(Dqk)
    announce(f"sparse_attn_decode dt={dt} H={H}")
    out, lse = tl.sparse_attn_decode(to_dev(q), to_dev(kv), torch.from_numpy(cu).to(DEV),
                                     torch.from_numpy(S).to(DEV), scale, Dv, want_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.sparse_attn_decode(dt, host(q), host(kv), cu, S, scale, Dv)
    tol = parity.ATTN_ATOL_F32 if dt == F32 else parity.ATTN_ATOL_BF16
    err = np.abs(out.float().cpu().numpy() - ref).max()
    assert err <= tol, err
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=1e-4, atol=1e-4)
