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
    rows = sample_rows(n, k, 40, seed=dt, extra=[255, 767, 768, 4351, 4352, 5375, 5376, 8447, 8448])
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


def _fp8_integer_inputs(n, HI, DI, seed):
    """fp8 inputs that are small integers (exact in e4m3) at unit scales, with
    weights in quarters: every product, sum and linear-part split on either
    side is exact in fp32, so selections and scores must match bit for bit."""
    g = torch.Generator().manual_seed(seed)
    q = torch.randint(-12, 13, (1, n, HI, DI), generator=g).float()
    k = torch.randint(-12, 13, (1, n, DI), generator=g).float()
    w = (torch.randint(-4, 5, (1, n, HI), generator=g).float() * 0.25).contiguous()
    q8 = q.to(torch.float8_e4m3fn).view(torch.uint8).contiguous()
    k8 = k.to(torch.float8_e4m3fn).view(torch.uint8).contiguous()
    return q8, torch.ones(1, n), k8, torch.ones(1, n), w


@pytest.mark.parametrize("HI", [8, 24, 40])
def test_index_prefill_fp8_integer_exact(HI):
    """fp8 prefill with one, two and four head blocks (24 and 40 leave masked
    heads in the last block): bit-exact against the oracle, ties included."""
    n, DI, k = 1200, 128, 96
    q8, qs, k8, ks, w = _fp8_integer_inputs(n, HI, DI, 70 + HI)
    announce(f"index_prefill fp8 integer HI={HI}")
    S, Ss = tl.index_prefill(to_dev(q8), to_dev(k8), to_dev(w), k, q_scale=to_dev(qs), k_scale=to_dev(ks),
                             want_scores=True)
    torch.cuda.synchronize()
    rows = np.arange(n)
    S_o, Ss_o, _, _ = oracle.index_prefill_rows(FP8, host(q8), host(qs), host(k8), host(ks), host(w), k, rows)
    np.testing.assert_array_equal(S[0].cpu().numpy(), S_o)
    np.testing.assert_array_equal(Ss[0].cpu().numpy(), Ss_o)


def test_prefill_decode_consistency_two_head_blocks():
    """As below with H^I = 24 (two head blocks, eight masked heads): the
    prefill row t equals the decode scan + top-k at length t+1 bit for bit,
    for rows in both linear-part slots (even and odd t)."""
    n, HI, DI, k = 1300, 24, 128, 200
    inp = synth.indexer_prefill(1, n, HI, DI, FP8, seed=17, planted=True)
    announce("prefill/decode consistency HI=24")
    S, Ss = _prefill_gpu(inp, k)
    ts = [0, 1, 199, 200, 777, 1298, 1299]
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


def test_attention_and_decode_step_deterministic():
    """Bitwise reproducibility, promised for every call but the training
    step's dk: the prefill attention and a whole decode step (scan, row
    top-k, decode attention) run twice give identical bytes."""
    n, k, H = 600, 256, 128
    q, kv = synth.attn_prefill(1, n, H, 576, BF16, seed=13)
    S = torch.from_numpy(_random_selection(n, k, seed=5)[None]).to(DEV)
    announce("sparse_attn_prefill determinism")
    runs = [tl.sparse_attn_prefill(to_dev(q), to_dev(kv), S, 1 / 24.0, 512, want_lse=True) for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(runs[0][0], runs[1][0]) and torch.equal(runs[0][1], runs[1][1])

    lengths = np.array([3000, 5000, 100, 0, 2049], dtype=np.int64)
    di = synth.indexer_decode(lengths, 64, 128, FP8, seed=17, device=DEV)
    qa, kva = synth.attn_decode(lengths, H, 576, BF16, seed=17, device=DEV)
    row_len = torch.as_tensor(lengths, dtype=torch.int32, device=DEV)
    announce("decode step determinism")
    outs = []
    for _ in range(2):
        sc = tl.index_decode(di.q, di.k, di.w, di.cu_seqlens, int(lengths.max()), q_scale=di.q_scale,
                             k_scale=di.k_scale)
        Sd, Ssd = tl.topk_select(sc, di.cu_seqlens[:-1].contiguous(), row_len, 512, int(lengths.max()),
                                 want_scores=True)
        o, lse = tl.sparse_attn_decode(qa, kva, di.cu_seqlens, Sd, 1 / 24.0, 512, want_lse=True)
        outs.append((sc, Sd, Ssd, o, lse))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("dt", [BF16, FP8])
def test_rank_invariance_on_the_gpu(dt):
    """DSA page, section 3.1: a positive rescaling of the scores leaves the
    selection unchanged.  Doubling w (and, for fp8, the key scales) doubles
    every product and sum exactly, so the GPU's S must be bit-identical and
    S_score exactly twice the original, in prefill and decode."""
    inp = synth.indexer_prefill(1, 3000, 64, 128, dt, seed=23, planted=True, device=DEV)
    k = 700
    announce(f"rank invariance dt={dt}")
    S1, Ss1 = tl.index_prefill(inp.q, inp.k, inp.w, k, q_scale=inp.q_scale, k_scale=inp.k_scale, want_scores=True)
    w2 = inp.w * 2
    ks2 = inp.k_scale * 2 if inp.k_scale is not None else None
    S2, Ss2 = tl.index_prefill(inp.q, inp.k, w2, k, q_scale=inp.q_scale, k_scale=ks2, want_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(S1, S2)
    assert torch.equal(Ss1 * (4 if dt == FP8 else 2), Ss2)
    lengths = np.array([2500, 40, 1800], dtype=np.int64)
    di = synth.indexer_decode(lengths, 64, 128, dt, seed=29, device=DEV)
    sc1 = tl.index_decode(di.q, di.k, di.w, di.cu_seqlens, 2500, q_scale=di.q_scale, k_scale=di.k_scale)
    dks2 = di.k_scale * 2 if di.k_scale is not None else None
    sc2 = tl.index_decode(di.q, di.k, di.w * 2, di.cu_seqlens, 2500, q_scale=di.q_scale, k_scale=dks2)
    torch.cuda.synchronize()
    assert torch.equal(sc1 * (4 if dt == FP8 else 2), sc2)


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


def test_sparse_attn_prefill_batch_of_two():
    """Two batch rows: each row's slots index its own sequence's entries
    (entry b*n + s), with holes, out-of-range and duplicate slots."""
    B, n, H, k = 2, 260, 128, 96
    q, kv = synth.attn_prefill(B, n, H, 576, BF16, seed=19)
    S = np.stack([_random_selection(n, k, seed=20 + b, messy=True) for b in range(B)])
    scale = 1.0 / math.sqrt(576)
    announce("sparse_attn_prefill B=2")
    out, lse = tl.sparse_attn_prefill(to_dev(q), to_dev(kv), torch.from_numpy(S).to(DEV), scale, 512,
                                      want_lse=True)
    torch.cuda.synchronize()
    per = sample_rows(n, k, 10, seed=21, extra=(31, 32, 95, 96, 97))
    rows = np.concatenate([b * n + per for b in range(B)])
    ref, ref_lse = oracle.sparse_attn_prefill_rows(BF16, host(q), host(kv), S, scale, rows, 512)
    got = out.float().cpu().numpy().reshape(B * n, H, 512)[rows]
    err = np.abs(got - ref).max()
    assert err <= parity.ATTN_ATOL_BF16, err
    np.testing.assert_allclose(lse.cpu().numpy().reshape(B * n, H)[rows], ref_lse, rtol=1e-4, atol=1e-4)


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


@pytest.mark.parametrize("dt,H,Dqk,Dv", [(BF16, 128, 576, 512), (BF16, 100, 576, 512), (F32, 4, 80, 64)])
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


def test_sparse_attn_decode_messy_slots():
    """Decode selections with holes (-1), positions at or past the sequence's
    length (skipped), duplicates (counted twice) and a whole 32-slot tile
    without a valid slot."""
    lengths = [700, 3000, 40, 2500]
    H, k = 128, 1024
    q, kv = synth.attn_decode(lengths, H, 576, BF16, seed=22)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    rng = np.random.default_rng(23)
    S = np.full((len(lengths), k), -1, np.int32)
    for b, L in enumerate(lengths):
        K = min(k, L)
        S[b, :K] = np.sort(rng.choice(L, size=K, replace=False))
        S[b, 5] = -1                 # hole
        S[b, 7] = L + 3              # past the sequence: skipped
        S[b, 9] = S[b, 8]            # duplicate
        S[b, 64:96] = -1             # a tile with no valid slot
    scale = 1.0 / math.sqrt(576)
    announce("sparse_attn_decode messy slots")
    out, lse = tl.sparse_attn_decode(to_dev(q), to_dev(kv), torch.from_numpy(cu).to(DEV),
                                     torch.from_numpy(S).to(DEV), scale, 512, want_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.sparse_attn_decode(BF16, host(q), host(kv), cu, S, scale, 512)
    err = np.abs(out.float().cpu().numpy() - ref).max()
    assert err <= parity.ATTN_ATOL_BF16, err
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=1e-4, atol=1e-4)


def test_sparse_attn_decode_entries_beyond_4gib():
    """A sequence whose latent entries span more than 4 GiB (3.8M entries of
    1152 bytes, its last 64 selected): its gathers take full 64-bit addresses
    instead of 32-bit offsets from the sequence's first entry, which the short
    sequence before it uses.  Checked against eq.(3) over the selected entries,
    gathered in slot order."""
    lengths = [5000, 3_800_000]
    H, Dqk, Dv, k = 128, 576, 512, 2048
    q, kv = synth.attn_decode(lengths, H, Dqk, BF16, seed=18, device=DEV)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    rng = np.random.default_rng(2)
    S = np.zeros((2, k), np.int32)
    S[0] = np.sort(rng.choice(lengths[0], size=k, replace=False))
    low = np.unique(rng.integers(0, lengths[1] - 64, size=4 * k))
    low = rng.permutation(low)[: k - 64]
    S[1] = np.sort(np.concatenate([low, np.arange(lengths[1] - 64, lengths[1])]))
    scale = 1.0 / math.sqrt(Dqk)
    announce("sparse_attn_decode, a sequence beyond 4 GiB of entries")
    out, lse = tl.sparse_attn_decode(q, kv, torch.from_numpy(cu).to(DEV), torch.from_numpy(S).to(DEV), scale, Dv,
                                     want_lse=True)
    torch.cuda.synchronize()
    sel = torch.from_numpy(np.concatenate([cu[b] + S[b] for b in range(2)])).to(DEV)
    kv_sel = kv.index_select(0, sel)
    del kv
    torch.cuda.empty_cache()
    S_sel = np.arange(2 * k, dtype=np.int32).reshape(2, k)
    ref, ref_lse = oracle.sparse_attn_rows(BF16, host(q), host(kv_sel), S_sel, np.full(2, 2 * k - 1), scale, Dv)
    err = np.abs(out.float().cpu().numpy() - ref).max()
    assert err <= parity.ATTN_ATOL_BF16, err
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=1e-4, atol=1e-4)


# ---------------------------------------------------------------------------
# the DSA page's worked example (section 1.1, eq.(4)-(6)) on the GPU
# ---------------------------------------------------------------------------
def _golden():
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("dt,DI", [(F32, 32), (BF16, 32), (FP8, 128)])
def test_worked_example_on_gpu(dt, DI):
    """The 3-token example, its two dims zero-padded to a built d^I: the padded
    dims add exact zeros, so the scores are exactly 1.5, 1.5, 1.0 and the
    selection at k=2 is {0, 1} (1-based {1, 2}); at k=1 the 1.5/1.5 tie goes
    to the lower position.  Prefill (query at t=2) and decode (one sequence of
    length 3, then topk_select) must both give it."""
    ex = _golden()["indexer"]
    HI = ex["H_I"]
    q = torch.zeros(1, 3, HI, DI)
    q[0, 2, :, :2] = torch.tensor(ex["q"], dtype=torch.float32)
    kk = torch.zeros(1, 3, DI)
    kk[0, :, :2] = torch.tensor(ex["keys"], dtype=torch.float32)
    w = torch.zeros(1, 3, HI)
    w[0, 2] = torch.tensor(ex["w"], dtype=torch.float32)
    if dt == FP8:
        # unit scales keep the small integers exact in e4m3
        qs = q.to(torch.float8_e4m3fn).view(torch.uint8)
        ks = kk.to(torch.float8_e4m3fn).view(torch.uint8)
        q_scale, k_scale = torch.ones(1, 3), torch.ones(1, 3)
    else:
        qs = q.to(torch.bfloat16) if dt == BF16 else q
        ks = kk.to(torch.bfloat16) if dt == BF16 else kk
        q_scale = k_scale = None
    announce(f"worked example dt={dt} DI={DI}")
    for k, want in ((ex["k"], [p - 1 for p in ex["selected_1based"]]), (1, [0]), (4, [0, 1, 2, -1])):
        S, Ss = tl.index_prefill(to_dev(qs), to_dev(ks), to_dev(w), k, q_scale=to_dev(q_scale),
                                 k_scale=to_dev(k_scale), want_scores=True)
        torch.cuda.synchronize()
        assert S[0, 2].tolist() == want, (k, S[0, 2].tolist())
        exp_sc = [ex["scores"][p] if p >= 0 else -math.inf for p in want]
        assert Ss[0, 2].tolist() == exp_sc
    # decode: the same query against the 3-key cache
    cu = torch.tensor([0, 3], dtype=torch.int64)
    sc = tl.index_decode(to_dev(qs[0, 2:3]), to_dev(ks[0]), to_dev(w[0, 2:3]), to_dev(cu), 3,
                         q_scale=to_dev(None if q_scale is None else q_scale[0, 2:3]),
                         k_scale=to_dev(None if k_scale is None else k_scale[0]))
    Sd, _ = tl.topk_select(sc, to_dev(cu[:1]), to_dev(torch.tensor([3], dtype=torch.int32)), ex["k"], 3)
    torch.cuda.synchronize()
    assert sc.cpu().tolist() == ex["scores"]
    assert Sd[0].tolist() == [p - 1 for p in ex["selected_1based"]]


def test_worked_example_attention_on_gpu():
    """eq.(5)-(6) of the example: logits 0.2 and 1.2 over values (2,0) and
    (0,3) give weights (0.269, 0.731) and output (0.538, 2.193).  Encoded in
    the fp32 build (Dqk = 80 = 64 value dims + 16 position dims): the values in
    dims 0-1, the logit in position dim 64, q = e_64, scale 1."""
    ex = _golden()["attention"]
    kv = torch.zeros(1, 3, 80)
    for s, (v, z) in enumerate(zip(ex["values"], ex["logits"])):
        kv[0, s, :2] = torch.tensor(v, dtype=torch.float32)
        kv[0, s, 64] = z
    q = torch.zeros(1, 3, 1, 80)
    q[0, 2, 0, 64] = 1.0
    S = torch.tensor([[[0, -1], [0, 1], [0, 1]]], dtype=torch.int32)
    announce("worked example attention")
    out, lse = tl.sparse_attn_prefill(to_dev(q), to_dev(kv), to_dev(S), 1.0, 64, want_lse=True)
    torch.cuda.synchronize()
    o = out[0, 2, 0].cpu().numpy()
    d = ex["printed_decimals"]
    assert [round(float(x), d) for x in o[:2]] == ex["output"]
    assert (o[2:] == 0).all()
    w = np.exp(np.array(ex["logits"]) - float(lse[0, 2, 0]))
    assert [round(float(x), d) for x in w] == ex["weights"]


# ---------------------------------------------------------------------------
# index_decode batch sizes: a multiple of the scan's 256-thread prefix loop,
# one past it, and the path for more than 4096 sequences
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("B,max_len", [(256, None), (257, None), (4096, None), (4096, 4_000_000), (4100, None)])
def test_index_decode_batch_sizes(B, max_len):
    """B = 4096 is the largest batch of the balanced scan: its LDS then holds
    the 4097-entry subtile prefix and sequence starts (~49 KB) next to the
    score stage; with a large max_len every wave stages its own scores in
    what is left (the most LDS the scan takes)."""
    rng = np.random.default_rng(B)
    lengths = rng.integers(1, 300, size=B)
    lengths[B // 3] = 0          # an empty sequence
    lengths[-1] = 513            # the last sequence is the longest
    inp = synth.indexer_decode(lengths, 64, 128, FP8, seed=B, planted=False)
    announce(f"index_decode B={B} sumL={int(lengths.sum())} max_len={max_len}")
    sc = tl.index_decode(to_dev(inp.q), to_dev(inp.k), to_dev(inp.w), to_dev(inp.cu_seqlens),
                         max_len or int(lengths.max()), q_scale=to_dev(inp.q_scale), k_scale=to_dev(inp.k_scale))
    torch.cuda.synchronize()
    ref, mag = oracle.index_decode(FP8, host(inp.q), host(inp.q_scale), host(inp.k), host(inp.k_scale),
                                   host(inp.w), host(inp.cu_seqlens))
    got = sc.cpu().numpy()
    assert np.isfinite(got).all()
    assert parity.check_score_vector(got, ref, mag, lowp=True) <= 1.0


def test_max_len_below_the_lengths_is_still_exact():
    """max_len only sizes the launch: a caller that passes a smaller value gets
    every key scored and every row selected in full."""
    lengths = np.array([9000, 30000, 5000, 17000])
    inp = synth.indexer_decode(lengths, 64, 128, BF16, seed=21, planted=True)
    announce("index_decode / topk_select with max_len below the lengths")
    cu = to_dev(inp.cu_seqlens)
    sc = tl.index_decode(to_dev(inp.q), to_dev(inp.k), to_dev(inp.w), cu, 1000)
    sc_ok = tl.index_decode(to_dev(inp.q), to_dev(inp.k), to_dev(inp.w), cu, int(lengths.max()))
    rl = to_dev(torch.tensor(lengths, dtype=torch.int32))
    S_small, Ss_small = tl.topk_select(sc_ok, cu[:-1].contiguous(), rl, 2048, 100, want_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(sc, sc_ok)
    S_o, Ss_o = oracle.topk_rows(sc_ok.cpu().numpy(), host(inp.cu_seqlens)[:-1], lengths, 2048)
    np.testing.assert_array_equal(S_small.cpu().numpy(), S_o)
    np.testing.assert_array_equal(Ss_small.cpu().numpy(), Ss_o)


# ---------------------------------------------------------------------------
# dsa_prefill: the path chosen by length
# ---------------------------------------------------------------------------
def test_dsa_prefill_dense_path_when_n_le_k():
    """n <= k: every row keeps all history; dsa_prefill skips the indexer and
    must equal both dense_attn_prefill and index_prefill + sparse_attn_prefill
    bit for bit, with S = 0..t then -1."""
    B, n, k, H = 2, 300, 512, 32
    ix = synth.indexer_prefill(B, n, 16, 64, BF16, seed=51, device=DEV)
    q, kv = synth.attn_prefill(B, n, H, 576, BF16, seed=52)
    qd, kvd = to_dev(q), to_dev(kv)
    announce("dsa_prefill dense path")
    out, lse, S = tl.dsa_prefill(ix.q, ix.k, ix.w, qd, kvd, k, 0.05, 512, want_S=True, want_lse=True)
    o_d, l_d = tl.dense_attn_prefill(qd, kvd, 0.05, 512, want_lse=True)
    S2, _ = tl.index_prefill(ix.q, ix.k, ix.w, k)
    o_s, l_s = tl.sparse_attn_prefill(qd, kvd, S2, 0.05, 512, want_lse=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(S.cpu().numpy(), np.concatenate(
        [_all_history(B, n), np.full((B, n, k - n), -1, np.int32)], axis=2))
    assert torch.equal(S, S2)
    assert torch.equal(out, o_d) and torch.equal(lse, l_d)
    assert torch.equal(out, o_s) and torch.equal(lse, l_s)


@pytest.mark.parametrize("keep_S", [True, False])
def test_dsa_prefill_sparse_path_when_n_gt_k(keep_S):
    """n > k: indexer, top-k and gather, equal to the two calls bit for bit;
    without an S argument the selection lives in the workspace."""
    n, k, H = 1500, 256, 128
    ix = synth.indexer_prefill(1, n, 64, 128, FP8, seed=53, planted=True, device=DEV)
    q, kv = synth.attn_prefill(1, n, H, 576, BF16, seed=54, device=DEV)
    announce(f"dsa_prefill sparse path keep_S={keep_S}")
    out, lse, S = tl.dsa_prefill(ix.q, ix.k, ix.w, q, kv, k, 1 / 24.0, 512, q_scale=ix.q_scale, k_scale=ix.k_scale,
                                 want_S=keep_S, want_lse=True)
    S2, _ = tl.index_prefill(ix.q, ix.k, ix.w, k, q_scale=ix.q_scale, k_scale=ix.k_scale)
    o2, l2 = tl.sparse_attn_prefill(q, kv, S2, 1 / 24.0, 512, want_lse=True)
    torch.cuda.synchronize()
    if keep_S:
        assert torch.equal(S, S2)
    assert torch.equal(out, o2) and torch.equal(lse, l2)
