"""GPU parity of indexer_loss_grad (the sparse-stage indexer loss of the DSA
page, section 1.2 eq.(8), and its gradient) against the oracle.

Tolerances follow from the arithmetic: scores accumulate in fp32 (relative
error ~1e-6 of their magnitude sum), the backward products take their
coefficients as two bf16 terms (2^-18 relative) and accumulate up to k terms
in fp32 (at most k * 2^-24 of the magnitude sum).  Each result is therefore
compared with the oracle's as |gpu - oracle| <= tol * mag + floor, mag being
the oracle's magnitude sum of the terms (with |g_i| replaced by R_i + P_i so
that an error in g is covered too): tol = 1e-4 for the loss, 2e-4 for dq and
dw, 5e-4 for dk (which also sums one contribution per selecting query).  A
term whose dot product q_j . k_s lies within fp32 accumulation rounding of
zero may fall on either side of ReLU's kink in the kernel, so dq and dk also
allow the oracle's kink band (those terms at full weight), as the selection
rule allows swaps within its margin.
"""
import numpy as np
import pytest
import torch

import oracle
import token_level_sparse_lightning_amd as tl
from token_level_sparse_lightning_amd import synth
from tests.gpu_util import DEV, announce, host, to_dev

pytestmark = pytest.mark.gpu

BF16 = synth.DT_BF16
TOL = {"loss": (1e-4, 1e-6), "dq": (2e-4, 1e-9), "dk": (5e-4, 1e-9), "dw": (2e-4, 1e-9)}


def _teacher(B, n, k, seed):
    """Synthetic teacher masses per slot (positive; the kernel renormalises)."""
    g = torch.Generator().manual_seed(seed)
    return (torch.rand((B, n, k), generator=g) ** 3 + 1e-3).float().contiguous()


def _compare(name, got, ora):
    worst = {}
    kink = {"dq": ora[8], "dk": ora[9]}
    for key, g_, (val, mag) in zip(("loss", "dq", "dk", "dw"), got, zip(ora[:4], ora[4:8])):
        tol, floor = TOL[key]
        err = np.abs(g_.cpu().numpy().astype(np.float64) - val)
        bound = tol * mag + kink.get(key, 0.0) + floor
        ratio = float((err / bound).max())
        worst[key] = ratio
        if ratio > 1.0:
            at = np.unravel_index(int(np.argmax(err / bound)), err.shape)
            print(f"[parity] {name} {key}: worst at {at}: gpu {float(g_.cpu().numpy()[at]):.9g} oracle {val[at]:.9g} "
                  f"mag {mag[at]:.3g} kink {float(kink[key][at]) if key in kink else 0.0:.3g}", flush=True)
        assert ratio <= 1.0, (name, key, ratio)
    print(f"[parity] {name}: worst error / tolerance " + ", ".join(f"{k_}={v:.3g}" for k_, v in worst.items()),
          flush=True)


def _run(inp, S, p):
    return tl.indexer_loss_grad(to_dev(inp.q), to_dev(inp.k), to_dev(inp.w), to_dev(S), to_dev(p))


def _oracle(inp, S, p):
    return oracle.indexer_kl(BF16, host(inp.q), None, host(inp.k), None, host(inp.w), host(S), host(p),
                             want_mags=True)


@pytest.mark.parametrize("n,k", [(700, 256), (2048, 1024)])
def test_indexer_loss_grad_on_the_prefill_selection(n, k):
    """S from index_prefill on the same inputs (HI=64, dI=128, bf16), planted keys."""
    inp = synth.indexer_prefill(1, n, 64, 128, BF16, seed=n, planted=True)
    announce(f"indexer_loss_grad on index_prefill's selection n={n} k={k}")
    S, _ = tl.index_prefill(to_dev(inp.q), to_dev(inp.k), to_dev(inp.w), k)
    S = S.cpu()
    p = _teacher(1, n, k, seed=n)
    got = _run(inp, S, p)
    torch.cuda.synchronize()
    _compare(f"train n={n} k={k}", got, _oracle(inp, S, p))


def test_indexer_loss_grad_ragged_selection():
    """Two batch rows, HI=16 (padded head blocks), k=100 (a partial last tile),
    slots that are -1, beyond t or repeated, a row whose teacher has no mass
    and a row with no valid slot."""
    B, n, HI, k = 2, 300, 16, 100
    inp = synth.indexer_prefill(B, n, HI, 128, BF16, seed=31)
    rng = np.random.default_rng(31)
    S = np.full((B, n, k), -1, np.int32)
    for b in range(B):
        for t in range(n):
            K = min(k, t + 1)
            S[b, t, :K] = np.sort(rng.choice(t + 1, K, replace=False))
            if t % 7 == 3 and K > 3:
                S[b, t, 0] = -1
                S[b, t, 1] = t + 1 + int(rng.integers(0, 50))   # beyond the causal limit
                S[b, t, 2] = S[b, t, 3]                          # repeated slot
    S[1, 50] = -1                                                # no valid slot
    p = _teacher(B, n, k, seed=32)
    p[0, 80] = 0.0                                               # no teacher mass
    S = torch.from_numpy(S)
    announce("indexer_loss_grad ragged selection")
    got = _run(inp, S, p)
    torch.cuda.synchronize()
    assert float(got[0][1, 50]) == 0.0 and float(got[0][0, 80]) == 0.0
    assert not got[1][1, 50].any() and not got[1][0, 80].any()
    _compare("train ragged", got, _oracle(inp, S, p))


def test_indexer_loss_grad_deterministic_parts():
    """loss, dq and dw are computed in a fixed order (bitwise equal on a
    second call); dk agrees within its tolerance."""
    n, k = 600, 128
    inp = synth.indexer_prefill(1, n, 64, 128, BF16, seed=41)
    S, _ = tl.index_prefill(to_dev(inp.q), to_dev(inp.k), to_dev(inp.w), k)
    p = to_dev(_teacher(1, n, k, seed=41))
    announce("indexer_loss_grad determinism")
    a = tl.indexer_loss_grad(to_dev(inp.q), to_dev(inp.k), to_dev(inp.w), S, p)
    b = tl.indexer_loss_grad(to_dev(inp.q), to_dev(inp.k), to_dev(inp.w), S, p)
    torch.cuda.synchronize()
    for x, y in zip((a[0], a[1], a[3]), (b[0], b[1], b[3])):
        assert torch.equal(x, y)
    # dk: atomics sum the contributions in a varying order (rounding only)
    scale = float(a[2].abs().max())
    assert float((a[2] - b[2]).abs().max()) <= 1e-5 * scale
