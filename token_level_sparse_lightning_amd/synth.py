"""Seeded synthetic inputs for the DSA token-selection path.

Both the HIP library and the CPU oracle consume the bytes made here; nothing in
this module computes an indexer score, a selection or an attention output.  It
only draws random numbers, casts them to the storage formats the library takes
(fp32, bf16, OCP fp8 e4m3 with one fp32 scale per token) and places the
"planted" keys that give each probe query a few strongly matching positions.

Recipe (all draws from one ``torch.Generator`` seeded with ``seed``):

* indexer, ``dist="normal"``: q^I, k^I ~ N(0,1)/sqrt(d^I), w^I ~ N(0,1)/sqrt(H^I)
  (so some weights are negative);
* indexer, ``dist="dyadic"``: q^I, k^I uniform integers in [-3, 3], w^I uniform
  over the nine multiples of 0.25 in [-1, 1]; every score is then exactly
  representable in fp32;
* planted keys: for probe queries t = 255, 511, ... (every 256th), 32 earlier
  positions s (distinct, never planted twice, distance t-s uniform in
  [1, min(t, max_dist)]) get k^I[s] = 0.5*u_t + eps with u_t the unit vector of
  the query head with the largest weight and eps ~ N(0,1)/sqrt(d^I);
* fp8: per token row, scale = max(amax/448, 2^-126), code = RNE(x/scale)
  clamped to +-448 (OCP e4m3fn, the format gfx950's matrix cores take);
* attention: q and the shared latent entries c ~ N(0,1), drawn in bf16 (or
  fp32).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

DT_F32, DT_BF16, DT_FP8 = 0, 1, 2
DT_NAMES = {DT_F32: "f32", DT_BF16: "bf16", DT_FP8: "fp8_e4m3"}

FP8_MAX = 448.0


def _generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(int(seed))
    return g


def quantize_fp8_rows(x: torch.Tensor, row_dims: int):
    """Cast float32 ``x`` to OCP e4m3 codes with one scale per leading index.

    The trailing ``row_dims`` dimensions share one scale (one token row).
    Returns ``(codes uint8 like x, scale float32 over the leading dims)``.
    """
    lead = x.shape[: x.dim() - row_dims]
    flat = x.reshape(*lead, -1).float()
    amax = flat.abs().amax(dim=-1)
    scale = torch.clamp(amax / FP8_MAX, min=2.0 ** -126)
    y = (flat / scale.unsqueeze(-1)).clamp(-FP8_MAX, FP8_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).reshape(x.shape)
    return codes.contiguous(), scale.float().contiguous()


def cast_storage(x: torch.Tensor, dt: int, row_dims: int):
    """Return ``(storage tensor, per-row scale or None)`` for dtype code ``dt``."""
    if dt == DT_F32:
        return x.float().contiguous(), None
    if dt == DT_BF16:
        return x.to(torch.bfloat16).contiguous(), None
    if dt == DT_FP8:
        return quantize_fp8_rows(x, row_dims)
    raise ValueError(f"unknown dtype code {dt}")


@dataclass
class IndexerPrefill:
    dt: int
    q: torch.Tensor            # [B,n,HI,DI] storage dtype
    q_scale: Optional[torch.Tensor]  # [B,n] f32 (fp8 only)
    k: torch.Tensor            # [B,n,DI]
    k_scale: Optional[torch.Tensor]  # [B,n]
    w: torch.Tensor            # [B,n,HI] f32
    probes: dict = field(default_factory=dict)  # (b,t) -> planted positions

    @property
    def shape(self):
        B, n, HI, DI = self.q.shape
        return B, n, HI, DI


@dataclass
class IndexerDecode:
    dt: int
    q: torch.Tensor            # [B,HI,DI]
    q_scale: Optional[torch.Tensor]  # [B]
    k: torch.Tensor            # [sumL,DI] packed cache
    k_scale: Optional[torch.Tensor]  # [sumL]
    w: torch.Tensor            # [B,HI] f32
    cu_seqlens: torch.Tensor   # [B+1] int64
    lengths: np.ndarray        # [B]
    planted: dict = field(default_factory=dict)  # b -> planted positions (row-relative)


def _draw_base(shape_q, shape_k, shape_w, DI, HI, dist, g, device):
    if dist == "dyadic":
        q = torch.randint(-3, 4, shape_q, generator=g, device=device).float()
        k = torch.randint(-3, 4, shape_k, generator=g, device=device).float()
        w = torch.randint(-4, 5, shape_w, generator=g, device=device).float() * 0.25
    elif dist == "normal":
        q = torch.randn(shape_q, generator=g, device=device) / math.sqrt(DI)
        k = torch.randn(shape_k, generator=g, device=device) / math.sqrt(DI)
        w = torch.randn(shape_w, generator=g, device=device) / math.sqrt(HI)
    else:
        raise ValueError(dist)
    return q, k, w


def _plant(k_row_sink, q_t_heads, w_t, positions, g, device, DI, alpha=0.5, beta=1.0):
    """Overwrite keys at ``positions`` with the query's strongest head direction plus noise."""
    j = int(torch.argmax(w_t).item())
    u = q_t_heads[j] / torch.clamp(q_t_heads[j].norm(), min=1e-30)
    eps = torch.randn((len(positions), DI), generator=g, device=device) / math.sqrt(DI)
    idx = torch.as_tensor(positions, device=device, dtype=torch.long)
    k_row_sink[idx] = alpha * u.unsqueeze(0) + beta * eps


def indexer_prefill(B, n, HI, DI, dt, seed, dist="normal", planted=False,
                    plant_max_dist=None, n_plant=32, probe_every=256,
                    device="cpu") -> IndexerPrefill:
    g = _generator(seed, device)
    q, k, w = _draw_base((B, n, HI, DI), (B, n, DI), (B, n, HI), DI, HI, dist, g, device)
    probes = {}
    if planted:
        rng = np.random.Generator(np.random.PCG64(seed + 7919))
        for b in range(B):
            used = np.zeros(n, dtype=bool)
            for t in range(probe_every - 1, n, probe_every):
                maxd = t if plant_max_dist is None else min(t, plant_max_dist)
                want = min(n_plant, int((~used[t - maxd:t]).sum()))
                pos = []
                while len(pos) < want:
                    s = t - int(rng.integers(1, maxd + 1))
                    if not used[s]:
                        used[s] = True
                        pos.append(s)
                if pos:
                    _plant(k[b], q[b, t], w[b, t], pos, g, device, DI)
                    probes[(b, t)] = sorted(pos)
    qs, q_scale = cast_storage(q, dt, 2)
    ks, k_scale = cast_storage(k, dt, 1)
    return IndexerPrefill(dt, qs, q_scale, ks, k_scale, w.float().contiguous(), probes)


def decode_lengths(B, lo, hi, seed) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(lo, hi + 1, size=B).astype(np.int64)


def indexer_decode(lengths, HI, DI, dt, seed, dist="normal", planted=True, n_plant=32,
                   device="cpu") -> IndexerDecode:
    lengths = np.asarray(lengths, dtype=np.int64)
    B = len(lengths)
    total = int(lengths.sum())
    g = _generator(seed, device)
    q, k, w = _draw_base((B, HI, DI), (total, DI), (B, HI), DI, HI, dist, g, device)
    cu = np.zeros(B + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    plants = {}
    if planted:
        rng = np.random.Generator(np.random.PCG64(seed + 7919))
        for b in range(B):
            L = int(lengths[b])
            m = min(n_plant, L)
            pos = np.sort(rng.choice(L, size=m, replace=False))
            _plant(k[int(cu[b]):int(cu[b + 1])], q[b], w[b], pos.tolist(), g, device, DI)
            plants[b] = pos.tolist()
    qs, q_scale = cast_storage(q, dt, 2)
    ks, k_scale = cast_storage(k, dt, 1)
    return IndexerDecode(dt, qs, q_scale, ks, k_scale, w.float().contiguous(),
                         torch.as_tensor(cu, device=device), lengths, plants)


def _randn_storage(shape, dt, g, device):
    if dt == DT_BF16:
        return torch.randn(shape, generator=g, device=device, dtype=torch.bfloat16)
    if dt == DT_F32:
        return torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    raise ValueError("attention inputs are bf16 or fp32")


def attn_prefill(B, n, H, Dqk, dt, seed, device="cpu"):
    """q [B,n,H,Dqk] and shared latent entries kv [B,n,Dqk], N(0,1)."""
    g = _generator(seed + 104729, device)
    q = _randn_storage((B, n, H, Dqk), dt, g, device)
    kv = _randn_storage((B, n, Dqk), dt, g, device)
    return q, kv


def attn_decode(lengths, H, Dqk, dt, seed, device="cpu"):
    """q [B,H,Dqk] (one new token per sequence) and the packed cache kv [sumL,Dqk]."""
    lengths = np.asarray(lengths, dtype=np.int64)
    g = _generator(seed + 104729, device)
    q = _randn_storage((len(lengths), H, Dqk), dt, g, device)
    kv = _randn_storage((int(lengths.sum()), Dqk), dt, g, device)
    return q, kv


def storage_to_numpy(x: Optional[torch.Tensor]):
    """Host numpy view of a storage tensor's bytes (bf16 as uint16, fp8 as uint8)."""
    if x is None:
        return None
    x = x.detach().cpu().contiguous()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view(np.uint16)
    return x.numpy()
