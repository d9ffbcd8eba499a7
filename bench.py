"""Benchmark of the DSA token-selection path on one MI355X.

Prints ONE JSON line.  The headline is the prefill Lightning Indexer + causal
top-k (index_prefill) on the largest single-GPU configuration: B=1, n=131072,
H^I=64, d^I=128, k=2048, fp8 e4m3 with per-token scales, planted keys at
distances up to 100,000.  Its metric is causal query-key pairs per second (a
pair is (t, s) with s <= t; B*n*(n+1)/2 per call).  The same line carries the
other rows of the path, each on its own workload (``extra``):

  attn_prefill_131072  sparse_attn_prefill over the headline's selection,
                       n=131072, H=128, Dqk=576, Dv=512, bf16
  prefill_bf16_8192    index_prefill, n=8192, bf16
  prefill_fp8_32768    index_prefill, n=32768, fp8
  attn_prefill_32768   sparse_attn_prefill over that selection
  attn_dense_2048      dense_attn_prefill (short prefill: n <= k, every query
                       over all of its history), n=2048, H=128
  dispatch_2048        dsa_prefill at n = k = 2048 (dense path: every row keeps
                       all history) against index_prefill + sparse_attn_prefill
  rerank_32768         index_prefill_rerank (fp8 recall k'=4096, bf16 re-rank to
                       k=2048) at n=32768 against fp8 and bf16 index_prefill
  decode               one decode step of 64 ragged sequences
                       (L ~ U[16384,131072]): index_decode + topk_select +
                       sparse_attn_decode, tokens/s
  train_8192           indexer_loss_grad (the eq.(8) training step: loss and
                       gradient) over index_prefill's selection, n=8192, bf16
  tiny_f32_512         index_prefill + sparse_attn_prefill on B=1, n=512,
                       H^I=4, d^I=32, k=64, fp32 (report only: launch-bound)

Timing: W untimed warm-up calls, then exactly K calls between two device
synchronisations (wall clock; `value` and ms_per_step use it), with HIP
events on the launch stream around every timed call (median and minimum
reported) and, through the library's kernel timer, HIP events on the same
stream around every launch of the workload's main kernel: the roofline of
the headline uses prefill_score_kernel's average launch time.  Inputs are
resident in HBM before the timed region; workspaces are allocated once
outside it.  A calibration leg measures a 1 GiB streaming copy and dense
bf16 / fp8 matrix-core loops on the same device.

The CPU baseline times the oracle (test infrastructure, double precision) on
a bounded sample of query rows of the headline workload.
"""
from __future__ import annotations

import argparse
import gc
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import token_level_sparse_lightning_amd as tl  # noqa: E402
from token_level_sparse_lightning_amd import synth  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
DEV = "cuda:0"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Timing:
    """Wall and event times of K timed calls (ms per call)."""

    def __init__(self, wall, ev, kern):
        self.wall = wall
        self.ev_med = float(np.median(ev))
        self.ev_min = float(np.min(ev))
        self.kernel_launches, tot, self.kernel_min, self.kernel_max = kern if kern else (0, 0.0, 0.0, 0.0)
        self.kernel_avg = tot / self.kernel_launches if self.kernel_launches else None

    def as_dict(self):
        d = dict(ms_per_call=self.wall, event_ms_median=self.ev_med, event_ms_min=self.ev_min)
        if self.kernel_launches:
            d.update(kernel_ms_avg=self.kernel_avg, kernel_ms_min=self.kernel_min, kernel_launches=self.kernel_launches)
        return d


def time_calls(fn, steps, warmup, kernel=None):
    """W untimed calls, then K calls between two synchronisations.  HIP events
    on the launch stream bracket every call; when ``kernel`` is named, the
    library also brackets each launch of that kernel with its own events."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    if kernel:
        tl.timer_arm(kernel, max_launches=8 * steps)
    # no garbage collection inside the timed region (a collection pass over
    # the input generator's bookkeeping can take tens of milliseconds)
    gc.collect()
    gc.disable()
    try:
        t0 = time.perf_counter()
        for a, b in evs:
            a.record(st)
            fn()
            b.record(st)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / steps
    finally:
        gc.enable()
    kern = tl.timer_collect() if kernel else None
    return Timing(wall, [a.elapsed_time(b) for a, b in evs], kern)


def causal_pairs(B, n):
    return B * n * (n + 1) // 2


# ---------------------------------------------------------------------------
def bench_prefill(n, dt, seed, steps, warmup, plant_max_dist=None):
    HI, DI, k = 64, 128, 2048
    torch.cuda.reset_peak_memory_stats()
    log(f"prefill n={n} dt={synth.DT_NAMES[dt]}: generating inputs")
    inp = synth.indexer_prefill(1, n, HI, DI, dt, seed, planted=True, plant_max_dist=plant_max_dist,
                                device=DEV)
    ws = torch.empty(tl.index_prefill_workspace_bytes(inp.q, inp.k, inp.w, k, inp.q_scale, inp.k_scale),
                     dtype=torch.uint8, device=DEV)
    S = torch.empty((1, n, k), dtype=torch.int32, device=DEV)

    def call():
        tl.index_prefill(inp.q, inp.k, inp.w, k, q_scale=inp.q_scale, k_scale=inp.k_scale, S=S, workspace=ws)

    tm = time_calls(call, steps, warmup, kernel="prefill_score_kernel")
    pairs = causal_pairs(1, n)
    flops = 2.0 * HI * DI * pairs
    peak = PEAK_FP8_TFLOPS if dt == synth.DT_FP8 else PEAK_BF16_TFLOPS
    call_tf = flops / (tm.ev_med * 1e-3) / 1e12
    kern_tf = flops / (tm.kernel_avg * 1e-3) / 1e12
    log(f"prefill n={n}: {tm.ev_med:.3f} ms/call (events, median; min {tm.ev_min:.3f}), {tm.wall:.3f} ms (wall), "
        f"{call_tf:.1f} TFLOP/s per call; prefill_score_kernel {tm.kernel_avg:.3f} ms avg over "
        f"{tm.kernel_launches} launches = {kern_tf:.1f} TFLOP/s")
    probes = inp.probes
    recall = None
    if probes:
        Sh = S[0].cpu().numpy()
        hit = tot = 0
        for (b, t), pos in probes.items():
            sel = set(Sh[t][Sh[t] >= 0].tolist())
            hit += sum(p in sel for p in pos)
            tot += len(pos)
        recall = hit / max(tot, 1)
    # algorithmic bytes of one call: Q^I, K^I, W^I and scales read once, S written once
    eb = 1 if dt == synth.DT_FP8 else (2 if dt == synth.DT_BF16 else 4)
    scale_b = 8 * n if dt == synth.DT_FP8 else 0
    nbytes = n * HI * DI * eb + n * DI * eb + n * HI * 4 + scale_b + n * k * 4
    res = dict(workload=f"prefill indexer + top-k: B=1, n={n}, H^I={HI}, d^I={DI}, k={k}, "
                        f"{synth.DT_NAMES[dt]}, planted keys",
               pairs_per_s=pairs / (tm.wall * 1e-3), pairs=pairs, flops_per_call=flops,
               call_tflops=call_tf, kernel="prefill_score_kernel", kernel_tflops=kern_tf, peak_tflops=peak,
               frac=kern_tf / peak, call_frac=call_tf / peak, algorithmic_bytes_per_call=nbytes,
               planted_recall=recall, peak_device_bytes=torch.cuda.max_memory_allocated(), **tm.as_dict())
    return res, inp, S


def bench_attn_prefill(S, n, seed, steps, warmup):
    H, Dqk, Dv = 128, 576, 512
    log(f"attn prefill n={n}: generating inputs")
    q, kv = synth.attn_prefill(1, n, H, Dqk, synth.DT_BF16, seed, device=DEV)
    out = torch.empty((1, n, H, Dv), dtype=torch.bfloat16, device=DEV)
    scale = 1.0 / math.sqrt(Dqk)

    def call():
        tl.sparse_attn_prefill(q, kv, S, scale, Dv, out=out)

    tm = time_calls(call, steps, warmup, kernel="sparse_attn_kernel")
    valid = int((S >= 0).sum().item())
    flops = 2.0 * H * (Dqk + Dv) * valid
    ach = flops / (tm.kernel_avg * 1e-3) / 1e12
    log(f"attn prefill: {tm.ev_med:.3f} ms/call (events, median), sparse_attn_kernel {tm.kernel_avg:.3f} ms, "
        f"{ach:.1f} TFLOP/s")
    del q, kv, out
    return dict(workload=f"sparse attention prefill: n={n}, H={H}, Dqk={Dqk}, Dv={Dv}, k=2048, bf16",
                valid_slots=valid, flops_per_call=flops, kernel="sparse_attn_kernel", kernel_tflops=ach,
                peak_tflops=PEAK_BF16_TFLOPS, frac=ach / PEAK_BF16_TFLOPS, **tm.as_dict())


def bench_attn_dense(n, seed, steps, warmup):
    H, Dqk, Dv = 128, 576, 512
    log(f"dense attn prefill n={n}: generating inputs")
    q, kv = synth.attn_prefill(1, n, H, Dqk, synth.DT_BF16, seed, device=DEV)
    out = torch.empty((1, n, H, Dv), dtype=torch.bfloat16, device=DEV)
    scale = 1.0 / math.sqrt(Dqk)

    def call():
        tl.dense_attn_prefill(q, kv, scale, Dv, out=out)

    tm = time_calls(call, steps, warmup, kernel="sparse_attn_kernel")
    pairs = n * (n + 1) // 2
    flops = 2.0 * H * (Dqk + Dv) * pairs
    ach = flops / (tm.kernel_avg * 1e-3) / 1e12
    log(f"dense attn prefill: {tm.ev_med:.3f} ms/call (events, median), {ach:.1f} TFLOP/s")
    del q, kv, out
    return dict(workload=f"dense (short) attention prefill: n={n}, H={H}, Dqk={Dqk}, Dv={Dv}, bf16",
                causal_pairs=pairs, flops_per_call=flops, kernel="sparse_attn_kernel", kernel_tflops=ach,
                peak_tflops=PEAK_BF16_TFLOPS, frac=ach / PEAK_BF16_TFLOPS, **tm.as_dict())


def bench_train(seed, steps, warmup):
    """The indexer's sparse-stage training step (indexer_loss_grad) on the
    n=8192 bf16 workload, over index_prefill's selection with a synthetic
    teacher.  Unit: one selected (query, key) pair; algorithmic flops per pair
    2*H^I*d^I each for the score, dq and dk contractions."""
    n, HI, DI, k = 8192, 64, 128, 2048
    log(f"train n={n}: generating inputs")
    inp = synth.indexer_prefill(1, n, HI, DI, synth.DT_BF16, seed, planted=True, device=DEV)
    S, _ = tl.index_prefill(inp.q, inp.k, inp.w, k)
    g = torch.Generator(device=DEV).manual_seed(seed)
    p = torch.rand((1, n, k), generator=g, device=DEV) ** 3 + 1e-3
    loss = torch.empty((1, n), dtype=torch.float32, device=DEV)
    dq = torch.empty((1, n, HI, DI), dtype=torch.float32, device=DEV)
    dk = torch.empty((1, n, DI), dtype=torch.float32, device=DEV)
    dw = torch.empty((1, n, HI), dtype=torch.float32, device=DEV)

    def call():
        tl.indexer_loss_grad(inp.q, inp.k, inp.w, S, p, loss=loss, dq=dq, dk=dk, dw=dw)

    tm = time_calls(call, steps, warmup, kernel="indexer_kl_kernel")
    pairs = int((S >= 0).sum().item())
    flops = 3 * 2.0 * HI * DI * pairs
    ach = flops / (tm.kernel_avg * 1e-3) / 1e12
    log(f"train: {tm.ev_med:.3f} ms/call (events, median), indexer_kl_kernel {tm.kernel_avg:.3f} ms, "
        f"{pairs / (tm.ev_med * 1e-3):.3g} pairs/s, {ach:.1f} TFLOP/s")
    del inp, S, p, dq, dk, dw
    return dict(workload=f"indexer training step (eq.(8) loss and gradient): B=1, n={n}, H^I={HI}, d^I={DI}, "
                         f"k={k}, bf16, index_prefill's selection, synthetic teacher",
                selected_pairs=pairs, pairs_per_s=pairs / (tm.wall * 1e-3), flops_per_call=flops,
                kernel="indexer_kl_kernel", kernel_tflops=ach, peak_tflops=PEAK_BF16_TFLOPS,
                frac=ach / PEAK_BF16_TFLOPS, **tm.as_dict())


def bench_dispatch(seed, steps, warmup):
    """dsa_prefill at n = k = 2048 (every row keeps all history, so it takes
    the dense path) against the two-call sparse path on the same inputs
    (fp8 indexer H^I=64, d^I=128; bf16 attention H=128, 576/512)."""
    n, k, H, Dqk, Dv = 2048, 2048, 128, 576, 512
    ix = synth.indexer_prefill(1, n, 64, 128, synth.DT_FP8, seed, planted=True, device=DEV)
    q, kv = synth.attn_prefill(1, n, H, Dqk, synth.DT_BF16, seed, device=DEV)
    scale = 1.0 / math.sqrt(Dqk)
    out = torch.empty((1, n, H, Dv), dtype=torch.bfloat16, device=DEV)
    S = torch.empty((1, n, k), dtype=torch.int32, device=DEV)
    ws = torch.empty(tl.index_prefill_workspace_bytes(ix.q, ix.k, ix.w, k, ix.q_scale, ix.k_scale), dtype=torch.uint8,
                     device=DEV)
    dws = torch.empty(256, dtype=torch.uint8, device=DEV)

    def dispatched():
        tl.dsa_prefill(ix.q, ix.k, ix.w, q, kv, k, scale, Dv, q_scale=ix.q_scale, k_scale=ix.k_scale, out=out,
                       workspace=dws)

    def two_calls():
        tl.index_prefill(ix.q, ix.k, ix.w, k, q_scale=ix.q_scale, k_scale=ix.k_scale, S=S, workspace=ws)
        tl.sparse_attn_prefill(q, kv, S, scale, Dv, out=out)

    td = time_calls(dispatched, steps, warmup)
    ts = time_calls(two_calls, steps, warmup)
    log(f"dispatch n={n} k={k}: dsa_prefill (dense path) {td.ev_med:.3f} ms, index_prefill + sparse_attn_prefill "
        f"{ts.ev_med:.3f} ms")
    del ix, q, kv, out, S, ws
    return dict(workload=f"prefill path chosen by length: n={n}, k={k} (every row keeps all history), fp8 indexer "
                         f"H^I=64 d^I=128, bf16 attention H={H} Dqk={Dqk} Dv={Dv}",
                dsa_prefill_dense_path=td.as_dict(), index_prefill_plus_sparse_attn=ts.as_dict(),
                speedup=ts.ev_med / td.ev_med)


def _overlap(Sa, Sb, k):
    """Mean fraction of Sb's selected positions that Sa also selects
    (rows [R,k], ascending then -1); analysis of the bench's outputs."""
    big = torch.iinfo(torch.int32).max
    a = torch.where(Sa < 0, big, Sa).reshape(-1, k)
    b = torch.where(Sb < 0, big, Sb).reshape(-1, k)
    idx = torch.searchsorted(a.contiguous(), b.contiguous()).clamp(max=k - 1)
    hit = (a.gather(1, idx) == b) & (b != big)
    return float(hit.sum()) / float((b != big).sum())


def bench_rerank(seed, steps, warmup):
    """fp8 coarse recall (k' = 4096) then bf16 re-rank to k = 2048 at n=32768,
    against the fp8 and the bf16 index_prefill at k = 2048 on the same values;
    the selections' agreement with the bf16 one."""
    n, HI, DI, k, kc = 32768, 64, 128, 2048, 4096
    inp = synth.indexer_prefill(1, n, HI, DI, synth.DT_BF16, seed, planted=True, device=DEV)
    q8, qs = synth.quantize_fp8_rows(inp.q.float(), 2)
    k8, ks = synth.quantize_fp8_rows(inp.k.float(), 1)
    S_rr = torch.empty((1, n, k), dtype=torch.int32, device=DEV)
    S_8 = torch.empty_like(S_rr)
    S_b = torch.empty_like(S_rr)
    ws_rr = torch.empty(_rerank_ws_bytes(n, k, kc), dtype=torch.uint8, device=DEV)
    ws_8 = torch.empty(tl.index_prefill_workspace_bytes(q8, k8, inp.w, k, qs, ks), dtype=torch.uint8, device=DEV)
    ws_b = torch.empty(tl.index_prefill_workspace_bytes(inp.q, inp.k, inp.w, k), dtype=torch.uint8, device=DEV)
    t_rr = time_calls(lambda: tl.index_prefill_rerank(q8, qs, k8, ks, inp.q, inp.k, inp.w, k, kc, S=S_rr,
                                                      workspace=ws_rr), steps, warmup, kernel="rerank_kernel")
    t_8 = time_calls(lambda: tl.index_prefill(q8, k8, inp.w, k, q_scale=qs, k_scale=ks, S=S_8, workspace=ws_8),
                     steps, warmup)
    t_b = time_calls(lambda: tl.index_prefill(inp.q, inp.k, inp.w, k, S=S_b, workspace=ws_b), steps, warmup)
    torch.cuda.synchronize()
    agree_rr, agree_8 = _overlap(S_rr, S_b, k), _overlap(S_8, S_b, k)
    log(f"rerank n={n}: fp8 k'={kc} + bf16 re-rank {t_rr.ev_med:.3f} ms (rerank_kernel {t_rr.kernel_avg:.3f} ms), "
        f"fp8 k={k} {t_8.ev_med:.3f} ms, bf16 k={k} {t_b.ev_med:.3f} ms; agreement with the bf16 selection: "
        f"re-ranked {agree_rr:.5f}, fp8 {agree_8:.5f}")
    del inp, q8, k8, S_rr, S_8, S_b, ws_rr, ws_8, ws_b
    return dict(workload=f"coarse recall + re-rank: B=1, n={n}, H^I={HI}, d^I={DI}, fp8 k'={kc}, bf16 re-rank to "
                         f"k={k}, planted keys",
                rerank=t_rr.as_dict(), fp8_index_prefill=t_8.as_dict(), bf16_index_prefill=t_b.as_dict(),
                agreement_with_bf16_selection={"reranked": agree_rr, "fp8_only": agree_8})


def _rerank_ws_bytes(n, k, kc):
    import ctypes
    lib = tl.load()
    size = ctypes.c_size_t(0)
    d = ctypes.c_void_p(16)
    rc = lib.index_prefill_rerank(d, d, d, d, d, d, d, 1, n, 64, 128, k, kc, d, None, None, None, ctypes.byref(size),
                                  None)
    assert rc == 0, lib.tlsl_last_error()
    return size.value


def bench_tiny(steps, warmup):
    """The tiny fp32 configuration (dyadic indexer inputs, exact scores):
    index_prefill and sparse_attn_prefill timed separately; report only."""
    B, n, HI, DI, k, H, Dqk, Dv = 1, 512, 4, 32, 64, 4, 80, 64
    inp = synth.indexer_prefill(B, n, HI, DI, synth.DT_F32, 1, dist="dyadic", device=DEV)
    ws = torch.empty(tl.index_prefill_workspace_bytes(inp.q, inp.k, inp.w, k), dtype=torch.uint8, device=DEV)
    S = torch.empty((B, n, k), dtype=torch.int32, device=DEV)
    ti = time_calls(lambda: tl.index_prefill(inp.q, inp.k, inp.w, k, S=S, workspace=ws), steps, warmup)
    q, kv = synth.attn_prefill(B, n, H, Dqk, synth.DT_F32, 1, device=DEV)
    out = torch.empty((B, n, H, Dv), dtype=torch.float32, device=DEV)
    ta = time_calls(lambda: tl.sparse_attn_prefill(q, kv, S, 1.0 / math.sqrt(Dqk), Dv, out=out), steps, warmup)
    pairs = causal_pairs(B, n)
    log(f"tiny f32 n={n}: index_prefill {ti.ev_med * 1e3:.1f} us, sparse_attn_prefill {ta.ev_med * 1e3:.1f} us")
    return dict(workload=f"tiny prefill: B=1, n={n}, H^I={HI}, d^I={DI}, k={k}, f32 dyadic; attention H={H}, "
                         f"Dqk={Dqk}, Dv={Dv}, f32 (report only: launch-bound)",
                pairs_per_s=pairs / (ti.wall * 1e-3), index_prefill=ti.as_dict(), sparse_attn_prefill=ta.as_dict())


def decode_bytes(lengths, HI, DI, H, Dqk, Dv, k):
    """Algorithmic HBM bytes of one decode step (score round trip excluded)."""
    L = np.asarray(lengths, dtype=np.float64)
    B = len(L)
    return float((L * (DI + 4)).sum() + (np.minimum(k, L) * Dqk * 2).sum()
                 + B * (HI * DI + 4 + 4 * HI) + B * H * (Dqk + Dv) * 2 + B * k * 4)


def decode_stage_bytes(lengths, HI, DI, H, Dqk, Dv, k):
    """Algorithmic bytes of each decode stage's main kernel: its inputs read
    once and its outputs written once."""
    L = np.asarray(lengths, dtype=np.float64)
    B = len(L)
    K = np.minimum(k, L)
    return {
        # K^I cache + scales, queries + scale + weights, scores out
        "decode_scan_kernel": float((L * (DI + 4 + 4)).sum() + B * (HI * DI + 4 + 4 * HI)),
        # scores in (full rows), S out
        "topk_filter_kernel": float((L * 4).sum() + B * k * 4),
        # gathered entries, queries, S, outputs
        "sparse_attn_kernel": float((K * Dqk * 2).sum() + B * H * Dqk * 2 + B * k * 4 + B * H * Dv * 2),
    }


def _margin_ws_bytes(R, k, max_len):
    """Workspace size of cutoff_margin (size query through the C ABI)."""
    import ctypes
    lib = tl.load()
    size = ctypes.c_size_t(0)
    d = ctypes.c_void_p(16)
    rc = lib.cutoff_margin(d, d, d, int(R), int(k), int(max_len), d, None, ctypes.byref(size), None)
    assert rc == 0, lib.tlsl_last_error()
    return size.value


def _quality_ws_bytes(R, k, m, max_len):
    """Workspace size of selection_quality (size query through the C ABI)."""
    import ctypes
    lib = tl.load()
    size = ctypes.c_size_t(0)
    d = ctypes.c_void_p(16)
    rc = lib.selection_quality(d, d, d, int(R), d, int(k), int(m), int(max_len), d, d, None, ctypes.byref(size), None)
    assert rc == 0, lib.tlsl_last_error()
    return size.value


def bench_decode(seed, steps, warmup):
    B, HI, DI, H, Dqk, Dv, k = 64, 64, 128, 128, 576, 512, 2048
    torch.cuda.reset_peak_memory_stats()
    lengths = synth.decode_lengths(B, 16384, 131072, seed)
    log(f"decode: sumL={int(lengths.sum())}: generating inputs")
    di = synth.indexer_decode(lengths, HI, DI, synth.DT_FP8, seed, device=DEV)
    qa, kva = synth.attn_decode(lengths, H, Dqk, synth.DT_BF16, seed, device=DEV)
    cu = di.cu_seqlens
    row_start = cu[:-1].contiguous()
    row_len = torch.as_tensor(lengths, dtype=torch.int32, device=DEV)
    max_len = int(lengths.max())
    scores = torch.empty(int(lengths.sum()), dtype=torch.float32, device=DEV)
    S = torch.empty((B, k), dtype=torch.int32, device=DEV)
    out = torch.empty((B, H, Dv), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(tl.sparse_attn_decode_workspace_bytes(qa, kva, S, Dv), dtype=torch.uint8, device=DEV)
    tws = torch.empty(tl.topk_select_workspace_bytes(B, k, max_len), dtype=torch.uint8, device=DEV)
    scale = 1.0 / math.sqrt(Dqk)

    def f_index():
        tl.index_decode(di.q, di.k, di.w, cu, max_len, q_scale=di.q_scale, k_scale=di.k_scale, scores=scores)

    def f_topk():
        tl.topk_select(scores, row_start, row_len, k, max_len, S=S, workspace=tws)

    def f_attn():
        tl.sparse_attn_decode(qa, kva, cu, S, scale, Dv, out=out, workspace=ws)

    def step():
        f_index()
        f_topk()
        f_attn()

    tm = time_calls(step, steps, warmup)
    nbytes = decode_bytes(lengths, HI, DI, H, Dqk, Dv, k)
    gbs = nbytes / (tm.ev_med * 1e-3) / 1e9
    # per stage: the whole call, and its main kernel on its own events
    sbytes = decode_stage_bytes(lengths, HI, DI, H, Dqk, Dv, k)
    stages = {}
    for name, fn, kerns in (("index_decode", f_index, ("decode_scan_kernel",)),
                            ("topk_select", f_topk, ("topk_threshold_kernel", "topk_filter_kernel",
                                                     "topk_final_kernel")),
                            ("sparse_attn_decode", f_attn, ("sparse_attn_kernel", "attn_combine_kernel"))):
        st = None
        kd = {}
        for kern in kerns:
            st = time_calls(fn, max(5, steps // 2), 1, kernel=kern)
            kd[kern] = {"kernel_ms_avg": st.kernel_avg}
            if kern in sbytes:
                kg = sbytes[kern] / (st.kernel_avg * 1e-3) / 1e9
                kd[kern].update(algorithmic_bytes=sbytes[kern], gbs=kg, frac=kg / PEAK_HBM_GBS)
        stages[name] = dict(event_ms_median=st.ev_med, event_ms_min=st.ev_min, kernels=kd)
    log(f"decode: {tm.ev_med:.3f} ms/step (median; min {tm.ev_min:.3f}), {gbs:.0f} GB/s; stages " +
        "; ".join(f"{n_}: {v['event_ms_median']:.3f} ms (" +
                  ", ".join(f"{kn} {kv['kernel_ms_avg']:.3f} ms" + (f" {kv['gbs']:.0f} GB/s" if 'gbs' in kv else "")
                            for kn, kv in v["kernels"].items()) + ")" for n_, v in stages.items()))
    # selection-quality diagnostics on the step's rows: the cutoff margin of
    # the indexer scores and recall / mass of a synthetic teacher (mass 1 on
    # each sequence's planted keys, a small uniform floor elsewhere)
    teacher = torch.full_like(scores, 1e-4)
    for b, pos in di.planted.items():
        teacher[int(cu[b]) + torch.as_tensor(pos, device=DEV)] = 1.0
    mg = torch.empty(B, dtype=torch.float32, device=DEV)
    rec = torch.empty(B, dtype=torch.float32, device=DEV)
    mass = torch.empty(B, dtype=torch.float32, device=DEV)
    mws = torch.empty(_margin_ws_bytes(B, k, max_len), dtype=torch.uint8, device=DEV)
    qws = torch.empty(_quality_ws_bytes(B, k, 32, max_len), dtype=torch.uint8, device=DEV)

    def f_diag():
        tl.cutoff_margin(scores, row_start, row_len, k, max_len, margin=mg, workspace=mws)
        tl.selection_quality(teacher, row_start, row_len, S, 32, max_len, recall=rec, mass=mass, workspace=qws)

    tdg = time_calls(f_diag, max(5, steps // 2), 2)
    diag = dict(event_ms_median=tdg.ev_med, teacher_bytes=float(lengths.sum() * 4),
                margin_median=float(mg.median()), recall_top32_mean=float(rec.mean()), mass_mean=float(mass.mean()))
    log(f"decode diagnostics: cutoff_margin + selection_quality {tdg.ev_med:.3f} ms; margin median "
        f"{diag['margin_median']:.3g}, recall of the planted keys {diag['recall_top32_mean']:.3f}, "
        f"mass {diag['mass_mean']:.3f}")
    Sh = S.cpu().numpy()
    hit = tot = 0
    for b, pos in di.planted.items():
        sel = set(Sh[b][Sh[b] >= 0].tolist())
        hit += sum(p in sel for p in pos)
        tot += len(pos)
    planted_hit = hit / max(tot, 1)
    del qa, kva, di
    return dict(workload=f"decode step: {B} sequences, L ~ U[16384,131072] (sumL={int(lengths.sum())}), "
                         f"fp8 indexer H^I={HI} d^I={DI}, top-{k}, bf16 attention H={H} Dqk={Dqk} Dv={Dv}",
                tokens_per_s=B / (tm.wall * 1e-3), bytes_per_step=nbytes, achieved_gbs=gbs,
                peak_gbs=PEAK_HBM_GBS, frac=gbs / PEAK_HBM_GBS, stages=stages, planted_recall=planted_hit,
                peak_device_bytes=torch.cuda.max_memory_allocated(),
                diagnostics=diag,
                **tm.as_dict())


def calibrate(steps):
    """Achievable rates on this device: a streaming copy and matrix-core loops."""
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device=DEV).fill_(1)
    dst = torch.empty_like(src)
    tm = time_calls(lambda: tl.calib_copy(src, dst), max(5, steps // 2), 2, kernel="calib_copy_kernel")
    copy_gbs = 2.0 * nbytes / (tm.kernel_avg * 1e-3) / 1e9
    del src, dst
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(cus * 8 * 256, dtype=torch.float32, device=DEV)
    res = dict(copy_bytes=nbytes, copy_gbs=copy_gbs, copy_frac_of_peak=copy_gbs / PEAK_HBM_GBS)
    # ~15 ms per launch: 2 ms launches read a few percent below the rate the
    # loop sustains (fp8: ~4.75 against ~4.95 PFLOP/s)
    for name, dt, iters, peak in (("bf16", tl.BF16, 32000, PEAK_BF16_TFLOPS), ("fp8", tl.FP8_E4M3, 16000,
                                                                               PEAK_FP8_TFLOPS)):
        fl = [0.0]

        def run():
            fl[0] = tl.calib_mfma(dt, cus * 8, iters, sink)

        t = time_calls(run, 5, 1, kernel="calib_mfma_kernel")
        tf = fl[0] / (t.kernel_avg * 1e-3) / 1e12
        res[f"mfma_{name}_tflops"] = tf
        res[f"mfma_{name}_frac_of_peak"] = tf / peak
    log("calibration: copy {copy_gbs:.0f} GB/s, bf16 loop {mfma_bf16_tflops:.0f} TFLOP/s, "
        "fp8 loop {mfma_fp8_tflops:.0f} TFLOP/s".format(**res))
    return res


def cpu_baseline(inp, k, n, S_gpu=None, target_s=15.0):
    """Oracle pairs/s on a bounded, evenly spread sample of query rows.

    A short calibration call sizes the sample to about ``target_s`` seconds.
    When the GPU's selection of the workload (``S_gpu`` [n, k], on the host)
    is given, the oracle's selections of the sampled rows are compared with
    it: the fraction of identical slots and the rows that differ (the margin
    rule on the differing slots is the GPU tests' job: it needs every score
    of the row)."""
    import oracle
    from oracle import parity
    sn = synth.storage_to_numpy
    oracle.build()
    nthreads = oracle.num_threads()
    q, qs, kk, ks, w = sn(inp.q), sn(inp.q_scale), sn(inp.k), sn(inp.k_scale), sn(inp.w)
    last = {}

    def run(rows):
        t0 = time.perf_counter()
        last["S"] = oracle.index_prefill_rows(inp.dt, q, qs, kk, ks, w, k, rows)[0]
        return time.perf_counter() - t0

    cal = np.linspace(n // 2, n - 1, nthreads).astype(np.int64)
    rate = (cal + 1).sum() / max(run(cal), 1e-3)            # pairs/s
    want_pairs = rate * target_s
    rows_n = int(np.clip(want_pairs / (n / 2), nthreads, n))
    sel = np.unique(np.linspace(0, n - 1, rows_n).astype(np.int64))
    dt = run(sel)
    pairs = int((sel + 1).sum())
    res = dict(value=pairs / dt, unit="pairs/s", cores=nthreads, kind="oracle",
               sample=f"{len(sel)} evenly spaced query rows of the headline workload "
                      f"({pairs} causal pairs, {dt:.1f} s, double precision, OpenMP over rows)")
    if S_gpu is not None:
        rep = parity.check_selection(S_gpu[sel], last["S"], sel, k)
        res["parity"] = dict(rows=rep.rows, slots=rep.slots, match=rep.matched / max(rep.slots, 1),
                             rows_differing=rep.mismatched_rows, structure_errors=len(rep.structure_errors))
        log(f"parity on the sampled rows: match {res['parity']['match']:.6f}, {rep.mismatched_rows} of "
            f"{rep.rows} rows differ, {len(rep.structure_errors)} structure errors")
    return res


# HBM traffic of a kernel per launch on one workload, from two rocprofv3 --pmc
# runs (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch, averaged over the
# kernel's dispatches), each scaled by the same counter's reading for the
# 1 GiB calibration copy of the same run (the reading that counts the copy's
# bytes exactly).  The figures hold only for the kernel sources they were
# taken on: when the hash of those sources differs, traffic is reported as
# null.  Commands and readings: profiles/prefill_score_kernel_fp8_n131072.md.
TRAFFIC_SOURCES = ("indexer.hip", "idx_tile.h", "tlsl_device.h", "tlsl_internal.h", "topk_common.h")
# HBM bytes per launch from two rocprofv3 counter passes over `bench.py --quick`
# (profiles/prefill_score_kernel_fp8_n131072.md): FETCH_SIZE and WRITE_SIZE in
# KiB per dispatch, each scaled by what the same counter reads for the 1 GiB
# calibration copy of the same run; valid while the kernel's sources hash the same
TRAFFIC = {
    ("prefill_score_kernel", "fp8_n131072"): {
        "fetch_kib": 2787172, "write_kib": 3200011,
        "copy_fetch_kib": 524301, "copy_write_kib": 1048576, "copy_bytes": 1073741824,
        "sources_sha256": "69459af235cee1be62cc17890bf0537816fb708a1b05b1620bd783b2c062b270",
    },
}


def sources_sha256(names):
    import hashlib
    h = hashlib.sha256()
    for nm in names:
        with open(os.path.join(ROOT, "token_level_sparse_lightning_amd", "csrc", nm), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(kernel, workload):
    rec = TRAFFIC.get((kernel, workload))
    if not rec or rec["sources_sha256"] != sources_sha256(TRAFFIC_SOURCES):
        return None
    copy = float(rec["copy_bytes"])
    return (rec["fetch_kib"] * copy / rec["copy_fetch_kib"] + rec["write_kib"] * copy / rec["copy_write_kib"])


EXTRAS = ("attn_prefill_131072", "prefill_bf16_8192", "prefill_fp8_32768", "attn_prefill_32768",
          "attn_dense_2048", "dispatch_2048", "rerank_32768", "decode", "train_8192", "tiny_f32_512")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--quick", action="store_true", help="headline workload (and calibration) only")
    ap.add_argument("--only", default="", help="comma list of extra workloads to run (default: all of "
                    + ",".join(EXTRAS) + ")")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-calib", action="store_true", help="skip the copy and matrix-core calibration")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (every workload runs on one "
              "device); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    tl.load()
    want = set() if args.quick else (set(args.only.split(",")) if args.only else set(EXTRAS))
    unknown = want - set(EXTRAS)
    if unknown:
        print(f"unknown workloads {sorted(unknown)}; choose from {EXTRAS}", file=sys.stderr)
        sys.exit(2)

    N_HEAD, K_HEAD, SEED_HEAD = 131072, 2048, 5
    head, inp, S = bench_prefill(N_HEAD, synth.DT_FP8, SEED_HEAD, args.steps, args.warmup, plant_max_dist=100000)
    # the headline inputs (and, for the parity statistics of the CPU baseline,
    # its selection) go to the host and are freed on the device before the
    # other workloads
    inp = synth.IndexerPrefill(inp.dt, inp.q.cpu(), inp.q_scale.cpu(), inp.k.cpu(), inp.k_scale.cpu(), inp.w.cpu(),
                               inp.probes)
    S_host = None if args.no_cpu else S[0].cpu().numpy()
    torch.cuda.empty_cache()
    extra = {}
    if "attn_prefill_131072" in want:
        extra["attn_prefill_131072"] = bench_attn_prefill(S, N_HEAD, SEED_HEAD, max(3, args.steps // 4), 1)
    del S
    torch.cuda.empty_cache()
    if "prefill_bf16_8192" in want:
        extra["prefill_bf16_8192"], _, S2 = bench_prefill(8192, synth.DT_BF16, 2, args.steps, args.warmup)
        del S2
        torch.cuda.empty_cache()
    if want & {"prefill_fp8_32768", "attn_prefill_32768"}:
        fp8, _, S3 = bench_prefill(32768, synth.DT_FP8, 3, max(5, args.steps // 2), 2)
        if "prefill_fp8_32768" in want:
            extra["prefill_fp8_32768"] = fp8
        if "attn_prefill_32768" in want:
            extra["attn_prefill_32768"] = bench_attn_prefill(S3, 32768, 3, max(3, args.steps // 4), 1)
        del S3
        torch.cuda.empty_cache()
    if "attn_dense_2048" in want:
        extra["attn_dense_2048"] = bench_attn_dense(2048, 6, max(5, args.steps // 2), 2)
        torch.cuda.empty_cache()
    if "dispatch_2048" in want:
        extra["dispatch_2048"] = bench_dispatch(7, max(5, args.steps // 2), 2)
        torch.cuda.empty_cache()
    if "rerank_32768" in want:
        extra["rerank_32768"] = bench_rerank(3, max(3, args.steps // 4), 1)
        torch.cuda.empty_cache()
    if "decode" in want:
        extra["decode"] = bench_decode(4, args.steps, args.warmup)
        torch.cuda.empty_cache()
    if "train_8192" in want:
        extra["train_8192"] = bench_train(2, max(5, args.steps // 2), 2)
        torch.cuda.empty_cache()
    if "tiny_f32_512" in want:
        extra["tiny_f32_512"] = bench_tiny(args.steps, args.warmup)
        torch.cuda.empty_cache()
    calib = None if args.no_calib else calibrate(args.steps)
    cpu = None if args.no_cpu else cpu_baseline(inp, K_HEAD, N_HEAD, S_gpu=S_host)

    roofline = {"bound": "mfma", "achieved": head["kernel_tflops"], "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                "frac": head["frac"],
                "traffic": recorded_traffic("prefill_score_kernel", "fp8_n131072"),
                "kernel": "prefill_score_kernel", "kernel_ms": head["kernel_ms_avg"],
                "launches": head["kernel_launches"], "flops_per_launch": head["flops_per_call"],
                "algorithmic_bytes_per_launch": head["algorithmic_bytes_per_call"]}
    if calib:
        roofline["measured_peak"] = calib["mfma_fp8_tflops"]
        roofline["frac_of_measured_peak"] = head["kernel_tflops"] / calib["mfma_fp8_tflops"]
    line = {
        "metric": "indexer+top-k query-key pairs/s (prefill)",
        "value": head["pairs_per_s"],
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_call"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": head["workload"], "B": 1, "n": N_HEAD, "H_I": 64, "d_I": 128, "k": K_HEAD,
                   "indexer_dtype": "fp8_e4m3 with per-token fp32 scales", "seed": SEED_HEAD},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "headline": head,
        "calibration": calib,
        "extra": extra,
        "library_sources_sha256": sources_sha256(sorted(
            f for f in os.listdir(os.path.join(ROOT, "token_level_sparse_lightning_amd", "csrc"))
            if f.endswith((".hip", ".cpp", ".h")))),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
