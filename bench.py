"""Benchmark of the DSA token-selection path on one MI355X.

Prints ONE JSON line.  The headline is the prefill Lightning Indexer + causal
top-k (index_prefill) on B=1, n=8192, H^I=64, d^I=128, k=2048, bf16 inputs
with planted keys; its metric is causal query-key pairs per second (a pair is
(t, s) with s <= t; B*n*(n+1)/2 per call).  The same line carries the other
rows of the path measured on their own workloads:

  prefill_fp8   index_prefill, n=32768, fp8 e4m3 with per-token scales
  prefill_long  index_prefill, n=131072, fp8                       (--long)
  attn_prefill  sparse_attn_prefill over that selection, n=32768,
                H=128, Dqk=576, Dv=512, bf16
  decode        one decode step of 64 ragged sequences (L ~ U[16384,131072]):
                index_decode + topk_select + sparse_attn_decode, tokens/s

Timing: W untimed warm-up calls, then exactly K calls between two device
synchronisations (wall clock), plus HIP events on the launch stream around
every timed call (the kernel time the roofline uses).  Inputs are resident in
HBM before the timed region; workspaces are allocated once outside it.

The CPU baseline times the oracle (test infrastructure, double precision) on
a bounded sample of query rows of the headline workload.
"""
from __future__ import annotations

import argparse
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


def time_calls(fn, steps, warmup):
    """Returns (wall ms per call, event ms per call)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record(st)
        fn()
        b.record(st)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    ev = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    return wall, ev


def causal_pairs(B, n):
    return B * n * (n + 1) // 2


# ---------------------------------------------------------------------------
def bench_prefill(n, dt, seed, steps, warmup, plant_max_dist=None):
    HI, DI, k = 64, 128, 2048
    log(f"prefill n={n} dt={synth.DT_NAMES[dt]}: generating inputs")
    inp = synth.indexer_prefill(1, n, HI, DI, dt, seed, planted=True, plant_max_dist=plant_max_dist,
                                device=DEV)
    ws = torch.empty(tl.index_prefill_workspace_bytes(inp.q, inp.k, inp.w, k, inp.q_scale, inp.k_scale),
                     dtype=torch.uint8, device=DEV)
    S = torch.empty((1, n, k), dtype=torch.int32, device=DEV)

    def call():
        tl.index_prefill(inp.q, inp.k, inp.w, k, q_scale=inp.q_scale, k_scale=inp.k_scale, S=S, workspace=ws)

    wall, ev = time_calls(call, steps, warmup)
    pairs = causal_pairs(1, n)
    flops = 2.0 * HI * DI * pairs
    peak = PEAK_FP8_TFLOPS if dt == synth.DT_FP8 else PEAK_BF16_TFLOPS
    ach = flops / (ev * 1e-3) / 1e12
    log(f"prefill n={n}: {ev:.3f} ms/call (events), {wall:.3f} ms (wall), {ach:.1f} TFLOP/s")
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
    res = dict(workload=f"prefill indexer + top-k: B=1, n={n}, H^I={HI}, d^I={DI}, k={k}, "
                        f"{synth.DT_NAMES[dt]}, planted keys",
               pairs_per_s=pairs / (wall * 1e-3), ms_per_call=wall, kernel_ms=ev, pairs=pairs,
               flops_per_call=flops, achieved_tflops=ach, peak_tflops=peak, frac=ach / peak,
               planted_recall=recall)
    return res, inp, S


def bench_attn_prefill(S, n, seed, steps, warmup):
    H, Dqk, Dv = 128, 576, 512
    log(f"attn prefill n={n}: generating inputs")
    q, kv = synth.attn_prefill(1, n, H, Dqk, synth.DT_BF16, seed, device=DEV)
    out = torch.empty((1, n, H, Dv), dtype=torch.bfloat16, device=DEV)
    scale = 1.0 / math.sqrt(Dqk)

    def call():
        tl.sparse_attn_prefill(q, kv, S, scale, Dv, out=out)

    wall, ev = time_calls(call, steps, warmup)
    valid = int((S >= 0).sum().item())
    flops = 2.0 * H * (Dqk + Dv) * valid
    ach = flops / (ev * 1e-3) / 1e12
    log(f"attn prefill: {ev:.3f} ms/call, {ach:.1f} TFLOP/s")
    del q, kv, out
    return dict(workload=f"sparse attention prefill: n={n}, H={H}, Dqk={Dqk}, Dv={Dv}, k=2048, bf16",
                ms_per_call=wall, kernel_ms=ev, valid_slots=valid, flops_per_call=flops,
                achieved_tflops=ach, peak_tflops=PEAK_BF16_TFLOPS, frac=ach / PEAK_BF16_TFLOPS)


def decode_bytes(lengths, HI, DI, H, Dqk, Dv, k):
    """Algorithmic HBM bytes of one decode step (score round trip excluded)."""
    L = np.asarray(lengths, dtype=np.float64)
    B = len(L)
    return float((L * (DI + 4)).sum() + (np.minimum(k, L) * Dqk * 2).sum()
                 + B * (HI * DI + 4 + 4 * HI) + B * H * (Dqk + Dv) * 2 + B * k * 4)


def bench_decode(seed, steps, warmup):
    B, HI, DI, H, Dqk, Dv, k = 64, 64, 128, 128, 576, 512, 2048
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

    def step():
        tl.index_decode(di.q, di.k, di.w, cu, max_len, q_scale=di.q_scale, k_scale=di.k_scale, scores=scores)
        tl.topk_select(scores, row_start, row_len, k, max_len, S=S, workspace=tws)
        tl.sparse_attn_decode(qa, kva, cu, S, scale, Dv, out=out, workspace=ws)

    wall, ev = time_calls(step, steps, warmup)
    # per-stage event timing
    stages = {}
    for name, fn in (("index_decode", lambda: tl.index_decode(di.q, di.k, di.w, cu, max_len, q_scale=di.q_scale,
                                                               k_scale=di.k_scale, scores=scores)),
                     ("topk_select", lambda: tl.topk_select(scores, row_start, row_len, k, max_len, S=S, workspace=tws)),
                     ("sparse_attn_decode", lambda: tl.sparse_attn_decode(qa, kva, cu, S, scale, Dv, out=out,
                                                                          workspace=ws))):
        stages[name] = time_calls(fn, max(3, steps // 2), 1)[1]
    nbytes = decode_bytes(lengths, HI, DI, H, Dqk, Dv, k)
    gbs = nbytes / (ev * 1e-3) / 1e9
    log(f"decode: {ev:.3f} ms/step, {gbs:.0f} GB/s, stages {stages}")
    planted_hit = None
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
                tokens_per_s=B / (wall * 1e-3), ms_per_step=wall, kernel_ms=ev, bytes_per_step=nbytes,
                achieved_gbs=gbs, peak_gbs=PEAK_HBM_GBS, frac=gbs / PEAK_HBM_GBS, stage_ms=stages,
                planted_recall=planted_hit)


def cpu_baseline(inp, k, n, target_s=15.0):
    """Oracle pairs/s on a bounded, evenly spread sample of query rows.

    A short calibration call sizes the sample to about ``target_s`` seconds."""
    import oracle
    sn = synth.storage_to_numpy
    oracle.build()
    nthreads = oracle.num_threads()
    q, qs, kk, ks, w = sn(inp.q), sn(inp.q_scale), sn(inp.k), sn(inp.k_scale), sn(inp.w)

    def run(rows):
        t0 = time.perf_counter()
        oracle.index_prefill_rows(inp.dt, q, qs, kk, ks, w, k, rows)
        return time.perf_counter() - t0

    cal = np.linspace(n // 2, n - 1, nthreads).astype(np.int64)
    rate = (cal + 1).sum() / max(run(cal), 1e-3)            # pairs/s
    want_pairs = rate * target_s
    rows_n = int(np.clip(want_pairs / (n / 2), nthreads, n))
    sel = np.unique(np.linspace(0, n - 1, rows_n).astype(np.int64))
    dt = run(sel)
    pairs = int((sel + 1).sum())
    return dict(value=pairs / dt, unit="pairs/s", cores=nthreads, kind="oracle",
                sample=f"{len(sel)} evenly spaced query rows of the headline workload "
                       f"({pairs} causal pairs, {dt:.1f} s, double precision, OpenMP over rows)")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=2)
    ap.add_argument("--long", action="store_true", help="also time the n=131072 prefill")
    ap.add_argument("--quick", action="store_true", help="headline workload only")
    ap.add_argument("--only", default="", help="comma list of extra workloads to run: "
                    "prefill_fp8,attn_prefill,decode,prefill_long (default: all but prefill_long)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (every workload runs on one "
              "device); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    tl.load()

    head, inp, S = bench_prefill(8192, synth.DT_BF16, args.seed, args.steps, args.warmup)
    extra = {}
    want = set(args.only.split(",")) if args.only else {"prefill_fp8", "attn_prefill", "decode"}
    if args.long:
        want.add("prefill_long")
    if not args.quick:
        if want & {"prefill_fp8", "attn_prefill"}:
            fp8, _, S3 = bench_prefill(32768, synth.DT_FP8, args.seed + 1, max(5, args.steps // 2), 2)
            extra["prefill_fp8"] = fp8
            if "attn_prefill" in want:
                extra["attn_prefill"] = bench_attn_prefill(S3, 32768, args.seed + 1, max(3, args.steps // 4), 1)
            del S3
            torch.cuda.empty_cache()
        if "decode" in want:
            extra["decode"] = bench_decode(args.seed + 3, args.steps, args.warmup)
            torch.cuda.empty_cache()
        if "prefill_long" in want:
            lg, _, _ = bench_prefill(131072, synth.DT_FP8, args.seed + 4, 3, 1, plant_max_dist=100000)
            extra["prefill_long"] = lg
    cpu = None if args.no_cpu else cpu_baseline(inp, 2048, 8192)

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
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": head["workload"], "B": 1, "n": 8192, "H_I": 64, "d_I": 128, "k": 2048,
                   "seed": args.seed},
        "roofline": {"bound": "mfma", "achieved": head["achieved_tflops"], "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": head["frac"], "traffic": None,
                     "kernel": "index_prefill (score + finalize + fallback kernels)",
                     "flops_per_launch": head["flops_per_call"], "kernel_ms": head["kernel_ms"]},
        "cpu_baseline": cpu,
        "planted_recall": head["planted_recall"],
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
