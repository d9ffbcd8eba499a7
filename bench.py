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
  attn_dense    dense_attn_prefill (short prefill: n <= k, every query over
                all of its history), n=2048, same heads and dims
  decode        one decode step of 64 ragged sequences (L ~ U[16384,131072]):
                index_decode + topk_select + sparse_attn_decode, tokens/s

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
               planted_recall=recall, **tm.as_dict())
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
    for name, dt, iters, peak in (("bf16", tl.BF16, 4000, PEAK_BF16_TFLOPS), ("fp8", tl.FP8_E4M3, 2000,
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


# HBM traffic of the headline kernel per launch, from two rocprofv3 --pmc runs of
# `bench.py --no-cpu --only decode --steps 3 --warmup 1` (FETCH_SIZE, then WRITE_SIZE,
# KiB per dispatch, averaged over the dispatches of the kernel), each scaled by
# the same counter's reading for the 1 GiB calibration copy (the reading that
# counts the copy's writes exactly; see profiles/prefill_score_kernel_bf16_n8192.md).
# The figures hold only for the kernel sources they were taken on: when the
# hash of those sources differs, the traffic is reported as null.
TRAFFIC_SOURCES = ("indexer.hip", "tlsl_device.h", "tlsl_internal.h", "topk_common.h")
TRAFFIC = {
    # profiles/prefill_score_kernel_bf16_n8192.md
    "prefill_score_kernel": {
        "sources_sha256": "848709082d78f13485d39216b597162e4cf04d8960f2fd8cd033ca121fb9af4d",
        "fetch_kib": 85372.9062, "write_kib": 168480.1562,
        "copy_fetch_kib": 524302.1429, "copy_write_kib": 1048576.0, "copy_bytes": 1 << 30,
    },
}


def sources_sha256(names):
    import hashlib
    h = hashlib.sha256()
    for nm in names:
        with open(os.path.join(ROOT, "token_level_sparse_lightning_amd", "csrc", nm), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(kernel):
    rec = TRAFFIC.get(kernel)
    if not rec or rec["sources_sha256"] != sources_sha256(TRAFFIC_SOURCES):
        return None
    copy = float(rec["copy_bytes"])
    return (rec["fetch_kib"] * copy / rec["copy_fetch_kib"] + rec["write_kib"] * copy / rec["copy_write_kib"])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=2)
    ap.add_argument("--long", action="store_true", help="also time the n=131072 prefill")
    ap.add_argument("--quick", action="store_true", help="headline workload (and calibration) only")
    ap.add_argument("--only", default="", help="comma list of extra workloads to run: "
                    "prefill_fp8,attn_prefill,attn_dense,decode,prefill_long (default: all but prefill_long)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-calib", action="store_true", help="skip the copy and matrix-core calibration")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (every workload runs on one "
              "device); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    tl.load()

    head, inp, S = bench_prefill(8192, synth.DT_BF16, args.seed, args.steps, args.warmup)
    # the headline inputs stay on the host for the CPU baseline and are freed
    # on the device before the other workloads
    inp = synth.IndexerPrefill(inp.dt, inp.q.cpu(), None if inp.q_scale is None else inp.q_scale.cpu(), inp.k.cpu(),
                               None if inp.k_scale is None else inp.k_scale.cpu(), inp.w.cpu(), inp.probes)
    del S
    torch.cuda.empty_cache()
    extra = {}
    want = set(args.only.split(",")) if args.only else {"prefill_fp8", "attn_prefill", "attn_dense", "decode"}
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
        if "attn_dense" in want:
            extra["attn_dense"] = bench_attn_dense(2048, args.seed + 2, max(5, args.steps // 2), 2)
            torch.cuda.empty_cache()
        if "decode" in want:
            extra["decode"] = bench_decode(args.seed + 3, args.steps, args.warmup)
            torch.cuda.empty_cache()
        if "prefill_long" in want:
            lg, _, _ = bench_prefill(131072, synth.DT_FP8, args.seed + 4, 3, 1, plant_max_dist=100000)
            extra["prefill_long"] = lg
    calib = None if args.no_calib else calibrate(args.steps)
    cpu = None if args.no_cpu else cpu_baseline(inp, 2048, 8192)

    roofline = {"bound": "mfma", "achieved": head["kernel_tflops"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": head["frac"], "traffic": recorded_traffic("prefill_score_kernel"),
                "kernel": "prefill_score_kernel", "kernel_ms": head["kernel_ms_avg"],
                "launches": head["kernel_launches"], "flops_per_launch": head["flops_per_call"],
                "algorithmic_bytes_per_launch": head["algorithmic_bytes_per_call"]}
    if calib:
        roofline["measured_peak"] = calib["mfma_bf16_tflops"]
        roofline["frac_of_measured_peak"] = head["kernel_tflops"] / calib["mfma_bf16_tflops"]
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
        "roofline": roofline,
        "cpu_baseline": cpu,
        "headline": head,
        "calibration": calib,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
