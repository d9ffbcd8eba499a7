"""Helpers shared by the GPU parity tests."""
import sys

import numpy as np
import torch

from token_level_sparse_lightning_amd import synth

DEV = "cuda:0"


def announce(msg: str):
    """Name the case before a GPU step (so a failing run says which one)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(x):
    return None if x is None else x.to(DEV, non_blocking=False).contiguous()


def host(x):
    return synth.storage_to_numpy(x)


def sample_rows(n, k, count, seed=0, extra=()):
    """Query rows to check against the oracle: edges around k and n, plus random."""
    base = {0, 1, min(n - 1, k - 2), min(n - 1, k - 1), min(n - 1, k), min(n - 1, k + 1), n - 1, n - 2}
    base |= {int(e) for e in extra if 0 <= e < n}
    rng = np.random.default_rng(seed)
    rest = rng.choice(n, size=min(n, count), replace=False)
    return np.array(sorted({int(x) for x in base if 0 <= x < n} | {int(x) for x in rest}), dtype=np.int64)


def stratified_rows(n, k, probes=(), uniform=0, seed=0):
    """The stratified query-row sample of the full-size checks: the edges of
    the selection rule t in {0, k-2, k-1, k, n-1} (where min(k, t+1) switches
    from "every position" to a real selection), every probe row (the queries
    with planted keys), and ``uniform`` more rows drawn uniformly."""
    base = {0, k - 2, k - 1, k, n - 1} | {int(t) for t in probes}
    rng = np.random.default_rng(seed)
    extra = rng.choice(n, size=min(n, uniform), replace=False) if uniform else []
    return np.array(sorted(t for t in base | {int(x) for x in extra} if 0 <= t < n), dtype=np.int64)
