"""The decode step (index_decode, topk_select, sparse_attn_decode) captured
in a HIP graph: the library allocates, clears and synchronises nothing
inside those calls, so the step can be recorded once and replayed.  Every
replay, with eager work and synchronisations of the program in between, must
equal the eager step bit for bit."""
import numpy as np
import pytest
import torch

import token_level_sparse_lightning_amd as tl
from token_level_sparse_lightning_amd import synth
from tests.gpu_util import DEV, announce

pytestmark = pytest.mark.gpu


def test_decode_step_graph_replays_equal_eager():
    B, HI, DI, H, Dqk, Dv, k = 6, 64, 128, 128, 576, 512, 256
    lengths = np.array([700, 0, 3000, 257, 1500, 64], dtype=np.int64)
    di = synth.indexer_decode(lengths, HI, DI, synth.DT_FP8, seed=21, device=DEV)
    qa, kva = synth.attn_decode(lengths, H, Dqk, synth.DT_BF16, seed=21, device=DEV)
    cu = di.cu_seqlens
    row_start = cu[:-1].contiguous()
    row_len = torch.as_tensor(lengths, dtype=torch.int32, device=DEV)
    max_len = int(lengths.max())
    scores = torch.empty(int(lengths.sum()), dtype=torch.float32, device=DEV)
    S = torch.empty((B, k), dtype=torch.int32, device=DEV)
    out = torch.empty((B, H, Dv), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, H), dtype=torch.float32, device=DEV)
    ws = torch.empty(tl.sparse_attn_decode_workspace_bytes(qa, kva, S, Dv), dtype=torch.uint8, device=DEV)
    tws = torch.empty(tl.topk_select_workspace_bytes(B, k, max_len), dtype=torch.uint8, device=DEV)

    def step():
        tl.index_decode(di.q, di.k, di.w, cu, max_len, q_scale=di.q_scale, k_scale=di.k_scale, scores=scores)
        tl.topk_select(scores, row_start, row_len, k, max_len, S=S, workspace=tws)
        tl.sparse_attn_decode(qa, kva, cu, S, 1 / 24.0, Dv, out=out, lse=lse, workspace=ws)

    announce("decode step, eager")
    step()
    torch.cuda.synchronize()
    ref = [x.clone() for x in (scores, S, out, lse)]

    announce("decode step, capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep in range(4):
        # eager work of the program between replays: clobber every output
        scores.fill_(float("nan"))
        S.fill_(-7)
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        announce(f"decode step, replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("scores", "S", "out", "lse"), (scores, S, out, lse), ref):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from the eager step"
