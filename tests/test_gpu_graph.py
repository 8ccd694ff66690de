"""A CSA2 layer step captured into a HIP graph replays bit-identically to the eager call.

Every kernel of a layer step is enqueued on the caller's stream, so the captured graph is a chain
of kernel nodes. Several replays run, with eager work on the outputs and synchronizations between
them, and every replay is compared with the eager result.
"""
import numpy as np
import pytest
import torch

import fp4_kv_cache_e2m1_amd as P
from fp4_kv_cache_e2m1_amd import workloads as W
from parity_util import k_idx_device, kv_rows_device, q_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("pool,pool_blocks", [(False, 0), (True, 64), (True, 256)])
def test_layer_step_graph_replay(pool, pool_blocks):
    wl = W.CONFIGS[4 if pool else 3].scaled(B=4, N=3000, k=128, pool_blocks=pool_blocks)
    rows, kidx = kv_rows_device(wl), k_idx_device(wl)
    q0, qi0 = q_device(wl, 0, "q"), q_device(wl, 0, "q_idx")
    q1, qi1 = q_device(wl, 1, "q"), q_device(wl, 1, "q_idx")
    kv = P.KVState(rows, kidx)
    idx = P.IdxState.empty(wl.B, wl.k, "cuda", pool_size=wl.pool_blocks * 8)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    out0 = torch.empty(wl.B, 1, wl.H, wl.D, device="cuda")
    out1 = torch.empty_like(out0)

    def step():
        P.layer_step(P.FULL, q0, kv, idx, q_idx=qi0, use_pool=pool, pool_blocks=wl.pool_blocks,
                     with_lse=False, ws=ws, out=out0)
        P.layer_step(P.REINDEX, q1, kv, idx, q_idx=qi1, use_pool=pool, with_lse=False, ws=ws, out=out1)

    step()
    torch.cuda.synchronize()
    ref0, ref1, ref_t = out0.clone(), out1.clone(), idx.topk.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        out0.fill_(float("nan"))
        out1.fill_(float("nan"))
        idx.topk.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out0, ref0) and torch.equal(out1, ref1), f"replay {rep} differs"
        assert torch.equal(idx.topk, ref_t), f"replay {rep}: Top-K differs"
