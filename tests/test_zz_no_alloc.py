"""csa2_layer_step_noalloc (scratch in the library's fixed device array) against csa2_layer_step
(scratch in a caller workspace): the same kernels, so every output, log-sum-exp and Top-K must be
bit-identical. Two schedules run with the no-allocation entry point back to back, the second with
a smaller input, so the second call finds the first call's contents in the scratch."""
import pytest
import torch

import fp4_kv_cache_e2m1_amd as P
from fp4_kv_cache_e2m1_amd import workloads as W
from parity_util import k_idx_device, kv_rows_device, q_device

pytestmark = pytest.mark.gpu


def _inputs(wl):
    nl = len(wl.modes)
    return (kv_rows_device(wl), k_idx_device(wl), [q_device(wl, l, "q") for l in range(nl)],
            [q_device(wl, l, "q_idx") for l in range(nl)])


def _schedule(wl, inp, no_alloc):
    rows, kidx, q, qi = inp
    use_pool = wl.pool_blocks > 0
    kv = P.KVState(rows, kidx)
    idx = P.IdxState.empty(wl.B * wl.T, wl.k, "cuda", pool_size=wl.pool_blocks * wl.block)
    res = []
    for l, mode in enumerate(wl.modes):
        out, lse = P.layer_step(mode, q[l], kv, idx, q_idx=qi[l] if mode != P.REUSE else None, use_pool=use_pool,
                                pool_blocks=wl.pool_blocks if use_pool else 0, no_alloc=no_alloc)
        res.append((out, lse, idx.topk.clone(), None if idx.pool is None else idx.pool.clone()))
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("cfg,big,small", [
    (3, dict(B=4, N=3000, k=128), dict(B=2, N=1000, k=64)),
    (4, dict(B=4, N=4000, k=128, pool_blocks=64), dict(B=2, N=1500, k=64, pool_blocks=16)),
    (2, dict(B=32, N=16384, k=512), dict(B=3, N=700, k=100))])
def test_noalloc_matches_layer_step(cfg, big, small):
    wls = [W.CONFIGS[cfg].scaled(**big), W.CONFIGS[cfg].scaled(**small)]
    inps = [_inputs(wl) for wl in wls]
    print(f"[noalloc] cfg {cfg}: {big} then {small}", flush=True)
    refs = [_schedule(wl, inp, no_alloc=False) for wl, inp in zip(wls, inps)]
    got = [_schedule(wl, inp, no_alloc=True) for wl, inp in zip(wls, inps)]   # two calls in a row
    for wl, r, g in zip(wls, refs, got):
        for l, (ra, ga) in enumerate(zip(r, g)):
            what = f"{wl.name} B={wl.B} N={wl.N} layer {l}"
            assert torch.equal(ga[0], ra[0]), f"{what}: output differs"
            assert torch.equal(ga[1], ra[1]), f"{what}: lse differs"
            assert torch.equal(ga[2], ra[2]), f"{what}: Top-K differs"
            if ra[3] is not None:
                assert torch.equal(ga[3], ra[3]), f"{what}: pool differs"
