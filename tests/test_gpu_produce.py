"""Producing the caches on the GPU (csa2_compress_kv) against the oracle's compressor (O14),
FP4 packing (O3/O4) and indexer-K projection (O15).

The compressed entries are floating point and are compared within a bound derived from their
arithmetic; the FP4 codes and scales, which floating point decides, are compared bit for bit with
the oracle's packing of the kernel's own fp32 entries (both sides decide in fp32); the indexer
keys are compared with the oracle's exact projection of those entries within half a bf16 unit in
the last place plus the fp32 accumulation bound."""
import numpy as np
import pytest
import torch

import fp4_kv_cache_e2m1_amd as P
from fp4_kv_cache_e2m1_amd import workloads as W
from oracle import csa2_oracle as O
from parity_util import dev_bf16, f64

pytestmark = pytest.mark.gpu

ENTRY_RTOL = 4e-6      # |e - e_ref| <= ENTRY_RTOL * sum_i w_i |c_i|: exp, fma and divide in fp32
KEY_ACC = 4e-5         # fp32 accumulation of 512 exact products, relative to sum |x w|


def _sync_np(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _check_entries(e_gpu, c, z, ratio, what):
    ref = O.compress_kv(c, z, ratio).astype(np.float64)
    mag = O.compress_kv(np.abs(c), z, ratio).astype(np.float64)
    err = np.abs(e_gpu.astype(np.float64) - ref)
    bad = err > ENTRY_RTOL * mag + 1e-37
    assert not bad.any(), f"{what}: {bad.sum()} entries out of tolerance, worst {err.max():.3g}"


def _check_keys(k_gpu, e_gpu, w_bits, Hk, Di, what):
    w = f64(w_bits)
    y = O.project_index_k(e_gpu, w, Hk, Di, rounded=False).reshape(len(e_gpu), -1)
    xb = O.round_bf16(e_gpu.astype(np.float64))
    absdot = np.abs(xb) @ np.abs(w).T
    kg = f64(k_gpu).reshape(len(e_gpu), -1)
    err = np.abs(kg - y)
    bad = err > 2.0 ** -8 * np.abs(y) + KEY_ACC * absdot
    assert not bad.any(), f"{what}: {bad.sum()} keys out of tolerance"
    # and nearly always the oracle's own rounding of the exact sum
    same = np.mean(kg == O.project_index_k(e_gpu, w, Hk, Di).reshape(len(e_gpu), -1))
    assert same > 0.99, f"{what}: only {same:.4f} of the keys equal the oracle's rounding"


def _run(B, n_tok, ratio, n_max, entry0, Hk, Di, seed, project=True):
    wl = W.CONFIGS[3].scaled(B=B, Hk=Hk, Di=Di, Hi=Hk)
    toks = [W.token_kv(wl, b, n_tok, first=seed) for b in range(B)]
    cb = np.stack([t[0] for t in toks])
    zb = np.stack([t[1] for t in toks])
    w_bits = W.w_index_k(wl)
    rows = torch.full((B, n_max, 288), 0xA5, dtype=torch.uint8, device="cuda")
    kidx = torch.full((B, n_max, Hk, Di), 7.0, dtype=torch.bfloat16, device="cuda") if project else None
    e0 = torch.tensor(entry0, dtype=torch.int32, device="cuda")
    ent = P.compress_kv(dev_bf16(cb), dev_bf16(zb), ratio, e0, rows, w_t=dev_bf16(w_bits) if project else None,
                        k_idx=kidx, return_entries=True)
    return cb, zb, w_bits, _sync_np(rows), (_sync_np(kidx.view(torch.int16)).view(np.uint16) if project else None), \
        _sync_np(ent)


@pytest.mark.parametrize("B,n_tok,ratio,n_max,entry0,Hk,Di", [
    (3, 4 * 37, 4, 200, [0, 50, 170], 8, 64),          # ragged tail, third sequence runs past n_max
    (2, 2 * 70, 2, 100, [10, 30], 1, 128),             # the shared 128-channel key
    (1, 8 * 9, 8, 12, [3], 4, 64),                     # 256 key channels
    (4, 33, 1, 40, [0, 7, 5, 2], 8, 64),               # ratio 1: the entry is the token
    (2, 4 * 5, 4, 8, [-2, 6], 8, 64),                  # entries before 0 or past n_max are skipped
    (2, 4 * 300, 4, 700, [0, 450], 1, 128),            # many entries (32-entry workgroups), ragged
    (3, 2 * 250, 2, 300, [5, 0, 60], 8, 64),           # many entries, 512 key channels
    (1, 4 * 1500, 4, 1600, [0], 8, 64),                # 16-entry workgroups, ragged last one
    (2, 4 * 1300, 4, 1400, [0, 200], 8, 64)])          # 32-entry workgroups, past n_max
def test_compress_kv(B, n_tok, ratio, n_max, entry0, Hk, Di):
    cb, zb, w_bits, rows, kidx, ent = _run(B, n_tok, ratio, n_max, entry0, Hk, Di, seed=n_tok + ratio)
    n_new = n_tok // ratio
    for b in range(B):
        c, z = f64(cb[b]), f64(zb[b])
        what = f"B={B} ratio={ratio} b={b}"
        if ratio == 1:
            assert np.array_equal(ent[b], c.astype(np.float32)), what
        _check_entries(ent[b], c, z, ratio, what)
        lo, hi = max(0, entry0[b]), min(n_max, entry0[b] + n_new)
        js = np.arange(lo - entry0[b], hi - entry0[b])
        if len(js):
            assert np.array_equal(rows[b, lo:hi], O.quantize_kv_fp4(ent[b][js])), f"{what}: FP4 rows differ"
            _check_keys(kidx[b, lo:hi], ent[b][js], w_bits, Hk, Di, what)
        untouched = np.ones(n_max, bool)
        untouched[lo:hi] = False
        assert np.all(rows[b, untouched] == 0xA5), f"{what}: rows outside the new entries changed"
        assert np.all(kidx[b, untouched] == 0x40E0), f"{what}: keys outside the new entries changed"


def test_compress_kv_without_projection():
    cb, zb, _, rows, _, ent = _run(2, 64, 4, 16, [0, 0], 8, 64, seed=3, project=False)
    for b in range(2):
        assert np.array_equal(rows[b], O.quantize_kv_fp4(ent[b]))
        _check_entries(ent[b], f64(cb[b]), f64(zb[b]), 4, f"no projection b={b}")


@pytest.mark.parametrize("B,n_tok,n_max,first", [(16, 4, 65536, 65535), (1, 4096, 33792, 32768)])
def test_compress_kv_full_size(B, n_tok, n_max, first):
    """The decode step of the 16 x 65536 stack (each sequence appends the entry of its last 4
    tokens) and the 4096-token prefill chunk (1024 entries appended after 32768)."""
    cb, zb, w_bits, rows, kidx, ent = _run(B, n_tok, 4, n_max, [first] * B, 8, 64, seed=first)
    for b in range(B):
        n_new = n_tok // 4
        _check_entries(ent[b], f64(cb[b]), f64(zb[b]), 4, f"full size b={b}")
        assert np.array_equal(rows[b, first:first + n_new], O.quantize_kv_fp4(ent[b]))
        _check_keys(kidx[b, first:first + n_new], ent[b], w_bits, 8, 64, f"full size b={b}")


@pytest.mark.parametrize("cfg", [3, 5])
def test_full_layer_produces_its_caches(cfg):
    """A Full layer that first compresses its own new tokens into the shared caches (csa2_layer_step
    with new tokens) at full size: the 16 x 65536 decode stack's first layer, each sequence
    appending the entry of its last 4 tokens at 65535, and the 4096-token prefill chunk appending
    1024 entries after 32768. The new rows and keys are checked as above; then, for sampled
    sequences and query rows, the layer's Top-K against the oracle's selection over the same
    caches (identical, or near-tie swaps only) and its attention against the oracle."""
    from parity_util import check_attn, compare_topk, k_idx_device, kv_rows_device, q_device
    wl = W.CONFIGS[cfg]
    if wl.T == 1:
        first, n_tok, bs, tr = wl.N - 1, 4, [0, 7, 15], np.array([0])
    else:
        first, n_tok, bs, tr = wl.n_existing, wl.T, [0], np.array([0, 1, 2, 3, 1000, 2047, 3001, 4095])
    n_new = n_tok // 4
    rows, kidx = kv_rows_device(wl), k_idx_device(wl)
    toks = [W.token_kv(wl, b, n_tok, first=4 * first) for b in range(wl.B)]
    cb, zb = np.stack([t[0] for t in toks]), np.stack([t[1] for t in toks])
    w_bits = W.w_index_k(wl)
    c_d, z_d, w_d = dev_bf16(cb), dev_bf16(zb), dev_bf16(w_bits)
    e0 = torch.full((wl.B,), first, dtype=torch.int32, device="cuda")
    # the kernel's fp32 entries (same kernel, written to a scratch cache)
    scratch = torch.empty(wl.B, first + n_new, 288, dtype=torch.uint8, device="cuda")
    ent = _sync_np(P.compress_kv(c_d, z_d, 4, e0, scratch, return_entries=True))
    n_vis = None
    if wl.T > 1:
        n_vis = P.prefill_n_vis([wl.p0] * wl.B, wl.T, wl.ratio, "cuda", n_max=wl.N)
    kv = P.KVState(rows, kidx, n_vis)
    idx = P.IdxState.empty(wl.B * wl.T, wl.k, "cuda")
    out, lse = P.layer_step(P.FULL, q_device(wl, 0, "q"), kv, idx, q_idx=q_device(wl, 0, "q_idx"),
                            produce=(c_d, z_d, 4, e0, w_d))
    out, lse, topk = _sync_np(out), _sync_np(lse), _sync_np(idx.topk).reshape(wl.B, wl.T, wl.k)
    new_rows = _sync_np(rows[:, first:first + n_new])
    new_keys = _sync_np(kidx[:, first:first + n_new].contiguous().view(torch.int16)).view(np.uint16)
    for b in range(wl.B):
        _check_entries(ent[b], f64(cb[b]), f64(zb[b]), 4, f"layer b={b}")
        assert np.array_equal(new_rows[b], O.quantize_kv_fp4(ent[b])), f"b={b}: FP4 rows differ"
        _check_keys(new_keys[b], ent[b], w_bits, wl.Hk, wl.Di, f"layer b={b}")
    nv_all = np.full(wl.T, wl.N) if wl.T == 1 else np.minimum(O.prefill_n_vis(wl.p0, wl.T, wl.ratio), wl.N)
    for b in bs:
        seq = W.sequence(wl, b, layers=1)
        kq = f64(seq["k_idx"])
        kq[first:first + n_new] = f64(new_keys[b]).reshape(n_new, wl.Hk, wl.Di)
        qi, q = f64(seq["q_idx"][0])[tr], f64(seq["q"][0])[tr]
        nv = nv_all[tr]
        scores = O.index_scores(qi, kq, nv)
        ref = O.topk(scores, wl.k, n_valid=nv)
        for i, t in enumerate(tr):
            compare_topk(topk[b, t], ref[i], lambda p: scores[i, p], f"cfg{cfg} b={b} t={t}")
        sel = topk[b, tr]
        need = np.unique(sel[sel >= 0])
        old, new = need[need < first], need[need >= first]
        packed = np.concatenate([O.quantize_kv_fp4(seq["kv_src"][old]), new_rows[b][new - first]])
        remap = np.full(wl.N, -1, np.int64)
        remap[np.concatenate([old, new])] = np.arange(len(need))
        local = np.where(sel >= 0, remap[np.maximum(sel, 0)], -1)
        o_ref, l_ref = O.sparse_attn(q, O.dequant_kv_fp4(packed), local, wl.sm_scale)
        check_attn(out.reshape(wl.B, wl.T, wl.H, -1)[b, tr], o_ref, lse.reshape(wl.B, wl.T, wl.H)[b, tr], l_ref,
                   f"cfg{cfg} b={b}")
