"""GPU parity of each HIP kernel against the CPU oracle (small and ragged shapes, edge cases).

Bars: FP4 pack/unpack and Top-K / pool index sets bit-exact; indexer scores within 1e-3 of
max(|s|, sum |q*k|); attention max-abs error within 2e-3 of the output row's L2 norm.
"""
import numpy as np
import pytest
import torch

import fp4_kv_cache_e2m1_amd as P
from fp4_kv_cache_e2m1_amd import workloads as W
from oracle import csa2_oracle as O
from parity_util import check_attn, check_scores, dev_bf16, f64, k_idx_device, kv_rows_device, q_device

pytestmark = pytest.mark.gpu


def _sync_np(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _codec_inputs(rows, dim, seed):
    g = np.random.default_rng(seed)
    x = g.standard_normal((rows, dim)).astype(np.float32)
    x *= (10.0 ** g.uniform(-7, 4, size=(rows, dim // 16, 1))).repeat(16, axis=2).reshape(rows, dim).astype(np.float32)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.75, -5.0, 7.0, -0.0, 0.0], np.float32)
    if rows >= 3:
        x[0] = 0.0
        x[1] = -0.0
        x[2, :16] = 6.0
        x[2, 1:1 + len(ties)] = ties                     # every E2M1 tie at scale 1.0
        x[2, 16:32] = 1e30                                # saturates at 448 x 6
        x[2, 32:48] = 3.0 * 2.0 ** -10                    # amax/6 exactly half the smallest subnormal
    return x


@pytest.mark.parametrize("dim,rows", [(512, 1), (512, 5), (512, 1001), (64, 7), (128, 33), (1024, 9)])
@pytest.mark.parametrize("bf16", [False, True])
def test_quantize_bitexact(dim, rows, bf16):
    x = _codec_inputs(rows, dim, seed=dim * 7 + rows)
    if bf16:
        src = torch.from_numpy(x).to(torch.bfloat16)
        ref_in = src.to(torch.float32).numpy()
    else:
        src = torch.from_numpy(x)
        ref_in = x
    got = _sync_np(P.quantize_kv_fp4(src.cuda()))
    want = O.quantize_kv_fp4(ref_in)
    assert got.shape == want.shape == (rows, dim // 2 + dim // 16)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} bytes differ, first {bad[:5].tolist()}"


def test_quantize_empty():
    out = P.quantize_kv_fp4(torch.empty(0, 512, device="cuda"))
    torch.cuda.synchronize()
    assert out.shape == (0, 288)


def test_dequant_exhaustive_codes_and_scales():
    # 8 rows x 32 groups cover every scale byte 0..255; each group holds all 16 value codes
    rows = np.zeros((8, 288), np.uint8)
    for r in range(8):
        for g in range(32):
            rows[r, 256 + g] = (32 * r + g) % 256
            for c in range(16):
                ch = 16 * g + c
                rows[r, ch // 2] |= np.uint8(c << (4 * (ch % 2)))
    got = _sync_np(P.dequant_kv_fp4(torch.from_numpy(rows).cuda()))
    want = O.dequant_kv_fp4(rows).astype(np.float32)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))


def test_roundtrip_on_normal_data():
    x = np.random.default_rng(1).standard_normal((300, 512)).astype(np.float32)
    rows = P.quantize_kv_fp4(torch.from_numpy(x).cuda())
    deq = _sync_np(P.dequant_kv_fp4(rows))
    assert np.array_equal(deq, O.dequant_kv_fp4(O.quantize_kv_fp4(x)).astype(np.float32))


# ---------------------------------------------------------------------------------------------
def _abs_dot(q, k):
    """sum_h sum_d |q||k| for every (row, entry): the scale of the dot product's rounding error."""
    R, Hi, Di = q.shape
    N, Hk, _ = k.shape
    kk = np.repeat(k, Hi, axis=1) if Hk == 1 else k
    return np.abs(q.reshape(R, -1)) @ np.abs(kk.reshape(N, -1)).T


@pytest.mark.parametrize("B,N,Hi,Hk,Di", [(3, 1000, 8, 8, 64), (2, 777, 4, 4, 64), (2, 513, 8, 1, 64),
                                          (1, 300, 16, 16, 64), (2, 64, 2, 2, 64), (1, 1, 8, 8, 64),
                                          (2, 2049, 8, 8, 128)])
def test_index_scores_decode(B, N, Hi, Hk, Di):
    if Hi * Di > 1024:
        pytest.skip("shape outside the streaming kernel")
    g = np.random.default_rng(N + Hi)
    qb = W.to_bf16_bits(g.standard_normal((B, 1, Hi, Di)).astype(np.float32))
    kb = W.to_bf16_bits(g.standard_normal((B, N, Hk, Di)).astype(np.float32))
    n_vis = np.array([N, max(1, N // 2), 3][:B], dtype=np.int32) if B > 1 else np.array([N], np.int32)
    s, bm = P.index_scores(dev_bf16(qb), dev_bf16(kb), n_vis=torch.from_numpy(n_vis).cuda(), block_max=True)
    s, bm = _sync_np(s), _sync_np(bm)
    for b in range(B):
        ref = O.index_scores(f64(qb[b]), f64(kb[b]), [n_vis[b]])[0]
        mask = np.arange(N) < n_vis[b]
        check_scores(s[b], ref, _abs_dot(f64(qb[b]), f64(kb[b]))[0], mask, f"b={b}")
        # the fused block max is the max of the kernel's own scores over visible block members
        nb = -(-int(n_vis[b]) // 8)
        own = O.block_max(s[b:b + 1], [n_vis[b]])[0][:nb]
        assert np.array_equal(bm[b, :nb], own)


@pytest.mark.parametrize("B,N,Hi,Di", [(3, 50000, 8, 64), (1, 40000, 4, 128), (5, 33000, 8, 128), (200, 9000, 8, 64),
                                       (100, 12345, 8, 64)])
def test_index_scores_decode_one_workgroup_per_cu(B, N, Hi, Di):
    """Flat decode scoring of 1 KiB and 2 KiB key rows at sizes that run one workgroup per CU (a few
    rows split into up to 256 tiles whose last one is ragged, one tile per row at 200 rows, two at
    100), with ragged visible counts (full, half, 3, 0 and scattered) and the fused block max."""
    g = np.random.default_rng(B * N + Di)
    qb = W.to_bf16_bits(g.standard_normal((B, 1, Hi, Di)).astype(np.float32))
    kb = W.to_bf16_bits(g.standard_normal((B, N, Hi, Di)).astype(np.float32))
    n_vis = np.array([N, N // 2, 3, 0] + [int(x) for x in g.integers(1, N + 1, size=max(0, B - 4))],
                     np.int32)[:B]
    s, bm = P.index_scores(dev_bf16(qb), dev_bf16(kb), n_vis=torch.from_numpy(n_vis).cuda(), block_max=True)
    s, bm = _sync_np(s), _sync_np(bm)
    for b in range(B):
        nvb = int(n_vis[b])
        if nvb == 0:
            continue
        ref = O.index_scores(f64(qb[b]), f64(kb[b, :nvb]), [nvb])[0]
        check_scores(s[b, :nvb], ref, _abs_dot(f64(qb[b]), f64(kb[b, :nvb]))[0], np.ones(nvb, bool), f"b={b}")
        nb = -(-nvb // 8)
        assert np.array_equal(bm[b, :nb], O.block_max(s[b:b + 1], [nvb])[0][:nb]), f"block max b={b}"


def test_index_scores_pool():
    g = np.random.default_rng(5)
    B, N, P_ = 3, 5000, 96
    qb = W.to_bf16_bits(g.standard_normal((B, 1, 8, 64)).astype(np.float32))
    kb = W.to_bf16_bits(g.standard_normal((B, N, 8, 64)).astype(np.float32))
    pool = np.full((B, P_), -1, np.int32)
    for b in range(B):
        blocks = np.sort(g.choice(N // 8, size=10, replace=False))
        pos = (blocks[:, None] * 8 + np.arange(8)).reshape(-1)[: P_ - 7 * b]
        pool[b, : len(pos)] = pos
    pool[2, -1] = N + 5                                   # out of range: treated as empty
    s = _sync_np(P.index_scores(dev_bf16(qb), dev_bf16(kb), cand=torch.from_numpy(pool).cuda()))
    for b in range(B):
        clean = np.where((pool[b] >= 0) & (pool[b] < N), pool[b], -1)
        ref = O.pool_scores(f64(qb[b]), f64(kb[b]), clean[None])[0]
        valid = clean >= 0
        assert np.all(np.isneginf(s[b][~valid]))
        ad = _abs_dot(f64(qb[b]), f64(kb[b]))[0]
        check_scores(s[b][valid], ref[valid], ad[clean[valid]], np.ones(valid.sum(), bool), f"pool b={b}")


@pytest.mark.parametrize("B,T,N,p0,ratio,Hi", [
    (1, 200, 700, 2500, 4, 8), (2, 64, 130, 0, 1, 8), (1, 300, 5000, 19000, 4, 8),
    (1, 520, 3000, 9000, 4, 4),      # 256 channels, three query slabs, ragged
    (2, 100, 900, 400, 4, 2),        # 128 channels: tiled form
    (1, 260, 1200, 2000, 4, 6)])     # 384 channels: tiled form, ragged
def test_index_scores_prefill_mfma(B, T, N, p0, ratio, Hi):
    g = np.random.default_rng(T + N + Hi)
    qb = W.to_bf16_bits(g.standard_normal((B, T, Hi, 64)).astype(np.float32))
    kb = W.to_bf16_bits(g.standard_normal((B, N, Hi, 64)).astype(np.float32))
    nv = P.prefill_n_vis(p0, T, ratio, "cuda")
    nv_ref = O.prefill_n_vis(p0, T, ratio)
    assert np.array_equal(nv.cpu().numpy(), nv_ref)
    nv_all = torch.cat([torch.clamp(nv, max=N)] * B)
    out = torch.full((B * T, N), float("nan"), device="cuda")
    s = _sync_np(P.index_scores(dev_bf16(qb), dev_bf16(kb), n_vis=nv_all, out=out))
    for b in range(B):
        nvb = np.minimum(nv_ref, N)
        ref = O.index_scores(f64(qb[b]), f64(kb[b]), nvb)
        mask = np.arange(N)[None, :] < nvb[:, None]
        check_scores(s[b * T:(b + 1) * T], ref, _abs_dot(f64(qb[b]), f64(kb[b])), mask, f"prefill b={b}")
        assert np.all(np.isnan(s[b * T:(b + 1) * T][~mask])), "slots past n_vis must stay unwritten"


def test_prefill_visibility_per_sequence():
    """csa2_prefill_visibility with a start position per sequence, capped at n_max, against the
    oracle's rule (reading R-6) sequence by sequence: positions before, across and past the cap."""
    starts, T, ratio, n_max = [0, 5, 131072, 400], 37, 4, 110
    nv = P.prefill_n_vis(starts, T, ratio, "cuda", n_max=n_max).cpu().numpy().reshape(len(starts), T)
    for b, p0 in enumerate(starts):
        assert np.array_equal(nv[b], np.minimum(O.prefill_n_vis(p0, T, ratio), n_max)), b


# ---------------------------------------------------------------------------------------------
TOPK_CASES = [(1, 1, 1), (3, 7, 3), (4, 100, 17), (2, 5000, 512), (32, 16384, 512), (2, 40000, 1024),
              (3, 100000, 512), (2, 262144, 512), (5, 300, 300), (2, 50, 64)]


@pytest.mark.parametrize("rows,n,k", TOPK_CASES)
@pytest.mark.parametrize("dist", ["normal", "ties", "signed_zero", "bounded"])
def test_topk_bitexact(rows, n, k, dist):
    s = W.random_scores(rows * 31 + k, rows, n, dist)
    nv = np.array([n - (r * 37) % max(1, n // 3) for r in range(rows)], np.int32)
    got = _sync_np(P.topk(torch.from_numpy(s).cuda(), k, n_valid=torch.from_numpy(nv).cuda()))
    want = O.topk(s, k, n_valid=nv)
    assert np.array_equal(got, want), f"rows differ: {np.where((got != want).any(1))[0][:5]}"


@pytest.mark.parametrize("n", [7000, 10000, 19000, 27000, 33792, 35000, 40960])
@pytest.mark.parametrize("dist", ["normal", "ties", "const", "signed_zero", "bounded"])
def test_topk_whole_rows_bitexact(n, dist):
    """Many rows (one workgroup per whole row, as in prefill) at row lengths that take each register
    count of that form (8, 12, 20, 28, 33, 36, 40 columns per lane), with ragged valid counts. Tied,
    constant and ±0 rows overflow the packed survivor list, and rows with few valid columns skip
    the pruning bound: both read the row again in this form."""
    rows, k = 260, 1024
    s = W.random_scores(n + 7, rows, n, dist)
    nv = np.array([n - (r * 131) % (n // 2) for r in range(rows)], np.int32)
    got = _sync_np(P.topk(torch.from_numpy(s).cuda(), k, n_valid=torch.from_numpy(nv).cuda()))
    want = O.topk(s, k, n_valid=nv)
    assert np.array_equal(got, want), f"rows differ: {np.where((got != want).any(1))[0][:5]}"


def test_topk_whole_rows_short_and_empty():
    """A many-row call whose rows hold 0 to ~2000 valid columns of 33792: empty rows, rows with
    fewer valid columns than k (no selection, everything taken) and rows just above k."""
    rows, n, k = 300, 33792, 1024
    s = W.random_scores(5, rows, n, "normal")
    nv = np.array([(r * 7) % 2100 for r in range(rows)], np.int32)
    got = _sync_np(P.topk(torch.from_numpy(s).cuda(), k, n_valid=torch.from_numpy(nv).cuda()))
    want = O.topk(s, k, n_valid=nv)
    assert np.array_equal(got, want), f"rows differ: {np.where((got != want).any(1))[0][:5]}"


def test_topk_const_rows_and_pool_columns():
    s = W.random_scores(3, 4, 3000, "const")
    got = _sync_np(P.topk(torch.from_numpy(s).cuda(), 100))
    assert np.array_equal(got, O.topk(s, 100))
    g = np.random.default_rng(0)
    s = W.random_scores(4, 4, 2048, "ties")
    pool = np.sort(g.choice(100000, size=(4, 2048), replace=False), axis=1).astype(np.int32)
    pool[:, 1900:] = -1
    got = _sync_np(P.topk(torch.from_numpy(s).cuda(), 256, col_to_pos=torch.from_numpy(pool).cuda()))
    assert np.array_equal(got, O.topk(s, 256, col_to_pos=pool))


@pytest.mark.parametrize("rows,n_pos,n_sel", [(2, 4003, 64), (4, 262144, 1024), (3, 800, 200), (1, 80, 16),
                                            (2, 262144, 2048), (3, 200000, 3000), (2, 131072, 4096)])
@pytest.mark.parametrize("dist", ["normal", "ties", "bounded"])
def test_hier_pool_bitexact(rows, n_pos, n_sel, dist):
    s = W.random_scores(n_pos + n_sel, rows, n_pos, dist)
    n_vis = np.array([n_pos - 13 * r for r in range(rows)], np.int32)
    bm_ref = O.block_max(s, n_vis)
    bm = torch.from_numpy(np.where(np.isneginf(bm_ref), np.float32(0), bm_ref)).cuda()
    got = _sync_np(P.hier_pool(bm, n_sel, n_vis=torch.from_numpy(n_vis).cuda()))
    want = O.hier_pool(bm_ref, n_vis, n_sel)
    assert np.array_equal(got, want)


# ---------------------------------------------------------------------------------------------
def _attn_case(B, T, H, N, K, seed, neg_frac=0.1, oob=False):
    g = np.random.default_rng(seed)
    src = g.standard_normal((B, N, 512)).astype(np.float32)
    rows = np.stack([O.quantize_kv_fp4(src[b]) for b in range(B)])
    qb = W.to_bf16_bits(g.standard_normal((B, T, H, 512)).astype(np.float32))
    idx = np.stack([[g.choice(N, size=K, replace=K > N) for _ in range(T)] for _ in range(B)]).astype(np.int32)
    idx[g.random(idx.shape) < neg_frac] = -1
    if oob:
        m = min(3, K)
        idx[0, 0, :m] = N + np.arange(m)
    return rows, qb, idx


def _attn_ref(rows, qb, idx, scale):
    B, T = idx.shape[:2]
    N = rows.shape[1]
    outs, lses = [], []
    for b in range(B):
        clean = np.where((idx[b] >= 0) & (idx[b] < N), idx[b], -1)
        o, l = O.sparse_attn(f64(qb[b]), O.dequant_kv_fp4(rows[b]), clean, scale)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


@pytest.mark.parametrize("B,T,H,N,K", [(2, 1, 64, 300, 512), (3, 1, 64, 1000, 100), (1, 3, 16, 200, 33),
                                       (2, 2, 32, 90, 64), (1, 1, 128, 500, 256), (1, 1, 48, 70, 31),
                                       (4, 1, 64, 2000, 1), (1, 40, 64, 600, 96), (1, 600, 64, 300, 70),
                                       (2, 1, 16, 5000, 1024), (1, 1, 64, 3000, 2048)])
def test_sparse_attn(B, T, H, N, K):
    rows, qb, idx = _attn_case(B, T, H, N, K, seed=B * 1000 + N + K, oob=True)
    scale = 1 / np.sqrt(512)
    out, lse = P.sparse_attn(dev_bf16(qb), torch.from_numpy(rows).cuda(), torch.from_numpy(idx).cuda(), scale)
    out, lse = _sync_np(out), _sync_np(lse)
    ref, lref = _attn_ref(rows, qb, idx, scale)
    check_attn(out, ref, lse, lref, f"attn B={B} T={T} H={H} K={K}")


@pytest.mark.parametrize("B,T,H,N,K,qmul", [(1, 512, 64, 1500, 1024, 1.0), (2, 300, 128, 400, 77, 1.0),
                                             (1, 520, 64, 90, 33, 16.0), (1, 530, 32, 200, 40, 1.0)])
def test_sparse_attn_many_rows(B, T, H, N, K, qmul):
    """Launches with >= 512 query rows: the 64-head prefill form (H % 64 == 0, K <= 1024) and the
    older wide form (H = 32). Checked against the oracle on a seeded sample of query rows (all
    heads), including a row whose selection is empty; qmul = 16 widens the score range so the
    lazy softmax rescale fires."""
    rows, qb, idx = _attn_case(B, T, H, N, K, seed=7 * T + K, oob=True)
    if qmul != 1.0:
        qb = W.to_bf16_bits(W.bf16_bits_to_f32(qb) * np.float32(qmul))
    idx[0, 1, :] = -1
    scale = 1 / np.sqrt(512)
    out, lse = P.sparse_attn(dev_bf16(qb), torch.from_numpy(rows).cuda(), torch.from_numpy(idx).cuda(), scale)
    out, lse = _sync_np(out), _sync_np(lse)
    g = np.random.default_rng(T + K)
    ts = np.unique(np.concatenate([[0, 1, T - 1], g.choice(T, size=6, replace=False)]))
    ref, lref = _attn_ref(rows, qb[:, ts], idx[:, ts], scale)
    check_attn(out[:, ts], ref, lse[:, ts], lref, f"attn B={B} T={T} H={H} K={K} qmul={qmul}")
    assert np.all(out[0, 1] == 0) and np.all(np.isneginf(lse[0, 1]))


def test_sparse_attn_full_selection_and_empty():
    rows, qb, _ = _attn_case(1, 2, 64, 128, 1, seed=3)
    scale = 0.07
    idx = np.stack([np.arange(128, dtype=np.int32), np.full(128, -1, np.int32)])[None]
    out, lse = P.sparse_attn(dev_bf16(qb), torch.from_numpy(rows).cuda(), torch.from_numpy(idx).cuda(), scale)
    out, lse = _sync_np(out), _sync_np(lse)
    ref, lref = _attn_ref(rows, qb, idx, scale)
    check_attn(out, ref, lse, lref, "full / empty")
    assert np.all(out[0, 1] == 0) and np.all(np.isneginf(lse[0, 1]))


def test_sparse_attn_single_entry_is_exact():
    rows, qb, _ = _attn_case(1, 1, 16, 50, 1, seed=4)
    idx = np.array([[[-1, 17, -1]]], np.int32)
    out, _ = P.sparse_attn(dev_bf16(qb), torch.from_numpy(rows).cuda(), torch.from_numpy(idx).cuda(), 0.1)
    out = _sync_np(out)
    x = O.dequant_kv_fp4(rows[0, 17:18])[0].astype(np.float32)
    assert np.array_equal(out[0, 0], np.broadcast_to(x, (16, 512)))


def test_determinism():
    rows, qb, idx = _attn_case(2, 1, 64, 400, 512, seed=9)
    args = (dev_bf16(qb), torch.from_numpy(rows).cuda(), torch.from_numpy(idx).cuda(), 0.05)
    a, la = P.sparse_attn(*args)
    b, lb = P.sparse_attn(*args)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)
    s = torch.from_numpy(W.random_scores(1, 8, 70000, "ties")).cuda()
    assert torch.equal(P.topk(s, 512), P.topk(s, 512))


def test_determinism_indexer_pool_and_layer():
    """Repeated calls give bit-identical results: decode and prefill indexer scores, the fused
    block maxima, the candidate pool, and a whole hierarchical Full layer followed by a Reindex
    layer (scores, Top-K, pool, attention output and log-sum-exp)."""
    g = np.random.default_rng(17)
    qd = dev_bf16(W.to_bf16_bits(g.standard_normal((3, 1, 8, 64)).astype(np.float32)))
    kd = dev_bf16(W.to_bf16_bits(g.standard_normal((3, 5000, 8, 64)).astype(np.float32)))
    s1, b1 = P.index_scores(qd, kd, block_max=True)
    s2, b2 = P.index_scores(qd, kd, block_max=True)
    assert torch.equal(s1, s2) and torch.equal(b1, b2)
    qp = dev_bf16(W.to_bf16_bits(g.standard_normal((1, 300, 8, 64)).astype(np.float32)))
    kp = dev_bf16(W.to_bf16_bits(g.standard_normal((1, 2000, 8, 64)).astype(np.float32)))
    nv = P.prefill_n_vis(6000, 300, 4, "cuda", n_max=2000)
    o1 = torch.zeros(300, 2000, device="cuda")
    o2 = torch.zeros(300, 2000, device="cuda")
    P.index_scores(qp, kp, n_vis=nv, out=o1)
    P.index_scores(qp, kp, n_vis=nv, out=o2)
    assert torch.equal(o1, o2)
    assert torch.equal(P.hier_pool(b1, 64), P.hier_pool(b1, 64))
    wl = W.CONFIGS[4].scaled(B=3, N=5000, k=200, pool_blocks=64)
    rows, kidx = kv_rows_device(wl), k_idx_device(wl)
    q = [q_device(wl, l, "q") for l in range(2)]
    qi = [q_device(wl, l, "q_idx") for l in range(2)]
    runs = []
    for _ in range(2):
        kv = P.KVState(rows, kidx)
        idx = P.IdxState.empty(wl.B, wl.k, "cuda", pool_size=wl.pool_blocks * 8)
        o0, l0 = P.layer_step(P.FULL, q[0], kv, idx, q_idx=qi[0], use_pool=True, pool_blocks=wl.pool_blocks)
        t0, p0 = idx.topk.clone(), idx.pool.clone()
        o1_, l1 = P.layer_step(P.REINDEX, q[1], kv, idx, q_idx=qi[1], use_pool=True)
        runs.append((o0, l0, t0, p0, o1_, l1, idx.topk.clone()))
    torch.cuda.synchronize()
    for a_, b_ in zip(*runs):
        assert torch.equal(a_, b_)


def test_split_merge_with_garbage_and_reused_workspace():
    """Rows split over several workgroups leave partial results in the workspace: a workspace of
    random bytes, reused for several calls of different shapes, must give the oracle's result
    every time."""
    g = torch.Generator().manual_seed(5)
    ws = torch.randint(0, 256, (64 << 20,), dtype=torch.uint8, generator=g).cuda()
    scale = 1 / np.sqrt(512)
    for B, K, seed in [(2, 512, 21), (2, 512, 22), (3, 300, 23), (1, 1024, 24), (2, 512, 25)]:
        rows, qb, idx = _attn_case(B, 1, 64, 1500, K, seed=seed)
        out, lse = P.sparse_attn(dev_bf16(qb), torch.from_numpy(rows).cuda(), torch.from_numpy(idx).cuda(), scale,
                                 ws=ws)
        out, lse = _sync_np(out), _sync_np(lse)
        ref, lref = _attn_ref(rows, qb, idx, scale)
        check_attn(out, ref, lse, lref, f"split merge B={B} K={K} seed={seed}")


# ---------------------------------------------------------------------------------------------
def _swa_case(B, H, N, K, Wn, n_win, seed, wide_exps=False):
    rows, qb, idx = _attn_case(B, 1, H, N, K, seed=seed, oob=K > 0)
    g = np.random.default_rng(seed + 1)
    src = g.standard_normal((B * Wn, 512)).astype(np.float32)
    if wide_exps:   # row magnitudes from 2^-24 to 2^14: row exponents across the whole range
        src *= np.ldexp(1.0, g.integers(-24, 15, size=(B * Wn, 1))).astype(np.float32)
    codes, exps = O.quantize_swa_fp8(src)
    return rows, qb[:, 0], idx[:, 0], codes.reshape(B, Wn, 512), exps.reshape(B, Wn), np.asarray(n_win, np.int32)


def _swa_ref(rows, qb, idx, codes, exps, n_win, scale):
    N = rows.shape[1]
    outs, lses = [], []
    for b in range(len(qb)):
        clean = np.where((idx[b] >= 0) & (idx[b] < N), idx[b], -1)
        win = O.dequant_swa_fp8(codes[b], exps[b])[None]
        o, l = O.sparse_attn_swa(f64(qb[b])[None], O.dequant_kv_fp4(rows[b]), clean[None], win,
                                 [min(max(int(n_win[b]), 0), codes.shape[1])], scale)
        outs.append(o[0])
        lses.append(l[0])
    return np.stack(outs), np.stack(lses)


def _swa_run(rows, qb, idx, codes, exps, n_win, scale, with_lse=True, ws=None):
    out, lse = P.sparse_attn_swa(dev_bf16(qb), torch.from_numpy(rows).cuda(), torch.from_numpy(idx).cuda(),
                                 torch.from_numpy(codes).cuda(), torch.from_numpy(exps).cuda(),
                                 torch.from_numpy(n_win).cuda(), scale, with_lse=with_lse, ws=ws)
    return _sync_np(out), (_sync_np(lse) if lse is not None else None)


@pytest.mark.parametrize("B,H,N,K,Wn,n_win", [(3, 64, 1000, 100, 128, [128, 1, 77]),
                                              (2, 16, 200, 33, 64, [0, 50]),
                                              (2, 32, 10, 0, 128, [128, 5]),
                                              (32, 64, 800, 512, 128, list(range(0, 128, 4))),
                                              (4, 128, 600, 1024, 100, [100, 99, 31, 33]),
                                              (1, 48, 70, 31, 16, [200]),
                                              (600, 16, 40, 24, 64, [(7 * b) % 70 for b in range(600)])])
def test_sparse_attn_swa(B, H, N, K, Wn, n_win):
    """Selected FP4 entries joined with the FP8 window as one softmax, against the oracle: one- and
    several-chunk windows, a ragged last chunk, an empty window, no selected entries (K = 0), the
    split sparse path (B = 32, K = 512), n_win above the reserved rows (clamped), and 600
    sequences (beyond the plain sparse attention's decode-form limit)."""
    case = _swa_case(B, H, N, K, Wn, n_win, seed=B * 100 + K + Wn)
    scale = 1 / np.sqrt(512)
    out, lse = _swa_run(*case, scale)
    ref, lref = _swa_ref(*case, scale)
    check_attn(out, ref, lse, lref, f"swa B={B} H={H} K={K} W={Wn}")


def test_sparse_attn_swa_merge_extremes_and_empty():
    """Row exponents over their whole range, with sm_scale chosen so the largest logit is ~300: in
    sequence 0 the window dominates and the selected entries' merge weight underflows, in
    sequence 1 (large FP4 rows, window rows near 2^-24) the reverse; a sequence with nothing to
    attend (0, -inf); and the call without lse on a workspace of random bytes."""
    B, H, N, K, Wn = 4, 64, 300, 64, 128
    rows, qb, idx, codes, exps, _ = _swa_case(B, H, N, K, Wn, [0] * B, seed=77, wide_exps=True)
    g = np.random.default_rng(78)
    rows[1] = O.quantize_kv_fp4((400.0 * g.standard_normal((N, 512))).astype(np.float32))
    tiny = np.ldexp(g.standard_normal((Wn, 512)), -22).astype(np.float32)
    codes[1], exps[1] = O.quantize_swa_fp8(tiny)
    qb[1] = W.to_bf16_bits(W.bf16_bits_to_f32(qb[1]) * np.float32(64.0))
    idx[2, :] = -1
    n_win = np.array([128, 100, 0, 64], np.int32)
    qf = W.bf16_bits_to_f32(qb).astype(np.float64)
    big = 0.0
    for b in range(B):
        sel = idx[b][(idx[b] >= 0) & (idx[b] < N)]
        x = np.concatenate([O.dequant_kv_fp4(rows[b])[sel], O.dequant_swa_fp8(codes[b], exps[b])[:n_win[b]]])
        if len(x):
            big = max(big, float(np.abs(qf[b] @ x.T).max()))
    scale = 300.0 / big
    out, lse = _swa_run(rows, qb, idx, codes, exps, n_win, scale)
    ref, lref = _swa_ref(rows, qb, idx, codes, exps, n_win, scale)
    check_attn(out, ref, lse, lref, "swa extremes")
    assert np.all(out[2] == 0) and np.all(np.isneginf(lse[2]))
    gt = torch.Generator().manual_seed(11)
    ws = torch.randint(0, 256, (8 << 20,), dtype=torch.uint8, generator=gt).cuda()
    out2, none = _swa_run(rows, qb, idx, codes, exps, n_win, scale, with_lse=False, ws=ws)
    assert none is None and np.array_equal(out2, out)


def test_sparse_attn_swa_window_only_single_row_is_exact():
    """One window row and no selected entries: the output is that row's dequantized value."""
    rows, qb, idx, codes, exps, _ = _swa_case(1, 16, 20, 2, 8, [1], seed=5, wide_exps=True)
    idx[:] = -1
    out, lse = _swa_run(rows, qb, idx, codes, exps, np.array([1], np.int32), 0.1)
    x = O.dequant_swa_fp8(codes[0, :1], exps[0, :1])[0].astype(np.float32)
    assert np.array_equal(out[0], np.broadcast_to(x, (16, 512)))


# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("B,T,N,C,spread", [(3, 1, 1000, 512, 0), (2, 1, 777, 256, 0), (1, 1, 1, 512, 0),
                                            (32, 1, 1100, 512, 0), (2, 3, 2049, 256, 6), (2, 1, 20000, 512, 0),
                                            (1, 20, 3000, 512, 2), (2, 16, 1500, 256, 0)])
def test_index_scores_mxfp4(B, T, N, C, spread):
    """FP4 (MXFP4) indexer against the oracle on MXFP4 rows the oracle quantized: ragged tiles,
    one entry, several query rows per sequence with n_vis cutting tiles, block magnitudes spread
    over 2^-spread .. 2^spread (different scales per block), and long rows over many tiles.
    Slots past n_vis stay as they were."""
    g = np.random.default_rng(N + C + T)
    xq = g.standard_normal((B * T, C)).astype(np.float32)
    xk = g.standard_normal((B * N, C)).astype(np.float32)
    if spread:
        xq *= np.ldexp(1.0, g.integers(-spread, spread + 1, size=(B * T, C // 32))).repeat(32, 1).astype(np.float32)
        xk *= np.ldexp(1.0, g.integers(-spread, spread + 1, size=(B * N, C // 32))).repeat(32, 1).astype(np.float32)
    q_rows = O.quantize_mxfp4(xq).reshape(B, T, -1)
    k_rows = O.quantize_mxfp4(xk).reshape(B, N, -1)
    n_vis = np.array([[max(1, N - 7 * (b * T + t) - 300 * t) for t in range(T)] for b in range(B)], np.int32).reshape(-1)
    n_vis[0] = N
    out = torch.full((B * T, N), 7.0, dtype=torch.float32).cuda()
    s = _sync_np(P.index_scores_mxfp4(torch.from_numpy(q_rows).cuda(), torch.from_numpy(k_rows).cuda(), C,
                                      n_vis=torch.from_numpy(n_vis).cuda(), out=out))
    for b in range(B):
        kd = O.dequant_mxfp4(k_rows[b], C)
        rows = range(b * T, b * T + T) if B <= 4 else [b * T]
        for r in rows:
            ref = O.index_scores_mxfp4(q_rows.reshape(B * T, -1)[r:r + 1], k_rows[b], C, [n_vis[r]])[0]
            qd = O.dequant_mxfp4(q_rows.reshape(B * T, -1)[r:r + 1], C)
            mask = np.arange(N) < n_vis[r]
            check_scores(s[r], ref, (np.abs(qd) @ np.abs(kd).T)[0], mask, f"mxfp4 r={r}")
            assert np.all(s[r][~mask] == 7.0)


@pytest.mark.parametrize("B,T,N,C,p0,rows", [
    (1, 1100, 3000, 512, 9000, None),      # three 512-row slabs, ragged keys and rows
    (2, 300, 1234, 256, 4000, None),       # 256 channels, two sequences
    (1, 64, 40, 512, 0, None),             # fewer keys than one tile, early rows see none
    (1, 4096, 33792, 512, 131072, [0, 1, 2, 3, 511, 512, 1023, 2047, 2048, 3000, 4093, 4095])])
def test_index_scores_mxfp4_prefill_mfma(B, T, N, C, p0, rows):
    """FP4 (MXFP4) indexer on the scaled FP4 MFMA (T >= 16, one key head per index head) against
    the oracle: causal visibility from the prefill rule, several query slabs, ragged key tiles,
    both channel counts, and the 4096-token prefill chunk over 33792 entries at full size (sampled
    rows, every visible column). Block magnitudes spread over 2^-3 .. 2^3 so the blocks' E8M0
    scales differ. Slots past n_vis stay as they were."""
    g = np.random.default_rng(T + N + C)
    spread = lambda n: np.ldexp(1.0, g.integers(-3, 4, size=(n, C // 32))).repeat(32, 1).astype(np.float32)
    xq = g.standard_normal((B * T, C)).astype(np.float32) * spread(B * T)
    xk = g.standard_normal((B * N, C)).astype(np.float32) * spread(B * N)
    q_rows = O.quantize_mxfp4(xq).reshape(B, T, -1)
    k_rows = O.quantize_mxfp4(xk).reshape(B, N, -1)
    nv = np.minimum(O.prefill_n_vis(p0, T, 4), N).astype(np.int32)
    nv_all = np.concatenate([nv] * B)
    out = torch.full((B * T, N), 7.0, dtype=torch.float32).cuda()
    s = _sync_np(P.index_scores_mxfp4(torch.from_numpy(q_rows).cuda(), torch.from_numpy(k_rows).cuda(), C,
                                      n_vis=torch.from_numpy(nv_all).cuda(), out=out))
    rs = range(T) if rows is None else rows
    for b in range(B):
        kd = O.dequant_mxfp4(k_rows[b], C)
        qrows = q_rows[b][list(rs)]
        ref = O.index_scores_mxfp4(qrows, k_rows[b], C, nv[list(rs)])
        qd = O.dequant_mxfp4(qrows, C)
        absdot = np.abs(qd) @ np.abs(kd).T
        for i, t in enumerate(rs):
            mask = np.arange(N) < nv[t]
            check_scores(s[b * T + t], ref[i], absdot[i], mask, f"mxfp4 prefill b={b} t={t}")
            assert np.all(s[b * T + t][~mask] == 7.0)


@pytest.mark.parametrize("B,T,N,Hi", [(2, 1, 3001, 32), (3, 2, 500, 1), (1, 1, 70000, 32), (4, 1, 1, 16)])
def test_index_scores_mxfp4_shared_key(B, T, N, Hi):
    """FP4 indexer with one shared 128-channel key per entry and Hi query heads (the paper-scale
    indexer shape) against the oracle: ragged tiles, several query rows with n_vis cuts, long
    rows, one entry."""
    g = np.random.default_rng(N + Hi)
    q_rows = O.quantize_mxfp4(g.standard_normal((B * T, Hi * 128)).astype(np.float32)).reshape(B, T, -1)
    k_rows = O.quantize_mxfp4(g.standard_normal((B * N, 128)).astype(np.float32)).reshape(B, N, -1)
    n_vis = np.array([max(1, N - 13 * r) for r in range(B * T)], np.int32)
    out = torch.full((B * T, N), 7.0, dtype=torch.float32).cuda()
    s = _sync_np(P.index_scores_mxfp4(torch.from_numpy(q_rows).cuda(), torch.from_numpy(k_rows).cuda(), 128,
                                      n_vis=torch.from_numpy(n_vis).cuda(), out=out, q_heads=Hi))
    for b in range(B):
        kd = O.dequant_mxfp4(k_rows[b], 128)
        for t in range(T):
            r = b * T + t
            qr = q_rows.reshape(B * T, -1)[r:r + 1]
            ref = O.index_scores_mxfp4(qr, k_rows[b], 128, [n_vis[r]], q_heads=Hi)[0]
            qd = O.dequant_mxfp4(qr, Hi * 128).reshape(Hi, 128)
            abs_dot = np.abs(qd).sum(axis=0) @ np.abs(kd).T
            mask = np.arange(N) < n_vis[r]
            check_scores(s[r], ref, abs_dot, mask, f"mxfp4 shared r={r}")
            assert np.all(s[r][~mask] == 7.0)


@pytest.mark.parametrize("Hi,Hk,Di", [(32, 1, 128), (8, 8, 64), (4, 4, 64)])
def test_index_scores_mxfp4_pool_and_block_max(Hi, Hk, Di):
    """FP4 indexer pool modes, shared-key and per-head forms: the fused 8-entry block max equals
    the max of the kernel's own scores over visible block members (ragged n_vis), and candidate
    scoring (empty slots and out-of-range positions give -inf) matches the oracle's pool scores."""
    B, N, n_pool = 2, 3001, 1000
    kc, qc = Hk * Di, Hi * Di
    g = np.random.default_rng(12 + Hi)
    q_rows = O.quantize_mxfp4(g.standard_normal((B, qc)).astype(np.float32)).reshape(B, 1, -1)
    k_rows = O.quantize_mxfp4(g.standard_normal((B * N, kc)).astype(np.float32)).reshape(B, N, -1)
    n_vis = np.array([N, 1237], np.int32)
    qd, kq = torch.from_numpy(q_rows).cuda(), torch.from_numpy(k_rows).cuda()
    C, qh = (Di, Hi) if Hk == 1 else (kc, 0)
    s, bm = P.index_scores_mxfp4(qd, kq, C, n_vis=torch.from_numpy(n_vis).cuda(), q_heads=qh, block_max=True)
    s, bm = _sync_np(s), _sync_np(bm)
    cand = np.sort(g.choice(N + 40, size=(B, n_pool), replace=True), axis=1).astype(np.int32)
    cand[:, -37:] = -1
    sp = _sync_np(P.index_scores_mxfp4(qd, kq, C, q_heads=qh, cand=torch.from_numpy(cand).cuda()))
    for b in range(B):
        qv = O.dequant_mxfp4(q_rows[b], qc).reshape(1, Hi, Di)
        kv = O.dequant_mxfp4(k_rows[b], kc).reshape(N, Hk, Di)
        abs_dot = _abs_dot(qv, kv)[0]
        ref = O.index_scores(qv, kv, [n_vis[b]])[0]
        mask = np.arange(N) < n_vis[b]
        check_scores(s[b], ref, abs_dot, mask, f"mxfp4 flat b={b}")
        nb = -(-int(n_vis[b]) // 8)
        assert np.array_equal(bm[b, :nb], O.block_max(s[b:b + 1], [n_vis[b]])[0][:nb])
        pref = O.pool_scores(qv, kv, np.where(cand[b:b + 1] < N, cand[b:b + 1], -1))[0]
        ok = (cand[b] >= 0) & (cand[b] < N)
        assert np.all(np.isneginf(sp[b][~ok]))
        check_scores(sp[b], pref, np.where(ok, abs_dot[np.clip(cand[b], 0, N - 1)], 0.0), ok, f"mxfp4 pool b={b}")


def test_index_scores_mxfp4_exact_blocks():
    """Keys equal to the query on one 32-channel block and zero elsewhere: every score is that
    block's exact sum of squares times its scale squared (one exact block, no rounding)."""
    C, N = 512, 300
    g = np.random.default_rng(3)
    xq = g.standard_normal((1, C)).astype(np.float32)
    q_rows = O.quantize_mxfp4(xq)
    k_src = np.zeros((N, C), np.float32)
    qd = O.dequant_mxfp4(q_rows, C)[0]
    for n in range(N):
        blk = n % 16
        k_src[n, 32 * blk: 32 * blk + 32] = qd[32 * blk: 32 * blk + 32]
    k_rows = O.quantize_mxfp4(k_src)
    s = _sync_np(P.index_scores_mxfp4(torch.from_numpy(q_rows[None]).cuda(), torch.from_numpy(k_rows[None]).cuda(), C))
    want = np.array([np.sum(qd[32 * (n % 16): 32 * (n % 16) + 32] ** 2) for n in range(N)], np.float32)
    assert np.array_equal(s[0], want)


@pytest.mark.parametrize("B,T,H,N,K,Wn,p0", [(1, 600, 64, 700, 64, 128, 50), (2, 260, 64, 900, 300, 100, 0),
                                             (1, 520, 128, 600, 64, 32, -3),
                                             (2, 40, 16, 300, 33, 64, 10),
                                             (1, 520, 32, 200, 40, 100, 500), (1, 3, 16, 20, 0, 8, 0),
                                             (2, 1, 16, 300, 33, 64, 10), (3, 1, 64, 500, 64, 128, 1000)])
def test_sparse_attn_swa_prefill(B, T, H, N, K, Wn, p0):
    """Prefill with each query token's own window (its last n tokens up to its own, n < W near the
    start of the sequence) joined to its selected entries, against the oracle: the 64-head prefill
    form with the window as further chunks of its own pass (600 rows; two sequences with ragged
    selections and windows, from 1 to 100 rows; 128 heads in two groups with one-chunk windows,
    the first three tokens' windows empty), the decode form with several query tokens (split path), the wide
    32-head form, no selected entries, and one-token chunks (T = 1: the window buffer holds W rows
    and the token takes its last n of them, with n < W and n = W)."""
    rows, qb, idx = _attn_case(B, T, H, N, K, seed=T + K + Wn, oob=K > 0) if K > 0 else _attn_case(B, T, H, N, 1, seed=5)
    if K == 0:
        idx = np.zeros((B, T, 0), np.int32)
    g = np.random.default_rng(T + Wn)
    codes, exps = O.quantize_swa_fp8(g.standard_normal((B * (T + Wn - 1), 512)).astype(np.float32))
    codes, exps = codes.reshape(B, T + Wn - 1, 512), exps.reshape(B, T + Wn - 1)
    n_win = np.array([[max(0, min(Wn, p0 + t + 1)) for t in range(T)] for _ in range(B)], np.int32)
    scale = 1 / np.sqrt(512)
    out, lse = P.sparse_attn_swa_prefill(dev_bf16(qb), torch.from_numpy(rows).cuda(), torch.from_numpy(idx).cuda(),
                                         torch.from_numpy(codes).cuda(), torch.from_numpy(exps).cuda(),
                                         torch.from_numpy(n_win).cuda(), scale)
    out, lse = _sync_np(out), _sync_np(lse)
    for b in range(B):
        win = O.prefill_windows(O.dequant_swa_fp8(codes[b], exps[b]), n_win[b], Wn)
        clean = np.where((idx[b] >= 0) & (idx[b] < N), idx[b], -1)
        ref, lref = O.sparse_attn_swa(f64(qb[b]), O.dequant_kv_fp4(rows[b]), clean, win, n_win[b], scale)
        check_attn(out[b], ref, lse[b], lref, f"swa prefill B={B} T={T} H={H} K={K} b={b}")


@pytest.mark.timeout(300)
def test_sparse_attn_swa_prefill_full_size():
    """The windowed prefill call at the prefill workload's full size, in the launch the bench times
    (T = 4096 tokens, 33792 entries, 64 heads, Top-1024, 128-row windows, partial windows for the
    first tokens of the sequence): sampled query rows against the oracle, one by one, and two
    identical calls bit-identical."""
    T, N, H, K, Wn, p0 = 4096, 33792, 64, 1024, 128, 60
    rng = np.random.default_rng(11)
    rows = O.quantize_kv_fp4(rng.standard_normal((N, 512)).astype(np.float32))
    qb = W.to_bf16_bits(rng.standard_normal((T, H, 512), dtype=np.float32))
    idx = rng.integers(0, N, size=(T, K), dtype=np.int32)
    idx[:, ::97] = -1
    codes, exps = O.quantize_swa_fp8(rng.standard_normal((T + Wn - 1, 512)).astype(np.float32))
    n_win = np.array([min(Wn, p0 + t + 1) for t in range(T)], np.int32)
    scale = 1 / np.sqrt(512)
    args = (dev_bf16(qb[None]), torch.from_numpy(rows[None]).cuda(), torch.from_numpy(idx[None]).cuda(),
            torch.from_numpy(codes[None]).cuda(), torch.from_numpy(exps[None]).cuda(),
            torch.from_numpy(n_win[None]).cuda(), scale)
    out, lse = P.sparse_attn_swa_prefill(*args)
    out2, lse2 = P.sparse_attn_swa_prefill(*args)
    assert torch.equal(out, out2) and torch.equal(lse, lse2), "two identical calls differ"
    tr = np.array([0, 1, 59, 60, 61, 127, 2048, 4095])
    out, lse = _sync_np(out)[0, tr], _sync_np(lse)[0, tr]
    win = O.prefill_windows(O.dequant_swa_fp8(codes, exps), n_win, Wn)[tr]
    ref, lref = O.sparse_attn_swa(f64(qb[tr]), O.dequant_kv_fp4(rows), idx[tr], win, n_win[tr], scale)
    check_attn(out, ref, lse, lref, "windowed prefill at full size")
