"""Pins of the oracle's Hierarchical Sparse Indexer, sparse attention and layer modes (CPU only).

HSI: brute-force block max, pool shape/order, pool = everything reduces to the flat indexer,
Full's Top-K lies inside the pool when blocks >= K. Attention: K = N equals torch's
scaled_dot_product_attention (fp64, CPU), one selected entry returns it exactly, q = 0 returns the
mean, empty selections give 0 / -inf, lse equals torch.logsumexp. Modes: Reuse equals attention
with the source layer's indices; Reindex with the Full layer's indexer query reproduces its Top-K.
"""
import numpy as np
import pytest
import torch

from oracle import csa2_oracle as O
from fp4_kv_cache_e2m1_amd import workloads as W


def _small(N=200, Hi=2, Di=16, H=4, k=16, seed=0):
    g = np.random.default_rng(seed)
    bf = lambda shape: W.bf16_bits_to_f32(W.to_bf16_bits(g.standard_normal(shape).astype(np.float32))).astype(np.float64)
    kv_src = g.standard_normal((N, 512)).astype(np.float32)
    kv = O.dequant_kv_fp4(O.quantize_kv_fp4(kv_src))
    return dict(q=bf((1, H, 512)), q_idx=bf((1, Hi, Di)), q_idx2=bf((1, Hi, Di)), k_idx=bf((N, Hi, Di)),
                kv=kv, N=N, k=k)


def test_block_max_bruteforce():
    s = W.random_scores(1, 3, 29, "ties")
    n_vis = np.array([29, 17, 8])
    bm = O.block_max(s, n_vis, 8)
    assert bm.shape == (3, 4)
    for r in range(3):
        for j in range(4):
            vals = [s[r, n] for n in range(8 * j, min(8 * j + 8, 29)) if n < n_vis[r]]
            assert bm[r, j] == (max(vals) if vals else -np.inf)


def test_pool_shape_order_and_padding():
    s = W.random_scores(2, 2, 61, "normal")
    n_vis = np.array([61, 61])
    pool = O.hier_pool(O.block_max(s, n_vis), n_vis, n_sel_blocks=5)
    assert pool.shape == (2, 40)
    for r in range(2):
        valid = pool[r][pool[r] >= 0]
        assert np.all(np.diff(valid) > 0)
        assert np.all(pool[r][len(valid):] == -1)
        assert len(valid) in (40, 37)          # the last block [56, 61) has only 5 positions
        blocks = np.unique(valid // 8)
        assert len(blocks) == 5
        # the chosen blocks are the 5 best by block max (ties impossible with normal scores)
        bm = O.block_max(s[r:r + 1], [61])[0]
        assert set(blocks) == set(np.argsort(-bm)[:5])
    # fewer valid blocks than asked for: everything visible, then -1
    pool = O.hier_pool(O.block_max(s[:1], [12]), [12], n_sel_blocks=4)
    assert pool[0].tolist() == list(range(12)) + [-1] * 20


def test_hierarchical_equals_flat_when_pool_covers_everything():
    d = _small(N=203)
    nb = -(-d["N"] // 8)
    full = O.layer_step(O.FULL, q=d["q"], kv_deq=d["kv"], k_idx=d["k_idx"], q_idx=d["q_idx"],
                        n_vis=[d["N"]], k=d["k"], pool_blocks=nb)
    assert full["pool"][0].tolist() == list(range(d["N"])) + [-1] * (8 * nb - d["N"])
    hier = O.layer_step(O.REINDEX, q=d["q"], kv_deq=d["kv"], k_idx=d["k_idx"], q_idx=d["q_idx2"],
                        n_vis=[d["N"]], k=d["k"], pool=full["pool"])
    flat = O.layer_step(O.REINDEX, q=d["q"], kv_deq=d["kv"], k_idx=d["k_idx"], q_idx=d["q_idx2"],
                        n_vis=[d["N"]], k=d["k"])
    assert np.array_equal(hier["topk"], flat["topk"])
    assert np.array_equal(hier["out"], flat["out"])


def test_full_topk_inside_pool_and_reindex_with_same_query():
    d = _small(N=400, k=16)
    full = O.layer_step(O.FULL, q=d["q"], kv_deq=d["kv"], k_idx=d["k_idx"], q_idx=d["q_idx"],
                        n_vis=[d["N"]], k=d["k"], pool_blocks=16)
    assert set(full["topk"][0].tolist()) <= set(full["pool"][0].tolist())
    re = O.layer_step(O.REINDEX, q=d["q"], kv_deq=d["kv"], k_idx=d["k_idx"], q_idx=d["q_idx"],
                      n_vis=[d["N"]], k=d["k"], pool=full["pool"])
    assert np.array_equal(re["topk"], full["topk"])
    assert np.array_equal(re["out"], full["out"])


def test_pool_scores_equal_flat_scores_at_pool_positions():
    d = _small(N=150)
    flat = O.index_scores(d["q_idx"], d["k_idx"], [150])
    pool = np.array([[3, 4, 5, 77, 149, -1, -1]])
    ps = O.pool_scores(d["q_idx"], d["k_idx"], pool)
    assert np.array_equal(ps[0, :5], flat[0, [3, 4, 5, 77, 149]])
    assert np.all(ps[0, 5:] == -np.inf)


def test_attention_full_selection_equals_sdpa():
    d = _small(N=64, H=5)
    idx = np.arange(64)[None, :]
    scale = 1 / np.sqrt(512)
    out, lse = O.sparse_attn(d["q"], d["kv"], idx, scale)
    q = torch.from_numpy(d["q"][0])[None]               # [1, H, D]
    kv = torch.from_numpy(d["kv"])[None, None].expand(1, 5, 64, 512)
    ref = torch.nn.functional.scaled_dot_product_attention(q[:, :, None, :], kv, kv, scale=scale)[0, :, 0]
    assert np.allclose(out[0], ref.numpy(), rtol=0, atol=2e-6)
    logits = (q[0] @ torch.from_numpy(d["kv"]).T) * scale
    assert np.allclose(lse[0], torch.logsumexp(logits, dim=1).numpy(), rtol=1e-6)


def test_attention_permutation_and_padding_invariance():
    d = _small(N=80)
    g = np.random.default_rng(4)
    idx = g.choice(80, size=20, replace=False)[None]
    a, la = O.sparse_attn(d["q"], d["kv"], idx, 0.1)
    pad = np.concatenate([idx[:, ::-1], -np.ones((1, 7), dtype=np.int64)], axis=1)
    b, lb = O.sparse_attn(d["q"], d["kv"], pad, 0.1)
    assert np.allclose(a, b, atol=1e-6) and np.allclose(la, lb, atol=1e-6)


def test_attention_degenerate_cases():
    d = _small(N=30)
    one, lse = O.sparse_attn(d["q"], d["kv"], np.array([[-1, 7, -1]]), 0.3)
    assert np.array_equal(one[0], np.broadcast_to(d["kv"][7].astype(np.float32), one[0].shape))
    zq = np.zeros_like(d["q"])
    mean, _ = O.sparse_attn(zq, d["kv"], np.array([[1, 2, 9]]), 0.3)
    assert np.allclose(mean[0, 0], d["kv"][[1, 2, 9]].mean(axis=0), atol=1e-6)
    empty, lse = O.sparse_attn(d["q"], d["kv"], np.full((1, 4), -1), 0.3)
    assert np.all(empty == 0) and np.all(lse == -np.inf)


def test_reuse_equals_attention_with_source_indices():
    d = _small(N=120)
    src = O.layer_step(O.FULL, q=d["q"], kv_deq=d["kv"], k_idx=d["k_idx"], q_idx=d["q_idx"],
                       n_vis=[d["N"]], k=d["k"])
    q2 = d["q"][:, ::-1].copy()
    reuse = O.layer_step(O.REUSE, q=q2, kv_deq=d["kv"], shared_topk=src["topk"])
    ref, _ = O.sparse_attn(q2, d["kv"], src["topk"], 1 / np.sqrt(512))
    assert np.array_equal(reuse["out"], ref)
    assert np.array_equal(reuse["topk"], src["topk"]) and reuse["scores"] is None


def test_planted_keys_dominate_full_topk():
    # the structured workload: 1% of keys shifted 3 sigma toward the first indexer query
    wl = W.CONFIGS[4].scaled(N=16384, k=64, B=1)
    kb = W.bf16_bits_to_f32(W.k_idx(wl, 0)).astype(np.float64)
    qb = W.bf16_bits_to_f32(W.q_idx(wl, 0, 0)).astype(np.float64)
    s = O.index_scores(qb, kb, [wl.N])
    sel = O.topk(s, wl.k)[0]
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([1000 * 4 + W.TID_PLANT, 0])))
    planted = set(g.choice(wl.N, size=int(round(0.01 * wl.N)), replace=False).tolist())
    assert set(sel.tolist()) <= planted
