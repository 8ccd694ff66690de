"""Pins of the oracle's indexer scores and Top-K (CPU only).

Scores: exact brute force with math.fsum over Python floats (tiny inputs), shared-key collapse,
visibility masking. Top-K: brute force sorted() on tiny rows including exhaustive ties,
torch.topk on distinct values, padding, pool columns, permutation equivariance.
"""
import itertools
import math

import numpy as np
import pytest
import torch

from oracle import csa2_oracle as O
from fp4_kv_cache_e2m1_amd import workloads as W


def _bf16_vals(g, shape):
    return W.bf16_bits_to_f32(W.to_bf16_bits(g.standard_normal(shape).astype(np.float32))).astype(np.float64)


@pytest.mark.parametrize("Hi,Hk,Di", [(4, 4, 64), (8, 8, 64), (3, 1, 16), (2, 2, 8)])
def test_index_scores_bruteforce(Hi, Hk, Di):
    g = np.random.default_rng(Hi * 100 + Hk)
    R, N = 3, 11
    q = _bf16_vals(g, (R, Hi, Di))
    k = _bf16_vals(g, (N, Hk, Di))
    n_vis = np.array([11, 7, 1])
    got = O.index_scores(q, k, n_vis)
    for r in range(R):
        for n in range(N):
            if n >= n_vis[r]:
                assert got[r, n] == -np.inf
                continue
            terms = [q[r, h, d] * k[n, 0 if Hk == 1 else h, d] for h in range(Hi) for d in range(Di)]
            exact = math.fsum(terms)
            assert got[r, n] == np.float32(exact)


def test_index_scores_shared_key_collapses_heads():
    g = np.random.default_rng(1)
    q = _bf16_vals(g, (2, 4, 16))
    k1 = _bf16_vals(g, (9, 1, 16))
    a = O.index_scores(q, k1, [9, 9])
    b = O.index_scores(q.sum(axis=1, keepdims=True), k1, [9, 9])   # sum over heads is exact here
    assert np.array_equal(a, b)


def _topk_bruteforce(row, k, pos=None):
    n = len(row)
    pos = list(range(n)) if pos is None else list(pos)
    items = [(float(row[c]), pos[c]) for c in range(n) if pos[c] >= 0]
    items.sort(key=lambda t: (-t[0], t[1]))
    sel = sorted(p for _, p in items[:k])
    return sel + [-1] * (k - len(sel))


@pytest.mark.parametrize("dist", ["normal", "ties", "const", "signed_zero", "bounded"])
def test_topk_bruteforce(dist):
    for n in (1, 5, 17, 64):
        s = W.random_scores(n, 4, n, dist)
        for k in (1, 3, n, n + 3):
            got = O.topk(s, k)
            for r in range(4):
                assert got[r].tolist() == _topk_bruteforce(s[r], k)


def test_topk_exhaustive_tiny_ties():
    # every row over the alphabet {0, 1, 2} of length 5 and every k
    for row in itertools.product([0.0, 1.0, 2.0], repeat=5):
        s = np.array([row], dtype=np.float32)
        for k in range(1, 6):
            assert O.topk(s, k)[0].tolist() == _topk_bruteforce(s[0], k)


def test_topk_matches_torch_on_distinct_values():
    s = W.random_scores(3, 6, 5000, "normal")
    assert all(len(np.unique(row)) == row.size for row in s)
    got = O.topk(s, 300)
    ref = torch.topk(torch.from_numpy(s), 300, dim=1).indices.numpy()
    for r in range(6):
        assert np.array_equal(got[r], np.sort(ref[r]))


def test_topk_n_valid_and_pool_columns():
    s = W.random_scores(4, 3, 40, "ties")
    got = O.topk(s, 8, n_valid=[40, 5, 0])
    assert got[0].tolist() == _topk_bruteforce(s[0], 8)
    assert got[1].tolist() == _topk_bruteforce(s[1][:5], 8)
    assert got[2].tolist() == [-1] * 8
    pool = np.array([[100 + 3 * c if c < 30 else -1 for c in range(40)]] * 3)
    got = O.topk(s, 8, col_to_pos=pool)
    for r in range(3):
        assert got[r].tolist() == _topk_bruteforce(s[r], 8, pool[r])


def test_topk_permutation_equivariance():
    g = np.random.default_rng(2)
    s = W.random_scores(5, 1, 200, "normal")
    perm = g.permutation(200)
    a = set(O.topk(s, 37)[0].tolist())
    b = set(perm[O.topk(s[:, perm], 37)[0]].tolist())
    assert a == b


def test_prefill_visibility_reproduces_32768_plus_1024():
    nv = O.prefill_n_vis(131072, 4096, 4)
    assert nv[0] == 32768 and nv[-1] == 32768 + 1024
    assert np.all(np.diff(nv) >= 0)
    wl = W.CONFIGS[5]
    assert wl.N == nv[-1] and wl.n_existing == nv[0]
