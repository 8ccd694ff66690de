"""Pins of the oracle's cache producers (O14 compressor, O15 indexer-K projection).

The pages give the compressor's structure (m tokens -> one entry, no overlap, no absolute
position encoding) and say indexer K is a projection of the main-KV entries, but print no
formula and no example. These tests pin the oracle to what that structure and the mathematics
fix: closed forms (one token per entry, equal weights, one dominant weight), invariants (shift of
the weights, token order inside a group, no overlap between groups, convexity), a brute-force
loop with correctly rounded sums, the bf16 rounding against torch's, and exact rational
projections.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from fp4_kv_cache_e2m1_amd import workloads as W
from oracle import csa2_oracle as O


def _bf16(x):
    return W.bf16_bits_to_f32(W.to_bf16_bits(np.asarray(x, np.float32))).astype(np.float64)


def _tokens(seed, n, d=64, zscale=1.0):
    g = np.random.default_rng(seed)
    return _bf16(g.standard_normal((n, d))), _bf16(zscale * g.standard_normal((n, d)))


def test_ratio_one_returns_the_tokens():
    c, z = _tokens(1, 40)
    assert np.array_equal(O.compress_kv(c, z, 1), c.astype(np.float32))


@pytest.mark.parametrize("ratio", [2, 4, 8])
def test_equal_weights_give_the_exact_mean(ratio):
    c, _ = _tokens(2, 8 * ratio)
    z = np.zeros_like(c) + 0.75                      # one weight value everywhere
    got = O.compress_kv(c, z, ratio)
    for j in range(8):
        for d in range(0, 64, 7):
            exact = sum(Fraction(float(c[j * ratio + i, d])) for i in range(ratio)) / ratio
            assert got[j, d] == np.float32(float(exact))


def test_one_dominant_weight_selects_its_token():
    c, _ = _tokens(3, 32)
    z = np.full_like(c, -60.0)
    pick = np.random.default_rng(3).integers(0, 4, size=(8, 64))
    for j in range(8):
        z[4 * j + pick[j], np.arange(64)] = 60.0
    got = O.compress_kv(c, z, 4)
    want = c.reshape(8, 4, 64)[np.arange(8)[:, None], pick, np.arange(64)[None, :]]
    assert np.array_equal(got, want.astype(np.float32))


def test_shift_of_the_weights_changes_nothing():
    c, z = _tokens(4, 64)
    shift = np.repeat(np.random.default_rng(4).integers(-8, 9, size=(16, 64)), 4, axis=0).astype(np.float64)
    assert np.array_equal(O.compress_kv(c, z, 4), O.compress_kv(c, z + shift, 4))


def test_token_order_inside_a_group_and_no_overlap():
    c, z = _tokens(5, 64)
    base = O.compress_kv(c, z, 4)
    perm = np.concatenate([4 * j + np.random.default_rng(j).permutation(4) for j in range(16)])
    np.testing.assert_allclose(O.compress_kv(c[perm], z[perm], 4), base, rtol=1e-6, atol=1e-30)
    c2, z2 = c.copy(), z.copy()
    c2[20:24] += 5.0                                  # tokens of group 5 only
    z2[20:24] -= 1.0
    got = O.compress_kv(c2, z2, 4)
    assert not np.array_equal(got[5], base[5])
    assert np.array_equal(np.delete(got, 5, axis=0), np.delete(base, 5, axis=0))


def test_entries_are_convex_combinations():
    c, z = _tokens(6, 128, zscale=4.0)
    got = O.compress_kv(c, z, 8).astype(np.float64)
    g = c.reshape(16, 8, 64)
    assert np.all(got >= g.min(axis=1) - 1e-6 * np.abs(g).max(axis=1))
    assert np.all(got <= g.max(axis=1) + 1e-6 * np.abs(g).max(axis=1))


def test_brute_force_loop():
    """Each entry against a plain loop: math.exp weights and correctly rounded sums (math.fsum)."""
    c, z = _tokens(7, 12, d=8, zscale=3.0)
    got = O.compress_kv(c, z, 3)
    for j in range(4):
        for d in range(8):
            zs = [float(z[3 * j + i, d]) for i in range(3)]
            top = max(zs)
            ws = [math.exp(v - top) for v in zs]
            tot = math.fsum(ws)
            val = math.fsum(ws[i] / tot * float(c[3 * j + i, d]) for i in range(3))
            assert abs(float(got[j, d]) - val) <= 2.0 ** -23 * abs(val) + 1e-300


def test_round_bf16_matches_torch():
    g = np.random.default_rng(8)
    x = (g.standard_normal(20000) * np.exp(g.uniform(-20, 20, 20000))).astype(np.float32)
    ties = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 3.0 * (1 + 2 ** -8)], np.float32)
    x = np.concatenate([x, ties])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_bf16(x.astype(np.float64)), want)


def test_projection_identity_is_bf16_rounding():
    g = np.random.default_rng(9)
    e = g.standard_normal((10, 64)).astype(np.float32)
    k = O.project_index_k(e, np.eye(64), 4, 16)
    want = torch.from_numpy(e).to(torch.bfloat16).to(torch.float64).numpy().reshape(10, 4, 16)
    assert np.array_equal(k, want)


def test_projection_exact_rational():
    """Small integer-valued entries and weights: the sum is an exact integer, and against an exact
    rational double loop with round-half-even to 8 significant bits."""
    g = np.random.default_rng(10)
    e = g.integers(-6, 7, size=(5, 32)).astype(np.float32) * np.float32(0.5)
    w = g.integers(-9, 10, size=(3 * 8, 32)).astype(np.float64) * 0.25
    k = O.project_index_k(e, w, 3, 8)
    y = O.project_index_k(e, w, 3, 8, rounded=False)
    for n in range(5):
        for o in range(24):
            exact = sum(Fraction(float(e[n, c])) * Fraction(float(w[o, c])) for c in range(32))
            assert y.reshape(5, 24)[n, o] == float(exact)
            if exact == 0:
                assert k.reshape(5, 24)[n, o] == 0
                continue
            ex = math.floor(math.log2(abs(exact)))
            q = exact / Fraction(2) ** (ex - 7)          # 8 significant bits before the point
            r = round(q)                                  # Python rounds half to even
            assert k.reshape(5, 24)[n, o] == float(r * Fraction(2) ** (ex - 7))


def test_projection_is_linear_in_the_weights():
    g = np.random.default_rng(11)
    e = g.integers(-4, 5, size=(6, 16)).astype(np.float32)
    w1 = g.integers(-3, 4, size=(16, 16)).astype(np.float64)
    w2 = g.integers(-3, 4, size=(16, 16)).astype(np.float64)
    y = lambda w: O.project_index_k(e, w, 2, 8, rounded=False)
    assert np.array_equal(y(w1 + w2), y(w1) + y(w2))
