"""Pins of the oracle's FP4 indexer format (O13): OCP MXFP4 rows (E2M1 elements, one E8M0 scale
per 32 channels) and the indexer score over them (CPU only).

Fixed outside the oracle: torch's float8_e8m0fnu decoder for all 256 scale codes, the OCP E2M1
table (golden file), the MX conversion rule restated here from the spec with math.frexp and a
brute-force nearest search, and an exact rational double loop for the score.
"""
import math
import os
from fractions import Fraction

import numpy as np
import torch

from oracle import csa2_oracle as O


def _e2m1_golden(golden_dir):
    vals = {}
    for line in open(os.path.join(golden_dir, "e2m1_values.txt")):
        line = line.split("#")[0].strip()
        if line:
            c, v = line.split()[:2]
            vals[int(c)] = float(v)
    return vals


def test_e8m0_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = O.e8m0_decode(codes)
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127


def test_dequant_layout_by_hand(golden_dir):
    e2m1 = _e2m1_golden(golden_dir)
    g = np.random.default_rng(3)
    rows = g.integers(0, 256, size=(5, O.mxfp4_row_bytes(256)), dtype=np.uint8)
    rows[:, 128:] = g.integers(100, 140, size=(5, 8))
    got = O.dequant_mxfp4(rows, 256)
    for r in range(5):
        for c in range(256):
            nib = (rows[r, c // 2] >> (4 * (c % 2))) & 0xF
            want = e2m1[int(nib)] * 2.0 ** (int(rows[r, 128 + c // 32]) - 127)
            assert got[r, c] == want, (r, c)


def _brute_block(x):
    """The MX conversion of one block of 32, restated: X = floor(log2 amax) - emax(E2M1 = 2)."""
    amax = max(abs(float(v)) for v in x)
    if amax == 0.0:
        X = -127
    else:
        m, e = math.frexp(amax)
        X = min(127, max(-127, e - 1 - 2))
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    codes = []
    for v in x:
        a = Fraction(abs(float(v)))
        sc = Fraction(2) ** X
        d = [abs(a - sc * Fraction(m)) for m in mags]
        best = min(d)
        js = [j for j in range(8) if d[j] == best]
        j = js[0] if len(js) == 1 else [j for j in js if j % 2 == 0][0]
        if a >= 6 * sc:
            j = 7
        codes.append((int(math.copysign(1, float(v)) < 0) << 3) | j)
    return codes, X


def test_quantize_matches_the_mx_rule_by_brute_force():
    g = np.random.default_rng(4)
    x = (g.standard_normal((6, 128)) * 10.0 ** g.uniform(-4, 3, size=(6, 1))).astype(np.float32)
    x[0, :32] = 0.0                                    # a zero block
    x[1, :32] = -0.0
    x[2, 5] = 6.0 * 2.0 ** 3                           # amax exactly at a power-of-two boundary
    x[3, 40:72] = np.float32(2.0 ** -130)              # below the E8M0 range: X clamps at -127
    rows = O.quantize_mxfp4(x)
    for r in range(x.shape[0]):
        for b in range(4):
            codes, X = _brute_block(x[r, 32 * b: 32 * b + 32])
            assert rows[r, 64 + b] == X + 127, (r, b)
            for i, c in enumerate(codes):
                ch = 32 * b + i
                assert (rows[r, ch // 2] >> (4 * (ch % 2))) & 0xF == c, (r, ch)


def test_quantize_error_bound_and_block_maximum():
    g = np.random.default_rng(5)
    x = g.standard_normal((64, 512)).astype(np.float32) * np.float32(3.0)
    rows = O.quantize_mxfp4(x)
    d = O.dequant_mxfp4(rows, 512)
    scale = np.repeat(O.e8m0_decode(rows[:, 256:]), 32, axis=1)
    # elements below 6 * 2^X round to within half a step (at most 1 * 2^X); above it saturate
    # (amax < 8 * 2^X), so every error is below 2 * 2^X
    assert np.all(np.abs(d - x) < 2.0 * scale)
    # the block maximum maps to 4 or 6 times the scale (amax / 2^X lies in [4, 8))
    xb = np.abs(x.reshape(64, 16, 32)).max(axis=-1)
    db = np.abs(d.reshape(64, 16, 32)).max(axis=-1)
    sb = O.e8m0_decode(rows[:, 256:])
    assert np.all((db == 4 * sb) | (db == 6 * sb))
    assert np.all((xb >= 4 * sb) & (xb < 8 * sb))


def test_quantize_is_exact_on_representable_values():
    g = np.random.default_rng(6)
    rows = g.integers(0, 256, size=(8, O.mxfp4_row_bytes(256)), dtype=np.uint8)
    rows[:, 128:] = g.integers(110, 140, size=(8, 8))
    v = O.dequant_mxfp4(rows, 256)
    again = O.dequant_mxfp4(O.quantize_mxfp4(v.astype(np.float32)), 256)
    # a block is re-encoded exactly when its maximum fixes the same exponent (max magnitude 4 or 6)
    vb = np.abs(v.reshape(8, 8, 32)).max(axis=-1)
    sb = O.e8m0_decode(rows[:, 128:])
    same = (vb == 4 * sb) | (vb == 6 * sb)
    same_ch = np.repeat(same, 32, axis=1)
    assert same.any()
    assert np.array_equal(again[same_ch], v[same_ch])


def test_index_score_is_the_exact_dot_product(golden_dir):
    e2m1 = _e2m1_golden(golden_dir)
    g = np.random.default_rng(7)
    C = 128
    q = O.quantize_mxfp4(g.standard_normal((3, C)).astype(np.float32))
    k = O.quantize_mxfp4((g.standard_normal((9, C)) * 5).astype(np.float32))

    def val(row, c):
        nib = (row[c // 2] >> (4 * (c % 2))) & 0xF
        return Fraction(e2m1[int(nib)]) * Fraction(2) ** (int(row[C // 2 + c // 32]) - 127)

    got = O.index_scores_mxfp4(q, k, C, [9, 9, 4])
    for r in range(3):
        for n in range(9):
            if n >= [9, 9, 4][r]:
                assert got[r, n] == -np.inf
                continue
            exact = sum(val(q[r], c) * val(k[n], c) for c in range(C))
            assert got[r, n] == np.float32(float(exact)), (r, n)


def test_index_score_shared_key_is_the_exact_sum_over_heads(golden_dir):
    """One 128-channel key per entry, four query heads: the exact sum over heads of each head's
    dot product with the key."""
    e2m1 = _e2m1_golden(golden_dir)
    g = np.random.default_rng(8)
    Dk, Hq = 128, 4
    q = O.quantize_mxfp4(g.standard_normal((2, Hq * Dk)).astype(np.float32))
    k = O.quantize_mxfp4((g.standard_normal((7, Dk)) * 3).astype(np.float32))

    def val(row, c, C):
        nib = (row[c // 2] >> (4 * (c % 2))) & 0xF
        return Fraction(e2m1[int(nib)]) * Fraction(2) ** (int(row[C // 2 + c // 32]) - 127)

    got = O.index_scores_mxfp4(q, k, Dk, [7, 5], q_heads=Hq)
    for r in range(2):
        for n in range(7):
            if n >= [7, 5][r]:
                assert got[r, n] == -np.inf
                continue
            exact = sum(val(q[r], h * Dk + c, Hq * Dk) * val(k[n], c, Dk) for h in range(Hq) for c in range(Dk))
            assert got[r, n] == np.float32(float(exact)), (r, n)
