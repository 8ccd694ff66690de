"""Pins of the oracle's FP4 quantizer and packing (CPU only).

Independent checks: an exact-rational brute force (fractions.Fraction) over every scale code and
every value code, torch's fp32 -> float8_e4m3fn rounding for the scale, hand-built ties (golden
file), saturation, zero groups, idempotence and the error bound.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import csa2_oracle as O

E2M1_EXACT = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
              Fraction(4), Fraction(6)]


def _e4m3_exact(code):
    e, m = (code >> 3) & 15, code & 7
    return Fraction(m, 512) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7)


E4M3_EXACT = [_e4m3_exact(c) for c in range(0x7F)]


def _nearest_even_bruteforce(values, target):
    best = None
    for i, v in enumerate(values):
        d = abs(v - target)
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
            best = (d, i)
    return best[1]


def _quantize_group_bruteforce(x):
    """Exact-rational brute force: nearest scale to amax/6, then nearest magnitude per value."""
    xs = [Fraction(float(v)) for v in x]
    amax = max(abs(v) for v in xs)
    sc = _nearest_even_bruteforce(E4M3_EXACT, amax / 6)
    s = E4M3_EXACT[sc]
    codes = []
    for v, raw in zip(xs, x):
        j = 0 if s == 0 else _nearest_even_bruteforce(E2M1_EXACT, abs(v) / s)
        codes.append((8 if np.signbit(raw) else 0) | j)
    return codes, sc


@pytest.mark.parametrize("scale_kind", ["normal", "small", "tiny", "huge", "mixed"])
def test_quantizer_matches_exact_bruteforce(scale_kind):
    g = np.random.default_rng(7)
    mult = {"normal": 1.0, "small": 0.02, "tiny": 2e-4, "huge": 900.0, "mixed": None}[scale_kind]
    for trial in range(60):
        m = mult if mult is not None else 10.0 ** g.uniform(-5, 4)
        x = (g.standard_normal(16) * m).astype(np.float32)
        if trial % 5 == 0:
            x[g.integers(16)] = -x[g.integers(16)]
        codes, sc = O.quantize_groups(x.reshape(1, 16))
        bc, bsc = _quantize_group_bruteforce(x)
        assert int(sc[0]) == bsc, (x, sc, bsc)
        assert codes[0].tolist() == bc, (x, codes, bc)


def test_scale_rounding_matches_torch_e4m3():
    # For amax = 6 t with t an fp32 of few bits, the chosen scale is the E4M3 rounding of t, which
    # torch's fp32 -> float8_e4m3fn conversion computes (round to nearest, ties to even).
    g = np.random.default_rng(11)
    t = np.ldexp(g.integers(1, 1 << 12, size=4000).astype(np.float64), g.integers(-22, -3, size=4000))
    t = t[t <= 448.0].astype(np.float32)
    x = np.zeros((len(t), 16), dtype=np.float32)
    x[:, 0] = 6.0 * t
    assert np.array_equal(x[:, 0].astype(np.float64), 6.0 * t.astype(np.float64))  # exact
    _, sc = O.quantize_groups(x)
    ref = torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(sc, ref)


def test_hand_built_ties(golden_dir):
    for line in open(os.path.join(golden_dir, "e2m1_ties.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        v, want = line.split()
        x = np.zeros(16, dtype=np.float32)
        x[0] = 6.0                      # amax 6 -> scale code 0x38 (1.0)
        x[5] = np.float32(v)
        if abs(float(v)) > 6.0:
            x[0] = 6.0 if float(v) > 0 else -6.0
            x[1] = 6.0
        codes, sc = O.quantize_groups(x.reshape(1, 16))
        if abs(float(v)) <= 6.0:
            assert sc[0] == 0x38
        assert codes[0, 5] == int(want), (v, codes[0, 5], want)


def test_scale_midpoint_ties():
    # amax/6 exactly between two E4M3 values -> the even code
    for lo_code in (0x38, 0x39, 0x3A, 0x01, 0x02, 0x07, 0x7D):
        lo, hi = O.E4M3_POS[lo_code], O.E4M3_POS[lo_code + 1]
        x = np.zeros((1, 16), dtype=np.float32)
        x[0, 2] = np.float32(6.0 * (lo + hi) / 2)
        assert float(x[0, 2]) == 6.0 * (lo + hi) / 2
        _, sc = O.quantize_groups(x)
        want = lo_code if lo_code % 2 == 0 else lo_code + 1
        assert sc[0] == want


def test_saturation_and_zero_groups():
    x = np.array([[1e4] + [0.0] * 15], dtype=np.float32)
    codes, sc = O.quantize_groups(x)
    assert sc[0] == 0x7E and codes[0, 0] == 7
    # far beyond the range (up to the largest fp32): every value saturates to +-6 at scale 448
    for big in (1e30, -1e30, 3.4028235e38):
        x = np.full((1, 16), big, dtype=np.float32)
        x[0, 3] = -x[0, 3]
        codes, sc = O.quantize_groups(x)
        assert sc[0] == 0x7E
        want = np.where(np.signbit(x[0]), 15, 7)
        assert np.array_equal(codes[0], want), (big, codes)
        bc, bsc = _quantize_group_bruteforce(x[0])
        assert bsc == 0x7E and bc == want.tolist()
    # a huge value next to a small one: the small one is measured against scale 448
    x = np.zeros((1, 16), np.float32)
    x[0, 0], x[0, 1], x[0, 2] = 1e30, 100.0, 1000.0
    codes, _ = O.quantize_groups(x)
    assert codes[0, :3].tolist() == [7, 0, 4]             # 100/448 -> 0, 1000/448 ~ 2.23 -> 2
    z = np.zeros((1, 16), dtype=np.float32)
    codes, sc = O.quantize_groups(z)
    assert sc[0] == 0 and np.all(codes == 0)
    nz = -z
    codes, sc = O.quantize_groups(nz)
    assert sc[0] == 0 and np.all(codes == 8)
    # below half the smallest subnormal scale: scale 0, all values keep only their sign
    tiny = np.full((1, 16), 6.0 * 2.0 ** -10, dtype=np.float32)
    tiny[0, 1] = -tiny[0, 1]
    codes, sc = O.quantize_groups(tiny)
    assert sc[0] == 0 and codes[0, 0] == 0 and codes[0, 1] == 8


def test_idempotent_on_normal_scales_and_amax_on_code7():
    g = np.random.default_rng(3)
    x = g.standard_normal((2000, 16)).astype(np.float32)
    codes, sc = O.quantize_groups(x)
    assert np.all(sc >= 0x08)                                  # normal scales for N(0,1) data
    xq = O.e2m1_decode(codes) * O.E4M3_POS[sc][:, None]
    codes2, sc2 = O.quantize_groups(xq.astype(np.float32))
    assert np.array_equal(sc2, sc) and np.array_equal(codes2, codes)
    amax_pos = np.argmax(np.abs(x), axis=1)
    assert np.all((codes[np.arange(len(x)), amax_pos] & 7) == 7)


def test_error_bound():
    g = np.random.default_rng(5)
    x = (g.standard_normal((3000, 16)) * 10.0 ** g.uniform(-1, 2, size=(3000, 1))).astype(np.float32)
    codes, sc = O.quantize_groups(x)
    s = O.E4M3_POS[sc][:, None]
    xq = O.e2m1_decode(codes) * s
    ax = np.abs(x.astype(np.float64))
    # half the local spacing of the E2M1 grid around |x|/s, or saturation error above 6 s
    spacing = np.select([ax <= 2 * s, ax <= 4 * s], [0.5 * s, 1.0 * s], 2.0 * s)
    err = np.abs(x - xq)
    sat = ax > 6 * s
    assert np.all(err[~sat] <= spacing[~sat] / 2)
    # with a normal scale amax/s <= 6.375, so saturation costs at most 0.375 s
    normal = np.broadcast_to(sc[:, None] >= 0x08, x.shape)
    sbig = np.broadcast_to(s, x.shape)
    assert np.all(err[sat & normal] <= 0.375 * sbig[sat & normal])
    assert np.all(ax.max(axis=1)[sc >= 0x08] / s[sc >= 0x08, 0] <= 6.375)


def test_pack_layout_and_roundtrip():
    # channel c of group g gets a distinct, exactly representable value; check the nibble layout
    x = np.zeros((1, 512), dtype=np.float32)
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(512):
        x[0, c] = mags[c % 8] * (1 if (c // 8) % 2 == 0 else -1)
    for gi in range(32):
        x[0, 16 * gi + 7] = 6.0   # every group has amax 6 -> scale 1.0
    row = O.quantize_kv_fp4(x)[0]
    assert row.shape == (288,)
    assert np.all(row[256:] == 0x38)
    for c in range(512):
        nib = (row[c // 2] >> (4 * (c % 2))) & 0xF
        want = O.quantize_groups(x[:, (c // 16) * 16:(c // 16) * 16 + 16])[0][0, c % 16]
        assert nib == want
    assert np.array_equal(O.dequant_kv_fp4(row[None])[0], x[0].astype(np.float64))


def test_bf16_source_equals_fp32_source():
    g = np.random.default_rng(9)
    x = g.standard_normal((64, 512)).astype(np.float32)
    xb = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(O.quantize_kv_fp4(xb), O.quantize_kv_fp4(xb.astype(np.float64)))
