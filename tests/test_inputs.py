"""The seeded synthetic inputs of the window and FP4-indexer benchmarks (CPU only): repeatable,
distinct per sequence and copy, and valid for the formats they feed (no NaN codes, scales in
their stated ranges)."""
import numpy as np

from fp4_kv_cache_e2m1_amd import workloads as W
from oracle import csa2_oracle as O


def test_window_rows_are_seeded_and_finite():
    wl = W.CONFIGS[2]
    c0, e0 = W.swa_window(wl, 0, 128)
    c0b, e0b = W.swa_window(wl, 0, 128)
    c1, _ = W.swa_window(wl, 1, 128)
    assert c0.shape == (128, wl.D) and e0.shape == (128,)
    assert np.array_equal(c0, c0b) and np.array_equal(e0, e0b) and not np.array_equal(c0, c1)
    assert not np.any((c0 & 0x7F) == 0x7F)                      # no E4M3 NaN codes
    assert e0.min() >= O.SWA_EXP_MIN and e0.max() <= O.SWA_EXP_MAX
    assert np.all(np.isfinite(O.dequant_swa_fp8(c0, e0)))


def test_mxfp4_rows_are_seeded_and_finite():
    wl = W.CONFIGS[2]
    C = wl.Hi * wl.Di
    r0 = W.mxfp4_rows(wl, 0, 300, C)
    assert r0.shape == (300, O.mxfp4_row_bytes(C))
    assert np.array_equal(r0, W.mxfp4_rows(wl, 0, 300, C))
    assert not np.array_equal(r0, W.mxfp4_rows(wl, 0, 300, C, copy=1))
    sc = r0[:, C // 2:]
    assert sc.min() >= 123 and sc.max() <= 129                   # 2^-4 .. 2^2
    assert np.all(np.isfinite(O.dequant_mxfp4(r0, C)))
