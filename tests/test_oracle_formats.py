"""Pins of the oracle's format decoders and layout (CPU only).

The decoders are checked against values fixed outside the oracle: the OCP E2M1 table (golden
file), torch's own float8_e4m3fn decoder for all 256 E4M3 codes, and the constants the model
pages print (448, 6, 2688, 890 bytes/token).
"""
import os

import numpy as np
import pytest
import torch

from oracle import csa2_oracle as O


def _read_pairs(path):
    out = []
    for line in open(path):
        line = line.split("#")[0].strip()
        if line:
            a, b = line.split()[:2]
            out.append((a, b))
    return out


def _constants(golden_dir):
    return {k: int(v) for k, v in _read_pairs(os.path.join(golden_dir, "format_constants.txt"))}


def test_e2m1_table_matches_ocp(golden_dir):
    pairs = _read_pairs(os.path.join(golden_dir, "e2m1_values.txt"))
    assert len(pairs) == 16
    codes = np.array([int(c) for c, _ in pairs])
    want = np.array([float(v) for _, v in pairs])
    got = O.e2m1_decode(codes)
    assert np.array_equal(got, want)
    # sign of zero: code 8 is -0
    assert np.signbit(got[8]) and not np.signbit(got[0])


def test_e4m3_all_256_codes_match_torch():
    codes = np.arange(256)
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_page_constants(golden_dir):
    c = _constants(golden_dir)
    assert O.e4m3_decode(0x7E) == c["e4m3_max"]
    assert np.nanmax(O.e4m3_decode(np.arange(256))) == c["e4m3_max"]
    assert O.E2M1_MAGS.max() == c["e2m1_max"]
    assert O.E2M1_MAGS.max() * O.E4M3_POS.max() == c["fp4_range_max"]
    # the largest value a packed entry can hold dequantizes to exactly 2688
    x = np.zeros((1, 512), dtype=np.float32)
    x[0, 3] = 2688.0
    assert O.dequant_kv_fp4(O.quantize_kv_fp4(x))[0, 3] == c["fp4_range_max"]
    # E4M3 codes 0x00..0x7E are the finite non-negative values, strictly increasing
    assert len(O.E4M3_POS) == 127 and np.all(np.diff(O.E4M3_POS) > 0)
    assert O.E4M3_POS[1] == 2.0 ** -9 and O.E4M3_POS[0x38] == 1.0 and O.E4M3_POS[0x08] == 2.0 ** -6


def test_row_bytes_and_890_bytes_per_token(golden_dir):
    c = _constants(golden_dir)
    assert O.row_bytes(c["latent_channels"]) == c["row_bytes"]
    assert O.quantize_kv_fp4(np.ones((3, 512), np.float32)).shape == (3, c["row_bytes"])
    # Reconciliation of the pages' 890 B/token: per Full layer the cache holds one 288-byte
    # main-KV entry plus one 128-channel MXFP4 indexer key (64 B of codes + 4 E8M0 scales).
    # The encoder has 3 Full layers at compression 2, the decoder one Full layer at ratio 1
    # (walkthrough 三(二)1). 3 * 356 / 2 + 356 = 890.
    per_entry = O.row_bytes(512) + (128 // 2 + 128 // 32)
    assert 3 * per_entry / 2 + per_entry == c["global_kv_bytes_per_token"]


def test_hsi_pool_arithmetic(golden_dir):
    c = _constants(golden_dir)
    assert c["hsi_max_blocks"] * c["hsi_block_positions"] == c["hsi_max_pool"]
    # the oracle's pool has blocks x 8 slots
    s = np.arange(64, dtype=np.float32)[None, :]
    pool = O.hier_pool(O.block_max(s, [64]), [64], n_sel_blocks=3)
    assert pool.shape == (1, 3 * c["hsi_block_positions"])


def test_dequant_values_exact_in_bf16_and_f16():
    # every product E2M1 x E4M3 (finite, non-negative scale) is exact in bf16 and in f16
    vals = (O.E2M1_MAGS[:, None] * O.E4M3_POS[None, :]).reshape(-1)
    t = torch.from_numpy(vals)
    assert torch.equal(t.to(torch.bfloat16).to(torch.float64), t)
    assert torch.equal(t.to(torch.float16).to(torch.float64), t)
