"""The C ABI library (CPU-side checks, no GPU needed).

The library must build for gfx950, load, and export every function include/csa2.h declares.
Argument, shape, workspace and shared-state validation happens on the host before any HIP call,
so those error paths are exercised here with null device pointers.
"""
import ctypes as C
import os
import re

import pytest

from fp4_kv_cache_e2m1_amd import _lib
from fp4_kv_cache_e2m1_amd._lib import LayerArgs, SharedIdx, SharedKV

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")

OK, E_ARG, E_SHAPE, E_STATE, E_WS, E_UNSUP = 0, 1, 2, 3, 4, 5
FAKE = 0x1000  # a 4 KiB-aligned non-null pointer value; validation fails before it is used


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        from fp4_kv_cache_e2m1_amd import build_lib
        build_lib.build(verbose=False)
    return _lib.lib()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function(L):
    declared = header_functions()
    assert len(declared) >= 12
    assert set(declared) == set(_lib.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def test_status_strings(L):
    for code in range(7):
        assert L.csa2_status_string(code)
    assert b"state" in L.csa2_status_string(E_STATE)


def test_quantize_validation(L):
    assert L.csa2_quantize_kv_fp4(None, 0, -1, 512, None, None) == E_ARG
    assert L.csa2_quantize_kv_fp4(None, 7, 4, 512, None, None) == E_ARG
    assert L.csa2_quantize_kv_fp4(None, 0, 4, 500, None, None) == E_SHAPE
    assert L.csa2_quantize_kv_fp4(None, 0, 4, 8192, None, None) == E_SHAPE
    assert L.csa2_quantize_kv_fp4(None, 0, 4, 512, None, None) == E_ARG
    assert L.csa2_quantize_kv_fp4(FAKE + 4, 0, 4, 512, FAKE, None) == E_ARG   # misaligned src
    assert L.csa2_quantize_kv_fp4(None, 0, 0, 512, None, None) == OK          # empty: nothing to do
    assert L.csa2_dequant_kv_fp4(None, 3, 512, None, None) == E_ARG
    assert L.csa2_dequant_kv_fp4(None, 3, 96, None, None) == E_SHAPE


def test_index_scores_validation(L):
    f = L.csa2_index_scores
    # q, k, B, T, Hi, Hk, Di, n_max, n_vis, cand, P, scores, block_max, block, stream
    assert f(None, None, -1, 1, 8, 8, 64, 10, None, None, 0, None, None, 8, None) == E_ARG
    assert f(None, None, 1, 1, 8, 4, 64, 10, None, None, 0, None, None, 8, None) == E_SHAPE   # Hk not in {1, Hi}
    assert f(None, None, 1, 1, 8, 8, 12, 10, None, None, 0, None, None, 8, None) == E_SHAPE   # Di % 8
    assert f(None, None, 1, 1, 32, 32, 64, 10, None, None, 0, None, None, 8, None) == E_SHAPE  # Hi*Di > 1024
    assert f(None, None, 0, 1, 32, 1, 128, 10, None, None, 0, None, None, 8, None) == OK       # shared key, 32 x 128
    assert f(None, None, 1, 1, 128, 1, 128, 10, None, None, 0, None, None, 8, None) == E_SHAPE  # Hi*Di > 8192
    assert f(None, None, 1, 1, 8, 8, 64, 10, None, FAKE, 4, None, FAKE, 8, None) == E_UNSUP   # block max on pool
    assert f(None, None, 1, 1, 8, 8, 64, 10, None, None, 0, None, FAKE, 4, None) == E_UNSUP   # block != 8
    assert f(None, None, 1, 1, 8, 8, 64, 10, None, None, 0, None, None, 8, None) == E_ARG     # null tensors
    assert f(None, None, 0, 1, 8, 8, 64, 10, None, None, 0, None, None, 8, None) == OK        # empty
    # 192-channel key rows: the streaming kernel has no such instantiation (decode, pool, block max)
    assert f(FAKE, FAKE, 1, 1, 3, 3, 64, 10, None, None, 0, FAKE, None, 8, None) == E_SHAPE
    assert f(FAKE, FAKE, 1, 64, 3, 3, 64, 10, None, FAKE, 4, FAKE, None, 8, None) == E_SHAPE
    assert f(FAKE, FAKE, 1, 64, 3, 3, 64, 10, None, None, 0, FAKE, FAKE, 8, None) == E_SHAPE
    # ... but the MFMA prefill form takes them
    assert f(None, None, 0, 64, 3, 3, 64, 10, None, None, 0, None, None, 8, None) == OK


def test_prefill_visibility_validation(L):
    f = L.csa2_prefill_visibility
    # p0, B, T, ratio, n_max, n_vis, stream
    assert f(FAKE, 1, 4, 0, 10, FAKE, None) == E_ARG        # ratio must be positive
    assert f(FAKE, -1, 4, 4, 10, FAKE, None) == E_ARG
    assert f(None, 1, 4, 4, 10, None, None) == E_ARG
    assert f(None, 0, 4, 4, 10, None, None) == OK           # empty
    assert f(FAKE, 65536, 65536, 4, 10, FAKE, None) == E_SHAPE


def test_topk_and_pool_validation(L):
    assert L.csa2_topk(None, -1, 10, None, None, 4, None, None, 0, None) == E_ARG
    assert L.csa2_topk(None, 2, 10, None, None, 5000, None, None, 0, None) == E_SHAPE
    assert L.csa2_topk(None, 2, 10, None, None, 4, None, None, 0, None) == E_ARG
    assert L.csa2_topk(None, 0, 10, None, None, 4, None, None, 0, None) == OK
    need = L.csa2_topk_workspace_size(4, 262144, 512)
    assert need > 0
    assert L.csa2_topk(FAKE, 4, 262144, None, None, 512, FAKE, None, 0, None) == E_WS
    assert L.csa2_topk(FAKE, 4, 262144, None, None, 512, FAKE, FAKE, need - 1, None) == E_WS
    assert L.csa2_topk_workspace_size(32, 16384, 512) == 0       # one segment per row: no scratch
    assert L.csa2_hier_pool(None, 2, 10, None, 0, 4, None, None, 0, None) == E_ARG
    assert L.csa2_hier_pool(None, 2, 10, None, 128, 4, None, None, 0, None) == E_SHAPE
    assert L.csa2_hier_pool(None, 2, 10, None, 8, 4, None, None, 0, None) == E_ARG


def test_sparse_attn_validation(L):
    f = L.csa2_sparse_attn
    # q, rows, n_max, idx, B, T, H, D, K, scale, out, lse, ws, ws_bytes, stream
    assert f(None, None, 10, None, 1, 1, 64, 256, 8, 1.0, None, None, None, 0, None) == E_SHAPE
    assert f(None, None, 10, None, 1, 1, 24, 512, 8, 1.0, None, None, None, 0, None) == E_SHAPE
    assert f(None, None, 10, None, 1, 1, 96, 512, 8, 1.0, None, None, None, 0, None) == E_SHAPE
    assert f(None, None, 10, None, 1, 1, 64, 512, 8, 1.0, None, None, None, 0, None) == E_ARG
    assert f(FAKE, FAKE + 8, 10, FAKE, 1, 1, 64, 512, 8, 1.0, FAKE, None, None, 0, None) == E_ARG  # misaligned
    assert f(FAKE, FAKE, 10, FAKE, 1, 1, 64, 512, 4097, 1.0, FAKE, None, FAKE, 1 << 30, None) == E_SHAPE
    assert L.csa2_sparse_attn_workspace_size(1, 1, 64, 512, 4097) == 0
    need = L.csa2_sparse_attn_workspace_size(32, 1, 64, 512, 512)
    assert need > 0                                                # decode is split over the entries
    assert f(FAKE, FAKE, 10, FAKE, 32, 1, 64, 512, 512, 1.0, FAKE, None, None, 0, None) == E_WS


def test_index_scores_mxfp4_pool_modes(L):
    f = L.csa2_index_scores_mxfp4
    # block max only in flat mode, 8 wide
    assert f(FAKE, FAKE, 1, 1, 8, 8, 64, 10, None, FAKE, 4, FAKE, FAKE, 8, None) == E_UNSUP
    assert f(FAKE, FAKE, 1, 1, 32, 1, 128, 10, None, FAKE, 4, FAKE, FAKE, 8, None) == E_UNSUP
    assert f(FAKE, FAKE, 1, 1, 32, 1, 128, 10, None, None, 0, FAKE, FAKE, 4, None) == E_UNSUP
    assert f(FAKE, FAKE, 1, 1, 32, 1, 128, 10, None, FAKE, -1, FAKE, None, 8, None) == E_ARG


def test_index_scores_mxfp4_validation(L):
    f = L.csa2_index_scores_mxfp4
    # q_rows, k_rows, B, T, Hi, Hk, Di, n_max, n_vis, cand, P, scores, block_max, block, stream
    assert f(FAKE, FAKE, 1, 1, 2, 2, 64, 10, None, None, 0, FAKE, None, 8, None) == E_SHAPE      # 128 channels per head pair
    assert f(FAKE, FAKE, 1, 1, 8, 8, 128, 10, None, None, 0, FAKE, None, 8, None) == E_SHAPE     # 1024 channels
    assert f(FAKE, FAKE, 1, 1, 8, 4, 64, 10, None, None, 0, FAKE, None, 8, None) == E_SHAPE      # Hk neither Hi nor 1
    assert f(FAKE, FAKE, 1, 1, 65, 1, 128, 10, None, None, 0, FAKE, None, 8, None) == E_SHAPE    # too many query heads
    assert f(FAKE, FAKE, 1, 1, 8, 1, 64, 10, None, None, 0, FAKE, None, 8, None) == E_SHAPE      # shared keys are 128 wide
    assert f(FAKE, FAKE, -1, 1, 8, 8, 64, 10, None, None, 0, FAKE, None, 8, None) == E_ARG
    assert f(None, FAKE, 1, 1, 8, 8, 64, 10, None, None, 0, FAKE, None, 8, None) == E_ARG
    assert f(FAKE + 4, FAKE, 1, 1, 8, 8, 64, 10, None, None, 0, FAKE, None, 8, None) == E_ARG    # misaligned rows
    assert f(None, None, 0, 1, 8, 8, 64, 10, None, None, 0, None, None, 8, None) == 0            # nothing to do
    assert f(None, None, 1, 1, 32, 1, 128, 0, None, None, 0, None, None, 8, None) == 0


def test_sparse_attn_swa_validation(L):
    f = L.csa2_sparse_attn_swa
    # q, rows, n_max, idx, B, H, D, K, swa_codes, swa_exp, n_win, W, scale, out, lse, ws, ws_bytes, stream
    assert f(None, None, 10, None, 1, 64, 256, 8, None, None, None, 128, 1.0, None, None, None, 0, None) == E_SHAPE
    assert f(None, None, 10, None, 1, 24, 512, 8, None, None, None, 128, 1.0, None, None, None, 0, None) == E_SHAPE
    assert f(FAKE, FAKE, 10, FAKE, 1, 64, 512, 8, FAKE, FAKE, FAKE, 129, 1.0, FAKE, None, FAKE, 1 << 30,
             None) == E_SHAPE                                      # window above 128 rows
    assert f(FAKE, FAKE, 10, FAKE, 1, 64, 512, 8, FAKE, FAKE, FAKE, -1, 1.0, FAKE, None, FAKE, 1 << 30,
             None) == E_ARG
    assert f(FAKE, FAKE, 10, FAKE, 1, 64, 512, 4097, FAKE, FAKE, FAKE, 128, 1.0, FAKE, None, FAKE, 1 << 30,
             None) == E_SHAPE                                      # K above the Top-K limit
    assert f(FAKE, FAKE, 10, FAKE, 1, 64, 512, 8, None, FAKE, FAKE, 128, 1.0, FAKE, None, FAKE, 1 << 30,
             None) == E_ARG                                        # window rows missing
    assert f(FAKE, FAKE, 10, FAKE, 1, 64, 512, 8, FAKE, FAKE, None, 128, 1.0, FAKE, None, FAKE, 1 << 30,
             None) == E_ARG                                        # n_win missing
    assert f(FAKE, FAKE, 10, FAKE, 1, 64, 512, 8, FAKE + 8, FAKE, FAKE, 128, 1.0, FAKE, None, FAKE, 1 << 30,
             None) == E_ARG                                        # misaligned window rows
    need = L.csa2_sparse_attn_swa_workspace_size(32, 64, 512, 512)
    assert need >= L.csa2_sparse_attn_workspace_size(32, 1, 64, 512, 512) + 2 * 32 * 64 * (512 * 4 + 8)
    assert L.csa2_sparse_attn_swa_workspace_size(32, 64, 512, 0) > 0   # the window's partials
    assert f(FAKE, FAKE, 10, FAKE, 32, 64, 512, 512, FAKE, FAKE, FAKE, 128, 1.0, FAKE, None, FAKE, need - 1,
             None) == E_WS
    assert f(FAKE, FAKE, 10, FAKE, 0, 64, 512, 512, None, None, None, 128, 1.0, None, None, None, 0, None) == 0


def _layer(T=1, H=64, Hi=8, K=512, pool_blocks=0, use_pool=0, block=8):
    kv = SharedKV(rows=FAKE, k_idx=FAKE, n_vis=None, B=4, n_max=4096, D=512, Hk=8, Di=64, valid=0)
    idx = SharedIdx(topk=FAKE, K=K, pool=FAKE if pool_blocks else None, P=pool_blocks * block,
                    topk_valid=0, pool_valid=0)
    a = LayerArgs(q=FAKE, q_idx=FAKE, T=T, H=H, Hi=Hi, sm_scale=0.04, use_pool=use_pool,
                  pool_blocks=pool_blocks, block=block, out=FAKE, lse=None, ws=None, ws_bytes=0)
    return a, kv, idx


def test_layer_step_state_rules(L):
    a, kv, idx = _layer()
    # Reindex / Reuse before a Full layer published the cache
    assert L.csa2_layer_step(1, C.byref(a), C.byref(kv), C.byref(idx), None) == E_STATE
    assert L.csa2_layer_step(2, C.byref(a), C.byref(kv), C.byref(idx), None) == E_STATE
    kv.valid = 1
    # Reuse still needs a Top-K
    assert L.csa2_layer_step(2, C.byref(a), C.byref(kv), C.byref(idx), None) == E_STATE
    # Full without workspace
    kv.valid = 0
    assert L.csa2_layer_step(0, C.byref(a), C.byref(kv), C.byref(idx), None) == E_WS
    assert L.csa2_layer_step(7, C.byref(a), C.byref(kv), C.byref(idx), None) == E_ARG
    n = C.c_size_t(0)
    assert L.csa2_layer_workspace_size(0, C.byref(a), C.byref(kv), C.byref(idx), C.byref(n)) == OK
    assert n.value >= 4 * 4096 * 4                                 # at least the score rows
    # a workspace of the right size that is not 256-byte aligned
    a.ws, a.ws_bytes = FAKE + 64, n.value
    assert L.csa2_layer_step(0, C.byref(a), C.byref(kv), C.byref(idx), None) == E_WS
    a.ws, a.ws_bytes = None, 0
    assert L.csa2_layer_workspace_size(2, C.byref(a), C.byref(kv), C.byref(idx), C.byref(n)) == OK
    # a key-row width the streaming indexer has no kernel for (3 heads x 64)
    kv.Hk, a.Hi = 3, 3
    assert L.csa2_layer_workspace_size(0, C.byref(a), C.byref(kv), C.byref(idx), C.byref(n)) == E_SHAPE


def test_layer_step_noalloc_limit(L):
    """The no-allocation layer step rejects a layer whose scratch exceeds its fixed array, before
    touching the device (a 4096-token prefill chunk over 33792 entries needs 528 MiB)."""
    a, kv, idx = _layer(T=4096, K=1024)
    kv.B, kv.n_max = 1, 33792
    n = C.c_size_t(0)
    assert L.csa2_layer_workspace_size(0, C.byref(a), C.byref(kv), C.byref(idx), C.byref(n)) == OK
    assert n.value > 64 << 20
    assert L.csa2_layer_step_noalloc(0, C.byref(a), C.byref(kv), C.byref(idx), None) == E_WS
    # the same state rules as csa2_layer_step
    a2, kv2, idx2 = _layer()
    assert L.csa2_layer_step_noalloc(1, C.byref(a2), C.byref(kv2), C.byref(idx2), None) == E_STATE
    assert L.csa2_layer_step_noalloc(7, C.byref(a2), C.byref(kv2), C.byref(idx2), None) == E_ARG


def test_layer_step_pool_rules(L):
    a, kv, idx = _layer(pool_blocks=128, use_pool=1)
    n = C.c_size_t(0)
    assert L.csa2_layer_workspace_size(0, C.byref(a), C.byref(kv), C.byref(idx), C.byref(n)) == OK
    a2, kv2, idx2 = _layer(pool_blocks=32, use_pool=1)               # pool (256) smaller than K (512)
    assert L.csa2_layer_workspace_size(0, C.byref(a2), C.byref(kv2), C.byref(idx2), C.byref(n)) == E_SHAPE
    a3, kv3, idx3 = _layer(pool_blocks=128, use_pool=1, block=4)     # fused block max is 8 wide
    assert L.csa2_layer_workspace_size(0, C.byref(a3), C.byref(kv3), C.byref(idx3), C.byref(n)) == E_UNSUP
    idx.P = 100                                                      # capacity must equal blocks * 8
    assert L.csa2_layer_workspace_size(0, C.byref(a), C.byref(kv), C.byref(idx), C.byref(n)) == E_SHAPE


def test_layer_step_window_rules(L):
    n = C.c_size_t(0)
    a, kv, idx = _layer()
    assert L.csa2_layer_workspace_size(0, C.byref(a), C.byref(kv), C.byref(idx), C.byref(n)) == OK
    plain = n.value
    a.swa_codes, a.swa_exp, a.swa_n, a.swa_W = FAKE, FAKE, FAKE, 128
    assert L.csa2_layer_workspace_size(0, C.byref(a), C.byref(kv), C.byref(idx), C.byref(n)) == OK
    assert n.value > plain                                          # the window's partial slots
    a.swa_W = 129
    assert L.csa2_layer_workspace_size(0, C.byref(a), C.byref(kv), C.byref(idx), C.byref(n)) == E_SHAPE
    a.swa_W = 128
    a.swa_exp = None                                                # exponents missing
    kv.valid, idx.topk_valid = 1, 1
    assert L.csa2_layer_step(2, C.byref(a), C.byref(kv), C.byref(idx), None) == E_ARG
    a2, kv2, idx2 = _layer(T=2)                                     # prefill: the prefill window sizing
    assert L.csa2_layer_workspace_size(0, C.byref(a2), C.byref(kv2), C.byref(idx2), C.byref(n)) == OK
    plain2 = n.value
    a2.swa_codes, a2.swa_exp, a2.swa_n, a2.swa_W = FAKE, FAKE, FAKE, 128
    assert L.csa2_layer_workspace_size(0, C.byref(a2), C.byref(kv2), C.byref(idx2), C.byref(n)) == OK
    assert n.value > plain2


def test_layer_step_fp4_indexer_rules(L):
    n = C.c_size_t(0)
    a, kv, idx = _layer()
    kv.k_mx = FAKE
    assert L.csa2_layer_workspace_size(0, C.byref(a), C.byref(kv), C.byref(idx), C.byref(n)) == OK
    assert L.csa2_layer_step(0, C.byref(a), C.byref(kv), C.byref(idx), None) == E_ARG   # no q_idx_mx
    a.Hi = 4                                                        # one key head per index head
    assert L.csa2_layer_workspace_size(0, C.byref(a), C.byref(kv), C.byref(idx), C.byref(n)) == E_SHAPE
    a2, kv2, idx2 = _layer(pool_blocks=128, use_pool=1)
    kv2.k_mx = FAKE
    assert L.csa2_layer_workspace_size(0, C.byref(a2), C.byref(kv2), C.byref(idx2), C.byref(n)) == OK
    kv2.Hk, kv2.Di, a2.Hi = 1, 128, 32                              # the shared-key form too
    assert L.csa2_layer_workspace_size(0, C.byref(a2), C.byref(kv2), C.byref(idx2), C.byref(n)) == OK


def test_sparse_attn_swa_prefill_validation(L):
    f = L.csa2_sparse_attn_swa_prefill
    # q, rows, n_max, idx, B, T, H, D, K, swa_codes, swa_exp, n_win, W, scale, out, lse, ws, ws_bytes, stream
    assert f(FAKE, FAKE, 10, FAKE, 1, 4, 64, 256, 8, FAKE, FAKE, FAKE, 128, 1.0, FAKE, None, FAKE, 1 << 30,
             None) == E_SHAPE
    assert f(FAKE, FAKE, 10, FAKE, 1, 4, 64, 512, 8, FAKE, FAKE, FAKE, 129, 1.0, FAKE, None, FAKE, 1 << 30,
             None) == E_SHAPE
    assert f(FAKE, FAKE, 10, FAKE, 1, 4, 64, 512, 8, FAKE, FAKE, None, 128, 1.0, FAKE, None, FAKE, 1 << 30,
             None) == E_ARG
    # 64-head groups with one split of selected entries: the window runs inside that pass, no scratch
    assert L.csa2_sparse_attn_swa_prefill_workspace_size(1, 600, 64, 512, 64) == 0
    assert L.csa2_sparse_attn_swa_prefill_workspace_size(1, 600, 128, 512, 1024) == 0
    # 32 heads: the sparse slot and one window slot, merged by a combine pass
    need = L.csa2_sparse_attn_swa_prefill_workspace_size(1, 600, 32, 512, 64)
    assert need >= 2 * 600 * 32 * 512 * 4
    assert f(FAKE, FAKE, 10, FAKE, 1, 600, 32, 512, 64, FAKE, FAKE, FAKE, 128, 1.0, FAKE, None, FAKE, need - 1,
             None) == E_WS
    assert f(FAKE, FAKE, 10, FAKE, 1, 600, 32, 512, 64, FAKE, FAKE, FAKE, 128, 1.0, FAKE, None, None, need,
             None) == E_WS                                          # missing
    assert f(FAKE, FAKE, 10, FAKE, 1, 600, 32, 512, 64, FAKE, FAKE, FAKE, 128, 1.0, FAKE, None, FAKE + 16, need,
             None) == E_WS                                          # workspace not 256-byte aligned
    assert f(None, None, 10, None, 1, 0, 64, 512, 8, None, None, None, 128, 1.0, None, None, None, 0, None) == 0


def test_compress_kv_validation(L):
    f = L.csa2_compress_kv
    # c, z, B, n_tok, D, ratio, entry0, n_max, rows, w_t, Hk, Di, k_idx, entries, stream
    assert f(FAKE, FAKE, 1, 8, 256, 4, FAKE, 64, FAKE, FAKE, 8, 64, FAKE, None, None) == E_SHAPE   # D
    assert f(FAKE, FAKE, 1, 9, 512, 3, FAKE, 64, FAKE, FAKE, 8, 64, FAKE, None, None) == E_SHAPE   # ratio 3
    assert f(FAKE, FAKE, 1, 6, 512, 4, FAKE, 64, FAKE, FAKE, 8, 64, FAKE, None, None) == E_SHAPE   # n_tok % ratio
    assert f(FAKE, FAKE, 1, 8, 512, 4, FAKE, 64, FAKE, FAKE, 3, 32, FAKE, None, None) == E_SHAPE   # 96 key channels
    assert f(FAKE, FAKE, 1, 8, 512, 4, FAKE, 64, FAKE, FAKE, 8, 256, FAKE, None, None) == E_SHAPE  # 2048 > 1024
    assert f(FAKE, FAKE, 1, 8, 512, 4, FAKE, 64, FAKE, None, 8, 64, FAKE, None, None) == E_ARG     # weight without keys
    assert f(FAKE, FAKE, 1, 8, 512, 4, FAKE, 64, FAKE, FAKE, 8, 64, None, None, None) == E_ARG     # keys without weight
    assert f(None, FAKE, 1, 8, 512, 4, FAKE, 64, FAKE, None, 8, 64, None, None, None) == E_ARG     # no c
    assert f(FAKE, FAKE, 1, 8, 512, 4, None, 64, FAKE, None, 8, 64, None, None, None) == E_ARG     # no entry0
    assert f(FAKE + 8, FAKE, 1, 8, 512, 4, FAKE, 64, FAKE, None, 8, 64, None, None, None) == E_ARG  # c misaligned
    assert f(FAKE, FAKE, 1, 8, 512, 0, FAKE, 64, FAKE, None, 8, 64, None, None, None) == E_ARG     # ratio 0
    assert f(FAKE, FAKE, -1, 8, 512, 4, FAKE, 64, FAKE, None, 8, 64, None, None, None) == E_ARG    # B < 0
    # nothing to do: no call is made
    assert f(None, None, 0, 8, 512, 4, None, 64, None, None, 8, 64, None, None, None) == OK
    assert f(None, None, 2, 0, 512, 4, None, 64, None, None, 8, 64, None, None, None) == OK
