"""Pins of the oracle's sliding-window branch (O12): the FP8 row format against torch's E4M3
decode and a brute-force nearest-code search, and the joined attention against dense attention
(torch scaled_dot_product_attention in fp64) over the concatenated rows."""
import numpy as np
import pytest
import torch

from oracle import csa2_oracle as O


def test_swa_dequant_exhaustive():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for e in (O.SWA_EXP_MIN, -6, 0, O.SWA_EXP_MAX):
        got = O.dequant_swa_fp8(codes[None], np.array([e], np.int8))[0]
        finite = ~np.isnan(ref)
        assert np.array_equal(got[finite], ref[finite] * 2.0 ** e)
        assert np.all(np.isnan(got[~finite]))
        # every finite value is exact in f16 at the allowed exponents (the GPU computes in f16)
        assert np.array_equal(got[finite].astype(np.float16).astype(np.float64), got[finite])


def test_swa_quantize_brute_force():
    g = np.random.default_rng(11)
    x = (g.standard_normal((40, 512)) * 10.0 ** g.uniform(-3, 2, size=(40, 1))).astype(np.float32)
    x[0] = 0.0
    x[1, :5] = [448.0, -448.0, 0.0, -0.0, 1.0]
    x[2] = np.float32(3.0e3)            # beyond 448 * 2^7: saturates at the largest exponent
    codes, exps = O.quantize_swa_fp8(x)
    table = O.e4m3_decode(np.arange(256))
    for r in range(x.shape[0]):
        e = int(exps[r])
        amax = float(np.abs(x[r]).max())
        if 0 < amax <= 448.0 * 2.0 ** O.SWA_EXP_MAX and e > O.SWA_EXP_MIN:
            assert 448.0 * 2.0 ** (e - 1) < amax <= 448.0 * 2.0 ** e
        y = x[r].astype(np.float64) * 2.0 ** -e
        for i in range(0, 512, 7):
            cands = [c for c in range(256) if not np.isnan(table[c]) and (c >> 7) == int(np.signbit(x[r, i]))]
            d = [abs(table[c] - y[i]) for c in cands]
            best = min(d)
            want = min(c for c, dd in zip(cands, d) if dd == best and ((c & 0x7F) % 2 == 0 or
                                                                     d.count(best) == 1))
            assert codes[r, i] == want, (r, i, x[r, i], e)


def test_swa_roundtrip_idempotent():
    g = np.random.default_rng(12)
    x = g.standard_normal((16, 512)).astype(np.float32)
    c1, e1 = O.quantize_swa_fp8(x)
    v1 = O.dequant_swa_fp8(c1, e1)
    c2, e2 = O.quantize_swa_fp8(v1.astype(np.float32))
    # the values survive a second quantization exactly (a row whose maximum rounded down to
    # 448 * 2^(e-1) is then stored with the next smaller exponent)
    assert np.array_equal(O.dequant_swa_fp8(c2, e2), v1)


def _dense(q, x, scale):
    qt = torch.from_numpy(q)[None].transpose(0, 1)          # [H, 1, D]
    xt = torch.from_numpy(x)[None].expand(q.shape[0], -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, xt, xt, scale=scale)
    return o[:, 0].numpy()


@pytest.mark.parametrize("n_sel,n_win", [(0, 37), (50, 0), (50, 128), (1, 1)])
def test_swa_attention_is_dense_attention_over_the_union(n_sel, n_win):
    g = np.random.default_rng(100 + n_sel + n_win)
    H, D, N, W = 16, 512, 300, 128
    kv = g.standard_normal((N, D))
    win_rows = g.standard_normal((1, W, D))
    q = g.standard_normal((1, H, D))
    idx = np.full((1, 64), -1, np.int64)
    idx[0, :n_sel] = g.choice(N, size=n_sel, replace=False)
    scale = 1 / np.sqrt(D)
    out, lse = O.sparse_attn_swa(q, kv, idx, win_rows, [n_win], scale)
    x = np.concatenate([kv[idx[0, :n_sel]], win_rows[0, :n_win]], axis=0)
    ref = _dense(q[0], x, scale)
    assert np.allclose(out[0], ref, rtol=0, atol=1e-5)
    logits = scale * q[0] @ x.T
    assert np.allclose(lse[0], np.log(np.exp(logits).sum(axis=1)), atol=1e-5)
    if n_win == 0:
        o2, l2 = O.sparse_attn(q, kv, idx, scale)
        assert np.array_equal(out, o2) and np.array_equal(lse, l2)


def test_swa_attention_empty_union():
    q = np.ones((1, 16, 512))
    out, lse = O.sparse_attn_swa(q, np.zeros((4, 512)), np.full((1, 8), -1), np.zeros((1, 128, 512)), [0], 0.1)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_layer_step_with_window_is_union_attention():
    """O11 with a window attends over the layer's own selection joined with the window (O12c);
    an empty window gives the plain layer."""
    g = np.random.default_rng(21)
    N, H, D, Wn = 200, 4, 512, 16
    kv = O.dequant_kv_fp4(O.quantize_kv_fp4(g.standard_normal((N, D)).astype(np.float32)))
    win = O.dequant_swa_fp8(*O.quantize_swa_fp8(g.standard_normal((Wn, D)).astype(np.float32)))[None]
    q = g.standard_normal((1, H, D))
    qi = g.standard_normal((1, 2, 64))
    ki = g.standard_normal((N, 2, 64))
    base = O.layer_step(O.FULL, q=q, kv_deq=kv, k_idx=ki, q_idx=qi, n_vis=[N], k=32)
    with_w = O.layer_step(O.FULL, q=q, kv_deq=kv, k_idx=ki, q_idx=qi, n_vis=[N], k=32, win=win, n_win=[Wn])
    assert np.array_equal(with_w["topk"], base["topk"])
    o, l = O.sparse_attn_swa(q, kv, base["topk"], win, [Wn], 1.0 / np.sqrt(512.0))
    assert np.array_equal(with_w["out"], o) and np.array_equal(with_w["lse"], l)
    empty = O.layer_step(O.FULL, q=q, kv_deq=kv, k_idx=ki, q_idx=qi, n_vis=[N], k=32, win=win, n_win=[0])
    assert np.allclose(empty["out"], base["out"], rtol=1e-6, atol=1e-6)


def test_prefill_windows_end_at_the_query_token():
    """Each query's window is its last n tokens up to and including its own (buffer row i holds
    token p0 - W + 1 + i); tokens before the sequence start are never taken."""
    W, T, p0 = 8, 12, 3
    tokens = np.arange(p0 - W + 1, p0 + T)[:, None].astype(np.float64)   # buffer rows = token ids
    n_win = [min(W, p0 + t + 1) for t in range(T)]
    win = O.prefill_windows(tokens, n_win, W)
    for t in range(T):
        p = p0 + t
        n = n_win[t]
        assert list(win[t, :n, 0]) == list(range(p - n + 1, p + 1))
        assert min(win[t, :n, 0]) >= 0
        assert np.all(win[t, n:] == 0)
