"""Helpers shared by the GPU parity tests, the smoke check and the benchmark.

Device inputs are built from the seeded generators in fp4_kv_cache_e2m1_amd.workloads; oracle
references are computed from the same generator output by oracle/ alone. Nothing here feeds a
GPU result into the oracle.
"""
from __future__ import annotations

import numpy as np
import torch

from fp4_kv_cache_e2m1_amd import workloads as W

# Tolerances (the hot path's stated bars).
SCORE_RTOL = 1e-3          # indexer scores, relative to max(|s|, sum |q*k|)
ATTN_TOL = 2e-3            # attention: max_d |o - o_ref| <= 2e-3 * ||o_ref||_2 per (row, head)
LSE_ATOL = 1e-3            # log-sum-exp, absolute (f16 probabilities: relative error of the sum ~2^-12)
SWAP_RTOL = 1e-6           # Top-K: an element may differ only if its score is within 1e-6 of the K-th


def dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def f64(bits: np.ndarray) -> np.ndarray:
    return W.bf16_bits_to_f32(bits).astype(np.float64)


def check_scores(gpu: np.ndarray, ref: np.ndarray, abs_dot: np.ndarray, mask: np.ndarray, what=""):
    """Scores within SCORE_RTOL of max(|ref|, sum |q*k|) on the masked entries."""
    g, r, a = gpu[mask].astype(np.float64), ref[mask].astype(np.float64), abs_dot[mask]
    err = np.abs(g - r)
    bound = SCORE_RTOL * np.maximum(np.abs(r), a)
    bad = err > bound
    assert not bad.any(), f"{what}: {bad.sum()} scores out of tolerance, worst err {err.max():.3g}"
    return float((err / np.maximum(np.abs(r), 1e-30)).max()) if err.size else 0.0


def check_attn(out: np.ndarray, ref: np.ndarray, lse=None, lse_ref=None, what=""):
    """out/ref [..., D]; per row max-abs error relative to the reference row's L2 norm."""
    o = out.reshape(-1, out.shape[-1]).astype(np.float64)
    r = ref.reshape(-1, ref.shape[-1]).astype(np.float64)
    nrm = np.linalg.norm(r, axis=1)
    err = np.abs(o - r).max(axis=1)
    zero = nrm == 0
    assert np.all(err[zero] == 0), f"{what}: rows with empty selection must be exactly 0"
    rel = err[~zero] / nrm[~zero]
    assert rel.size == 0 or rel.max() <= ATTN_TOL, f"{what}: attention rel err {rel.max():.3g} > {ATTN_TOL}"
    if lse is not None:
        l, lr = lse.reshape(-1).astype(np.float64), lse_ref.reshape(-1).astype(np.float64)
        inf = np.isinf(lr)
        assert np.array_equal(np.isinf(l), inf) and np.all(l[inf] == lr[inf]), f"{what}: lse -inf mismatch"
        d = np.abs(l[~inf] - lr[~inf])
        assert d.size == 0 or d.max() <= LSE_ATOL, f"{what}: lse err {d.max():.3g}"
    return float(rel.max()) if rel.size else 0.0


def compare_topk(gpu_idx: np.ndarray, ref_idx: np.ndarray, ref_score_of, what="") -> bool:
    """Top-K index sets: identical, or differing only among entries whose (oracle) score is within
    SWAP_RTOL of the oracle's K-th best. ref_score_of(p) -> fp32 oracle score of position p.
    Returns True when the sets are identical."""
    G = set(int(x) for x in gpu_idx if x >= 0)
    R = set(int(x) for x in ref_idx if x >= 0)
    assert len(G) == int((gpu_idx >= 0).sum()), f"{what}: duplicate positions in GPU Top-K"
    assert list(gpu_idx[gpu_idx >= 0]) == sorted(G), f"{what}: GPU Top-K not ascending"
    assert np.all(gpu_idx[len(G):] == -1), f"{what}: padding must follow the positions"
    if G == R:
        return True
    assert len(G) == len(R), f"{what}: Top-K sizes differ {len(G)} vs {len(R)}"
    kth = min(float(ref_score_of(p)) for p in R)
    for p in G ^ R:
        s = float(ref_score_of(p))
        assert abs(s - kth) <= SWAP_RTOL * abs(kth), f"{what}: position {p} (score {s}) vs K-th {kth}"
    return False


def kv_rows_device(wl: W.Workload, bs=None) -> tuple:
    """Generate every sequence's KV source on the host and quantize it on the device.
    Returns (rows [B, N, 288] uint8 on device)."""
    import fp4_kv_cache_e2m1_amd as P
    bs = range(wl.B) if bs is None else bs
    rows = torch.empty(wl.B, wl.N, P.row_bytes(wl.D), dtype=torch.uint8, device="cuda")
    for b in bs:
        src = torch.from_numpy(W.kv_source(wl, b)).to("cuda")
        P.quantize_kv_fp4(src, out=rows[b])
        del src
    return rows


def k_idx_device(wl: W.Workload) -> torch.Tensor:
    k = torch.empty(wl.B, wl.N, wl.Hk, wl.Di, dtype=torch.bfloat16, device="cuda")
    for b in range(wl.B):
        k[b] = dev_bf16(W.k_idx(wl, b))
    return k


def q_device(wl: W.Workload, layer: int, kind: str) -> torch.Tensor:
    gen = W.q_idx if kind == "q_idx" else W.q_main
    return torch.stack([dev_bf16(gen(wl, b, layer)) for b in range(wl.B)])
