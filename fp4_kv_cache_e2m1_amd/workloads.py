"""Seeded synthetic workloads for the CSA2 hot path.

This module only draws random inputs and describes shapes. It holds none of the method's
arithmetic (no quantization, scoring, selection or attention), so both the HIP path and the CPU
oracle can be fed from it without sharing any of the computation.

Recipe: every tensor of every sequence comes from its own numpy PCG64 stream, seeded with
(1000 * config + tensor id, sequence index [, layer]), so one sequence can be regenerated without
drawing the others. Values are standard normal fp32; bf16 tensors are the round-to-nearest-even
bf16 of those fp32 draws. The five shapes follow the decode and prefill workloads the model
pages describe (512-channel latent, 64 query heads of dim 512, Top-K 512, candidate blocks of
8 positions), scaled as listed in `CONFIGS`.
"""

from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import numpy as np
import torch

FULL, REINDEX, REUSE = 0, 1, 2

# tensor ids inside a config's seed space
TID_KV, TID_KIDX, TID_QIDX, TID_Q, TID_PLANT, TID_SWA, TID_MXFP4 = 1, 2, 3, 4, 5, 6, 7
TID_TOK_KV, TID_TOK_Z, TID_W_IK = 8, 9, 10


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shapes of one synthetic CSA2 workload.

    B sequences, each with T query tokens and N compressed entries of D channels; H attention
    heads; Hi indexer query heads of dim Di; Hk indexer-key heads (Hi, or 1 for a shared key);
    Top-K `k`; `modes` lists the static mode of each layer in the stack; `pool_blocks` > 0 makes
    the first Full layer build a candidate pool of that many 8-position blocks that later
    Reindex layers score; `p0`/`ratio` set causal visibility for prefill (T > 1).
    """
    name: str
    cfg_id: int
    B: int
    T: int
    N: int
    H: int = 64
    Hi: int = 8
    Di: int = 64
    Hk: int = 8
    D: int = 512
    k: int = 512
    modes: Tuple[int, ...] = (FULL,)
    pool_blocks: int = 0
    block: int = 8
    p0: int = 0
    ratio: int = 4
    planted_frac: float = 0.0
    n_existing: Optional[int] = None   # prefill: entries already in the cache before the chunk

    @property
    def sm_scale(self) -> float:
        return float(1.0 / np.sqrt(self.D))

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    1: Workload("full_decode_b1_n2048", 1, B=1, T=1, N=2048, H=16, Hi=4, Hk=4, k=256),
    2: Workload("full_decode_b32_n16384", 2, B=32, T=1, N=16384, H=64, Hi=8, Hk=8, k=512),
    3: Workload("stack_full_reindex_reuse_b16_n65536", 3, B=16, T=1, N=65536, H=64, Hi=8, Hk=8,
                k=512, modes=(FULL, REINDEX, REUSE)),
    4: Workload("hsi_decode_b4_n262144_pool8192", 4, B=4, T=1, N=262144, H=64, Hi=8, Hk=8, k=512,
                modes=(FULL, REINDEX, REINDEX), pool_blocks=1024, planted_frac=0.01),
    5: Workload("prefill_t4096_n33792", 5, B=1, T=4096, N=33792, H=64, Hi=8, Hk=8, k=1024,
                p0=131072, ratio=4, n_existing=32768),
    # the decoder's layer schedule at the model's own shapes: one Full layer and three Reuse
    # layers, then four times a Reindex layer and three Reuse layers, all on one shared cache;
    # the Full layer builds a pool of 2048 blocks x 8 that every Reindex layer scores; indexer
    # 32 query heads x 128 against one shared 128-channel key per entry; compression ratio 1
    6: Workload("decoder20_hsi_b4_n262144_pool16384", 6, B=4, T=1, N=262144, H=64, Hi=32, Di=128,
                Hk=1, k=512, modes=(FULL, REUSE, REUSE, REUSE) + (REINDEX, REUSE, REUSE, REUSE) * 4,
                pool_blocks=2048, ratio=1),
}


def _rng(wl: Workload, tid: int, *stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([1000 * wl.cfg_id + tid, *stream])))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even) and return the uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def kv_source(wl: Workload, b: int) -> np.ndarray:
    """fp32 [N, D] main-KV values of sequence b before FP4 quantization, N(0, 1)."""
    return _rng(wl, TID_KV, b).standard_normal((wl.N, wl.D), dtype=np.float32)


def q_idx(wl: Workload, b: int, layer: int) -> np.ndarray:
    """bf16 bits [T, Hi, Di]: the indexer query of sequence b at the given layer."""
    x = _rng(wl, TID_QIDX, b, layer).standard_normal((wl.T, wl.Hi, wl.Di), dtype=np.float32)
    return to_bf16_bits(x)


def q_main(wl: Workload, b: int, layer: int) -> np.ndarray:
    """bf16 bits [T, H, D]: the attention query of sequence b at the given layer."""
    x = _rng(wl, TID_Q, b, layer).standard_normal((wl.T, wl.H, wl.D), dtype=np.float32)
    return to_bf16_bits(x)


def k_idx(wl: Workload, b: int) -> np.ndarray:
    """bf16 bits [N, Hk, Di]: the indexer keys of sequence b.

    With planted_frac > 0, that fraction of entries is shifted by 3 (three standard deviations)
    along the unit direction of the first layer's indexer query, head by head, before rounding
    to bf16, so the best entries are well separated from the rest.
    """
    x = _rng(wl, TID_KIDX, b).standard_normal((wl.N, wl.Hk, wl.Di), dtype=np.float32)
    if wl.planted_frac > 0:
        q0 = bf16_bits_to_f32(q_idx(wl, b, 0))[0]                       # [Hi, Di]
        direction = q0 / np.linalg.norm(q0, axis=1, keepdims=True)
        n_plant = int(round(wl.planted_frac * wl.N))
        planted = _rng(wl, TID_PLANT, b).choice(wl.N, size=n_plant, replace=False)
        x[planted] += (3.0 * direction[: wl.Hk]).astype(np.float32)
    return to_bf16_bits(x)


def mxfp4_rows(wl: Workload, b: int, rows: int, channels: int, copy: int = 0) -> np.ndarray:
    """MXFP4 rows of sequence b: uint8 [rows, C/2 + C/32], codes uniform over all 16 E2M1 codes,
    scale codes uniform over 2^-4 .. 2^2 (E8M0 123 .. 129)."""
    g = _rng(wl, TID_MXFP4, b, copy)
    out = g.integers(0, 256, size=(rows, channels // 2 + channels // 32), dtype=np.uint8)
    out[:, channels // 2:] = g.integers(123, 130, size=(rows, channels // 32), dtype=np.uint8)
    return out


def token_kv(wl: Workload, b: int, n_tok: int, first: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """bf16 bits [n_tok, D] x 2: the per-token KV values and compression weights of tokens
    first .. first + n_tok - 1 of sequence b (the compressor's inputs), both N(0, 1)."""
    c = _rng(wl, TID_TOK_KV, b, first).standard_normal((n_tok, wl.D), dtype=np.float32)
    z = _rng(wl, TID_TOK_Z, b, first).standard_normal((n_tok, wl.D), dtype=np.float32)
    return to_bf16_bits(c), to_bf16_bits(z)


def w_index_k(wl: Workload) -> np.ndarray:
    """bf16 bits [Hk * Di, D]: the indexer-key projection weight, row o holding the D input
    weights of key channel o, N(0, 1/D) so that keys of N(0, 1) entries have unit scale."""
    w = _rng(wl, TID_W_IK).standard_normal((wl.Hk * wl.Di, wl.D), dtype=np.float32)
    return to_bf16_bits(w * np.float32(1.0 / np.sqrt(wl.D)))


def swa_window(wl: Workload, b: int, rows: int) -> Tuple[np.ndarray, np.ndarray]:
    """A sliding window of FP8 rows of sequence b: uint8 [rows, D] E4M3 codes, uniform over the
    non-NaN codes, and int8 [rows] row exponents, uniform over [-8, 0]."""
    g = _rng(wl, TID_SWA, b)
    codes = g.integers(0, 256, size=(rows, wl.D), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0
    exps = g.integers(-8, 1, size=rows).astype(np.int8)
    return codes, exps


def sequence(wl: Workload, b: int, layers: Optional[int] = None) -> dict:
    """All inputs of sequence b: kv source, indexer keys, and per-layer queries."""
    nl = len(wl.modes) if layers is None else layers
    return {
        "kv_src": kv_source(wl, b),
        "k_idx": k_idx(wl, b),
        "q_idx": [q_idx(wl, b, l) for l in range(nl)],
        "q": [q_main(wl, b, l) for l in range(nl)],
    }


def random_scores(seed: int, rows: int, n: int, dist: str = "normal") -> np.ndarray:
    """fp32 score rows for stand-alone Top-K tests.

    dist: "normal" (distinct values), "ties" (values drawn from 8 levels, many exact ties),
    "const" (every value equal), "signed_zero" (a mix of +0, -0 and a few normals),
    "bounded" (the sum of 4 uniforms: a tail that ends, so the maxima of small groups bunch up
    near the top).
    """
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, rows, n])))
    if dist == "normal":
        return g.standard_normal((rows, n), dtype=np.float32) * np.float32(20.0)
    if dist == "ties":
        return g.integers(-4, 4, size=(rows, n)).astype(np.float32) * np.float32(0.5)
    if dist == "const":
        return np.full((rows, n), 1.25, dtype=np.float32)
    if dist == "signed_zero":
        x = np.where(g.random((rows, n)) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
        few = g.random((rows, n)) < 0.01
        x[few] = g.standard_normal(int(few.sum()), dtype=np.float32)
        return x
    if dist == "bounded":
        return (g.random((rows, n, 4), dtype=np.float32).sum(-1) - np.float32(2.0)) * np.float32(20.0)
    raise ValueError(dist)
