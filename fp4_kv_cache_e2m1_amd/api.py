"""Python binding of the CSA2 C ABI: the same six calls, over torch device tensors.

This layer only marshals arguments (shapes, dtypes, pointers, the current HIP stream) and sizes
scratch buffers through torch's allocator; every step of the computation runs in the HIP kernels
of libcsa2.so. See include/csa2.h for the exact semantics of each call.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass, field
from typing import Optional, Tuple

import torch

from . import _lib
from ._lib import LayerArgs, SharedIdx, SharedKV, check

FULL, REINDEX, REUSE = 0, 1, 2
F32, BF16 = 0, 1
D_LATENT = 512


def row_bytes(dim: int = D_LATENT) -> int:
    return dim // 2 + dim // 16


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _need(t: torch.Tensor, name: str, dtype, dev=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")


def _ws(nbytes: int, dev, ws: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return ws
    if ws is not None and ws.numel() * ws.element_size() >= nbytes:
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=dev)


# ---------------------------------------------------------------------------------------------
def quantize_kv_fp4(src: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """[..., dim] fp32/bf16 -> [..., dim/2 + dim/16] uint8 FP4 entries (E2M1 + E4M3 per 16)."""
    if src.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("src must be float32 or bfloat16")
    _need(src, "src", None)
    dim = src.shape[-1]
    n_rows = src.numel() // dim if dim else 0
    if out is None:
        out = torch.empty(*src.shape[:-1], row_bytes(dim), dtype=torch.uint8, device=src.device)
    _need(out, "out", torch.uint8, src.device)
    if out.numel() != n_rows * row_bytes(dim):
        raise ValueError("out has the wrong size")
    code = _lib.lib().csa2_quantize_kv_fp4(_ptr(src), BF16 if src.dtype == torch.bfloat16 else F32,
                                           n_rows, dim, _ptr(out), _stream(src.device))
    check("csa2_quantize_kv_fp4", code)
    return out


def compress_kv(c: torch.Tensor, z: torch.Tensor, ratio: int, entry0: torch.Tensor, rows: torch.Tensor,
                w_t: Optional[torch.Tensor] = None, k_idx: Optional[torch.Tensor] = None,
                return_entries: bool = False) -> Optional[torch.Tensor]:
    """The compressor, FP4 packing and indexer-K projection (csa2_compress_kv).

    c, z [B, n_tok, 512] bf16 (new tokens' KV values and compression weights); entry0 [B] int32
    (index of each sequence's first new entry); rows [B, n_max, 288] uint8 written in place;
    w_t [Hk*Di, 512] bf16 and k_idx [B, n_max, Hk, Di] bf16 (written in place), or both None.
    Returns the fp32 entries [B, n_tok/ratio, 512] when return_entries, else None."""
    _need(c, "c", torch.bfloat16)
    dev = c.device
    _need(z, "z", torch.bfloat16, dev)
    _need(entry0, "entry0", torch.int32, dev)
    _need(rows, "rows", torch.uint8, dev)
    B, n_tok, D = c.shape
    if z.shape != c.shape or entry0.numel() != B or rows.shape[0] != B or rows.shape[2] != row_bytes(D):
        raise ValueError("inconsistent shapes for c / z / entry0 / rows")
    Hk = Di = 0
    if (w_t is None) != (k_idx is None):
        raise ValueError("w_t and k_idx go together")
    if k_idx is not None:
        _need(w_t, "w_t", torch.bfloat16, dev)
        _need(k_idx, "k_idx", torch.bfloat16, dev)
        _, n2, Hk, Di = k_idx.shape
        if n2 != rows.shape[1] or w_t.shape != (Hk * Di, D):
            raise ValueError("k_idx must be [B, n_max, Hk, Di] and w_t [Hk*Di, D]")
    ent = torch.empty(B, n_tok // max(ratio, 1), D, dtype=torch.float32, device=dev) if return_entries else None
    code = _lib.lib().csa2_compress_kv(_ptr(c), _ptr(z), B, n_tok, D, ratio, _ptr(entry0), rows.shape[1], _ptr(rows),
                                       _ptr(w_t), Hk, Di, _ptr(k_idx), _ptr(ent), _stream(dev))
    check("csa2_compress_kv", code)
    return ent


def dequant_kv_fp4(rows: torch.Tensor, dim: int = D_LATENT) -> torch.Tensor:
    """[..., dim/2 + dim/16] uint8 -> [..., dim] fp32 (exact)."""
    _need(rows, "rows", torch.uint8)
    if rows.shape[-1] != row_bytes(dim):
        raise ValueError("last dim of rows must be dim/2 + dim/16")
    n_rows = rows.numel() // row_bytes(dim)
    out = torch.empty(*rows.shape[:-1], dim, dtype=torch.float32, device=rows.device)
    check("csa2_dequant_kv_fp4",
          _lib.lib().csa2_dequant_kv_fp4(_ptr(rows), n_rows, dim, _ptr(out), _stream(rows.device)))
    return out


def index_scores(q_idx: torch.Tensor, k_idx: torch.Tensor, n_vis: Optional[torch.Tensor] = None,
                 cand: Optional[torch.Tensor] = None, block_max: bool = False,
                 out: Optional[torch.Tensor] = None, block_max_out: Optional[torch.Tensor] = None):
    """Indexer scores. q_idx [B, T, Hi, Di] bf16, k_idx [B, N, Hk, Di] bf16.

    Flat: returns scores [B*T, N] fp32 (entries >= n_vis unwritten) and, with block_max=True or
    a block_max_out buffer, the 8-entry block maxima [B*T, ceil(N/8)]. Pool (cand [B*T, P]
    int32): scores [B*T, P].
    """
    _need(q_idx, "q_idx", torch.bfloat16)
    _need(k_idx, "k_idx", torch.bfloat16, q_idx.device)
    B, T, Hi, Di = q_idx.shape
    B2, N, Hk, Di2 = k_idx.shape
    if B2 != B or Di2 != Di:
        raise ValueError("q_idx and k_idx disagree on B or Di")
    dev = q_idx.device
    if n_vis is not None:
        _need(n_vis, "n_vis", torch.int32, dev)
        if n_vis.numel() != B * T:
            raise ValueError("n_vis must have B*T entries")
    P = 0
    if cand is not None:
        _need(cand, "cand", torch.int32, dev)
        P = cand.shape[-1]
        if cand.numel() != B * T * P:
            raise ValueError("cand must be [B*T, P]")
    ncols = P if cand is not None else N
    if out is None:
        out = torch.empty(B * T, ncols, dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, dev)
    bm = block_max_out
    if bm is not None:
        _need(bm, "block_max_out", torch.float32, dev)
        if bm.numel() != B * T * ((N + 7) // 8):
            raise ValueError("block_max_out must be [B*T, ceil(N/8)]")
    elif block_max:
        bm = torch.empty(B * T, (N + 7) // 8, dtype=torch.float32, device=dev)
    code = _lib.lib().csa2_index_scores(_ptr(q_idx), _ptr(k_idx), B, T, Hi, Hk, Di, N, _ptr(n_vis),
                                        _ptr(cand), P, _ptr(out), _ptr(bm), 8, _stream(dev))
    check("csa2_index_scores", code)
    return (out, bm) if bm is not None else out


def mxfp4_row_bytes(channels: int) -> int:
    return channels // 2 + channels // 32


def index_scores_mxfp4(q_rows: torch.Tensor, k_rows: torch.Tensor, channels: int,
                       n_vis: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                       q_heads: int = 0, cand: Optional[torch.Tensor] = None, block_max: bool = False):
    """Indexer scores over MXFP4 rows -> scores [B*T, N] fp32 (entries >= n_vis unwritten).

    q_heads = 0: q_rows [B, T, C/2 + C/32] and k_rows [B, N, C/2 + C/32] hold C = `channels`
    channels each (one key head per index head). q_heads = Hi: one shared key of `channels` = 128
    channels per entry, q_rows [B, T, Hi*C/2 + Hi*C/32]. With the shared key, cand [B*T, P] int32
    scores the pool (-> [B*T, P]) and block_max=True also returns the 8-entry block maxima."""
    _need(q_rows, "q_rows", torch.uint8)
    dev = q_rows.device
    _need(k_rows, "k_rows", torch.uint8, dev)
    B, T, RB = q_rows.shape
    B2, N, RB2 = k_rows.shape
    Hi = q_heads if q_heads else 1
    if B2 != B or RB2 != mxfp4_row_bytes(channels) or RB != mxfp4_row_bytes(Hi * channels):
        raise ValueError("q_rows / k_rows disagree with B or the row sizes")
    if n_vis is not None:
        _need(n_vis, "n_vis", torch.int32, dev)
        if n_vis.numel() != B * T:
            raise ValueError("n_vis must have B*T entries")
    P = 0
    if cand is not None:
        _need(cand, "cand", torch.int32, dev)
        P = cand.shape[-1]
        if cand.numel() != B * T * P:
            raise ValueError("cand must be [B*T, P]")
    if out is None:
        out = torch.empty(B * T, P if cand is not None else N, dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, dev)
    bm = torch.empty(B * T, (N + 7) // 8, dtype=torch.float32, device=dev) if block_max else None
    code = _lib.lib().csa2_index_scores_mxfp4(_ptr(q_rows), _ptr(k_rows), B, T, Hi, 1, channels,
                                              N, _ptr(n_vis), _ptr(cand), P, _ptr(out), _ptr(bm), 8, _stream(dev))
    check("csa2_index_scores_mxfp4", code)
    return (out, bm) if block_max else out


def topk(scores: torch.Tensor, k: int, n_valid: Optional[torch.Tensor] = None,
         col_to_pos: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """k best columns per row as ascending positions, -1 padded. scores [rows, n] fp32."""
    _need(scores, "scores", torch.float32)
    rows, n = scores.shape
    dev = scores.device
    if n_valid is not None:
        _need(n_valid, "n_valid", torch.int32, dev)
    if col_to_pos is not None:
        _need(col_to_pos, "col_to_pos", torch.int32, dev)
        if col_to_pos.shape != scores.shape:
            raise ValueError("col_to_pos must have the shape of scores")
    idx = torch.empty(rows, k, dtype=torch.int32, device=dev)
    L = _lib.lib()
    nbytes = L.csa2_topk_workspace_size(rows, max(n, 1), k) if rows and k else 0
    ws = _ws(nbytes, dev, ws)
    code = L.csa2_topk(_ptr(scores), rows, n, _ptr(n_valid), _ptr(col_to_pos), k, _ptr(idx), _ptr(ws),
                       nbytes, _stream(dev))
    check("csa2_topk", code)
    return idx


def hier_pool(block_max: torch.Tensor, n_sel_blocks: int, n_vis: Optional[torch.Tensor] = None,
              block: int = 8, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Candidate pool [rows, n_sel_blocks * block]: ascending visible positions of the best blocks."""
    _need(block_max, "block_max", torch.float32)
    rows, nb = block_max.shape
    dev = block_max.device
    if n_vis is not None:
        _need(n_vis, "n_vis", torch.int32, dev)
    pool = torch.empty(rows, n_sel_blocks * block, dtype=torch.int32, device=dev)
    L = _lib.lib()
    nbytes = L.csa2_hier_pool_workspace_size(rows, max(nb, 1), n_sel_blocks) if rows and n_sel_blocks else 0
    ws = _ws(nbytes, dev, ws)
    code = L.csa2_hier_pool(_ptr(block_max), rows, nb, _ptr(n_vis), block, n_sel_blocks, _ptr(pool), _ptr(ws),
                            nbytes, _stream(dev))
    check("csa2_hier_pool", code)
    return pool


def sparse_attn_workspace_size(B: int, T: int, H: int, D: int, K: int) -> int:
    return int(_lib.lib().csa2_sparse_attn_workspace_size(B, T, H, D, K))


def sparse_attn(q: torch.Tensor, rows: torch.Tensor, idx: torch.Tensor, sm_scale: float,
                with_lse: bool = True, ws: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None):
    """q [B, T, H, 512] bf16, rows [B, N, 288] uint8, idx [B, T, K] int32 -> out fp32 [B, T, H, 512], lse."""
    _need(q, "q", torch.bfloat16)
    dev = q.device
    _need(rows, "rows", torch.uint8, dev)
    _need(idx, "idx", torch.int32, dev)
    B, T, H, D = q.shape
    N = rows.shape[1]
    K = idx.shape[-1]
    if rows.shape[0] != B or rows.shape[2] != row_bytes(D) or idx.shape[:2] != (B, T):
        raise ValueError("inconsistent shapes for q / rows / idx")
    if out is None:
        out = torch.empty(B, T, H, D, dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, dev)
    if out.numel() != B * T * H * D:
        raise ValueError("out must be [B, T, H, D]")
    lse = torch.empty(B, T, H, dtype=torch.float32, device=dev) if with_lse else None
    L = _lib.lib()
    nbytes = L.csa2_sparse_attn_workspace_size(B, T, H, D, K)
    ws = _ws(nbytes, dev, ws)
    code = L.csa2_sparse_attn(_ptr(q), _ptr(rows), N, _ptr(idx), B, T, H, D, K, float(sm_scale), _ptr(out),
                              _ptr(lse), _ptr(ws), nbytes, _stream(dev))
    check("csa2_sparse_attn", code)
    return out, lse


def sparse_attn_swa(q: torch.Tensor, rows: torch.Tensor, idx: torch.Tensor, swa_codes: torch.Tensor,
                    swa_exp: torch.Tensor, n_win: torch.Tensor, sm_scale: float, with_lse: bool = True,
                    ws: Optional[torch.Tensor] = None):
    """Decode attention over the selected entries joined with each sequence's window of FP8 rows.

    q [B, H, 512] bf16, rows [B, N, 288] uint8, idx [B, K] int32, swa_codes [B, W, 512] uint8,
    swa_exp [B, W] int8, n_win [B] int32 -> out fp32 [B, H, 512], lse fp32 [B, H].
    """
    _need(q, "q", torch.bfloat16)
    dev = q.device
    _need(rows, "rows", torch.uint8, dev)
    _need(idx, "idx", torch.int32, dev)
    _need(swa_codes, "swa_codes", torch.uint8, dev)
    _need(swa_exp, "swa_exp", torch.int8, dev)
    _need(n_win, "n_win", torch.int32, dev)
    B, H, D = q.shape
    N, K, W = rows.shape[1], idx.shape[-1], swa_codes.shape[1]
    if (rows.shape[0] != B or rows.shape[2] != row_bytes(D) or idx.shape[0] != B or swa_codes.shape != (B, W, D)
            or swa_exp.shape != (B, W) or n_win.shape != (B,)):
        raise ValueError("inconsistent shapes for q / rows / idx / window")
    out = torch.empty(B, H, D, dtype=torch.float32, device=dev)
    lse = torch.empty(B, H, dtype=torch.float32, device=dev) if with_lse else None
    L = _lib.lib()
    nbytes = L.csa2_sparse_attn_swa_workspace_size(B, H, D, K)
    ws = _ws(max(nbytes, 1), dev, ws)
    code = L.csa2_sparse_attn_swa(_ptr(q), _ptr(rows), N, _ptr(idx), B, H, D, K, _ptr(swa_codes), _ptr(swa_exp),
                                  _ptr(n_win), W, float(sm_scale), _ptr(out), _ptr(lse), _ptr(ws), nbytes,
                                  _stream(dev))
    check("csa2_sparse_attn_swa", code)
    return out, lse


def sparse_attn_swa_prefill(q: torch.Tensor, rows: torch.Tensor, idx: torch.Tensor, swa_codes: torch.Tensor,
                            swa_exp: torch.Tensor, n_win: torch.Tensor, sm_scale: float, with_lse: bool = True,
                            ws: Optional[torch.Tensor] = None):
    """Many query tokens over their selected entries joined with each token's window (its last
    n_win tokens up to its own). q [B, T, H, 512] bf16, rows [B, N, 288] uint8, idx [B, T, K]
    int32, swa_codes [B, T + W - 1, 512] uint8, swa_exp [B, T + W - 1] int8, n_win [B, T] int32
    -> out fp32 [B, T, H, 512], lse fp32 [B, T, H]."""
    _need(q, "q", torch.bfloat16)
    dev = q.device
    _need(rows, "rows", torch.uint8, dev)
    _need(idx, "idx", torch.int32, dev)
    _need(swa_codes, "swa_codes", torch.uint8, dev)
    _need(swa_exp, "swa_exp", torch.int8, dev)
    _need(n_win, "n_win", torch.int32, dev)
    B, T, H, D = q.shape
    N, K = rows.shape[1], idx.shape[-1]
    W = swa_codes.shape[1] - T + 1
    if (rows.shape[0] != B or rows.shape[2] != row_bytes(D) or idx.shape[:2] != (B, T) or W < 0
            or swa_codes.shape != (B, T + W - 1, D) or swa_exp.shape != (B, T + W - 1) or n_win.numel() != B * T):
        raise ValueError("inconsistent shapes for q / rows / idx / window")
    out = torch.empty(B, T, H, D, dtype=torch.float32, device=dev)
    lse = torch.empty(B, T, H, dtype=torch.float32, device=dev) if with_lse else None
    L = _lib.lib()
    nbytes = L.csa2_sparse_attn_swa_prefill_workspace_size(B, T, H, D, K)
    ws = _ws(nbytes, dev, ws)              # none for wide calls: the window runs inside their pass
    code = L.csa2_sparse_attn_swa_prefill(_ptr(q), _ptr(rows), N, _ptr(idx), B, T, H, D, K, _ptr(swa_codes),
                                          _ptr(swa_exp), _ptr(n_win), W, float(sm_scale), _ptr(out), _ptr(lse),
                                          _ptr(ws), nbytes, _stream(dev))
    check("csa2_sparse_attn_swa_prefill", code)
    return out, lse


def prefill_n_vis(p0, T: int, ratio: int, device, n_max: int = 2 ** 31 - 1) -> torch.Tensor:
    """Visible compressed entries of query tokens at positions p0[b] .. p0[b]+T-1, from
    csa2_prefill_visibility: int32 [B*T]. p0 is one start position or one per sequence."""
    dev = torch.device(device)
    starts = torch.as_tensor([p0] if isinstance(p0, int) else list(p0), dtype=torch.int64).to(dev)
    B = starts.numel()
    out = torch.empty(B * T, dtype=torch.int32, device=dev)
    code = _lib.lib().csa2_prefill_visibility(_ptr(starts), B, T, ratio, n_max, _ptr(out), _stream(dev))
    check("csa2_prefill_visibility", code)
    return out


# ---------------------------------------------------------------------------------------------
# Layer step with caller-owned shared state
# ---------------------------------------------------------------------------------------------
@dataclass
class KVState:
    """The cache of the most recent Full layer: FP4 rows and indexer keys (device tensors).

    The indexer keys are bf16 (k_idx), or FP4 (k_mx: MXFP4 rows [B, N, C/2 + C/32] of
    C = Hk * Di channels, with k_idx None and mx_heads = (Hk, Di))."""
    rows: torch.Tensor                 # [B, N, 288] uint8
    k_idx: Optional[torch.Tensor]      # [B, N, Hk, Di] bf16, or None with k_mx
    n_vis: Optional[torch.Tensor] = None  # [B*T] int32
    k_mx: Optional[torch.Tensor] = None   # [B, N, C/2 + C/32] uint8
    mx_heads: Tuple[int, int] = (0, 0)
    c: SharedKV = field(default_factory=SharedKV)

    def __post_init__(self):
        _need(self.rows, "rows", torch.uint8)
        B, N, rb = self.rows.shape
        if self.k_mx is not None:
            _need(self.k_mx, "k_mx", torch.uint8, self.rows.device)
            Hk, Di = self.mx_heads
            C = Hk * Di
            if self.k_mx.shape != (B, N, mxfp4_row_bytes(C)):
                raise ValueError("k_mx must be [B, N, C/2 + C/32] with C = Hk * Di")
        else:
            _need(self.k_idx, "k_idx", torch.bfloat16, self.rows.device)
            _, N2, Hk, Di = self.k_idx.shape
            if N2 != N:
                raise ValueError("rows and k_idx disagree on N")
        self.c.rows, self.c.k_idx, self.c.n_vis = _ptr(self.rows), _ptr(self.k_idx), _ptr(self.n_vis)
        self.c.k_mx = _ptr(self.k_mx)
        self.c.B, self.c.n_max, self.c.D, self.c.Hk, self.c.Di = B, N, (rb * 16) // 9, Hk, Di
        self.c.valid = 0

    @property
    def valid(self) -> bool:
        return bool(self.c.valid)


@dataclass
class IdxState:
    """The newest Top-K (and candidate pool) of the latest index-producing layer."""
    topk: torch.Tensor                 # [B*T, K] int32
    pool: Optional[torch.Tensor] = None  # [B*T, P] int32
    c: SharedIdx = field(default_factory=SharedIdx)

    @staticmethod
    def empty(rows: int, k: int, device, pool_size: int = 0) -> "IdxState":
        t = torch.full((rows, k), -1, dtype=torch.int32, device=device)
        p = torch.full((rows, pool_size), -1, dtype=torch.int32, device=device) if pool_size else None
        return IdxState(t, p)

    def __post_init__(self):
        _need(self.topk, "topk", torch.int32)
        self.c.topk, self.c.K = _ptr(self.topk), self.topk.shape[-1]
        if self.pool is not None:
            _need(self.pool, "pool", torch.int32, self.topk.device)
            self.c.pool, self.c.P = _ptr(self.pool), self.pool.shape[-1]
        self.c.topk_valid = 0
        self.c.pool_valid = 0


def layer_workspace_size(mode: int, args: LayerArgs, kv: KVState, idx: IdxState) -> int:
    n = C.c_size_t(0)
    check("csa2_layer_workspace_size",
          _lib.lib().csa2_layer_workspace_size(mode, C.byref(args), C.byref(kv.c), C.byref(idx.c), C.byref(n)))
    return n.value


def layer_args(mode: int, q: torch.Tensor, kv: KVState, idx: IdxState, q_idx: Optional[torch.Tensor] = None,
               sm_scale: Optional[float] = None, use_pool: bool = False, pool_blocks: int = 0, block: int = 8,
               window: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
               q_idx_mx: Optional[torch.Tensor] = None,
               produce: Optional[Tuple[torch.Tensor, torch.Tensor, int, torch.Tensor, torch.Tensor]] = None
               ) -> LayerArgs:
    """The csa2_layer_args struct of one CSA2 layer (FULL / REINDEX / REUSE) over caller-owned
    shared state, without output, LSE or workspace (layer_step fills those).

    window: the layer's sliding window joined to the selected entries as one softmax: decode
    (swa_codes [B, W, D] uint8, swa_exp [B, W] int8, n_win [B] int32), or prefill (swa_codes
    [B, T + W - 1, D], swa_exp [B, T + W - 1], n_win [B, T]: each token's last n tokens).
    q_idx_mx: [B, T, C/2 + C/32] uint8 MXFP4 indexer query, for a KVState with FP4 keys (then
    q_idx only gives Hi and may be None with Hi taken from the state).
    produce: (new_kv [B, n_tok, D] bf16, new_z [B, n_tok, D] bf16, ratio, entry0 [B] int32,
    w_ik [Hk*Di, D] bf16): a Full layer first compresses its new tokens into the shared caches."""
    _need(q, "q", torch.bfloat16, kv.rows.device)
    dev = q.device
    B, T, H, D = q.shape
    a = LayerArgs()
    a.q = _ptr(q)
    a.T, a.H = T, H
    if q_idx is not None:
        _need(q_idx, "q_idx", torch.bfloat16, dev)
        a.q_idx, a.Hi = _ptr(q_idx), q_idx.shape[2]
    if q_idx_mx is not None:
        _need(q_idx_mx, "q_idx_mx", torch.uint8, dev)
        if q_idx_mx.shape[:2] != (B, T):
            raise ValueError("q_idx_mx must be [B, T, C/2 + C/32]")
        qc = q_idx_mx.shape[2] * 32 // 17                           # channels of a query row
        a.q_idx_mx, a.Hi = _ptr(q_idx_mx), qc // kv.c.Di
    a.sm_scale = float(sm_scale if sm_scale is not None else D ** -0.5)
    a.use_pool, a.pool_blocks, a.block = int(use_pool), pool_blocks, block
    if window is not None:
        codes, exps, n_win = window
        _need(codes, "swa_codes", torch.uint8, dev)
        _need(exps, "swa_exp", torch.int8, dev)
        _need(n_win, "n_win", torch.int32, dev)
        Wn = codes.shape[1] - T + 1
        if (codes.shape[0] != B or codes.shape[2] != D or exps.shape != codes.shape[:2] or Wn < 0
                or n_win.numel() != (B if T == 1 else B * T)):
            raise ValueError("window shapes must be [B, T + W - 1, D], [B, T + W - 1], [B] or [B, T]")
        a.swa_codes, a.swa_exp, a.swa_n, a.swa_W = _ptr(codes), _ptr(exps), _ptr(n_win), Wn
    if produce is not None:
        nk, nz, ratio, entry0, w_ik = produce
        _need(nk, "new_kv", torch.bfloat16, dev)
        _need(nz, "new_z", torch.bfloat16, dev)
        _need(entry0, "new_entry0", torch.int32, dev)
        _need(w_ik, "w_ik", torch.bfloat16, dev)
        if nk.shape != nz.shape or nk.shape[0] != B or nk.shape[2] != D or entry0.numel() != B:
            raise ValueError("new_kv / new_z must be [B, n_tok, D] and new_entry0 [B]")
        a.new_kv, a.new_z, a.new_tokens, a.ratio = _ptr(nk), _ptr(nz), nk.shape[1], ratio
        a.new_entry0, a.w_ik = _ptr(entry0), _ptr(w_ik)
    return a


def layer_step(mode: int, q: torch.Tensor, kv: KVState, idx: IdxState, q_idx: Optional[torch.Tensor] = None,
               sm_scale: Optional[float] = None, use_pool: bool = False, pool_blocks: int = 0, block: int = 8,
               with_lse: bool = True, ws: Optional[torch.Tensor] = None,
               out: Optional[torch.Tensor] = None,
               window: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
               q_idx_mx: Optional[torch.Tensor] = None,
               no_alloc: bool = False,
               produce: Optional[Tuple[torch.Tensor, torch.Tensor, int, torch.Tensor, torch.Tensor]] = None
               ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """One CSA2 layer (FULL / REINDEX / REUSE) over caller-owned shared state; returns (out, lse).
    Arguments as layer_args; out [B, T, H, D] fp32 (allocated if None), ws a uint8 workspace of at
    least layer_workspace_size bytes (allocated if None or too small). no_alloc=True calls
    csa2_layer_step_noalloc instead, which takes its scratch from the library's fixed device array
    (ws is then ignored)."""
    a = layer_args(mode, q, kv, idx, q_idx=q_idx, sm_scale=sm_scale, use_pool=use_pool, pool_blocks=pool_blocks,
                   block=block, window=window, q_idx_mx=q_idx_mx, produce=produce)
    dev = q.device
    B, T, H, D = q.shape
    if out is None:
        out = torch.empty(B, T, H, D, dtype=torch.float32, device=dev)
    lse = torch.empty(B, T, H, dtype=torch.float32, device=dev) if with_lse else None
    a.out, a.lse = _ptr(out), _ptr(lse)
    if no_alloc:
        code = _lib.lib().csa2_layer_step_noalloc(mode, C.byref(a), C.byref(kv.c), C.byref(idx.c), _stream(dev))
        check("csa2_layer_step_noalloc", code)
        return out, lse
    nbytes = layer_workspace_size(mode, a, kv, idx)
    ws = _ws(nbytes, dev, ws)
    a.ws, a.ws_bytes = _ptr(ws), nbytes
    code = _lib.lib().csa2_layer_step(mode, C.byref(a), C.byref(kv.c), C.byref(idx.c), _stream(dev))
    check("csa2_layer_step", code)
    return out, lse
