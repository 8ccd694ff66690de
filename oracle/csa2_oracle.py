"""CPU oracle for the CSA2 decode/prefill hot path with an FP4 (E2M1 + E4M3/16) main KV cache.

TEST INFRASTRUCTURE ONLY. Nothing in the product path (the HIP library, its C-ABI, the Python
binding) imports, calls or links this module. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may use it.

It is a plain, slow, obviously-correct restatement of what the method computes, in numpy fp64.
Each function names the passage it follows. The sources are web pages about DeepSeek-V4.1-Flash:

  [walkthrough]  "【论文解读】 DeepSeek-V4.1-Flash" (wkq9411.github.io, a walkthrough of the
                 V4.1 tech report). Sections used:
                   一(四) "Compressed Sparse Attention 2 (CSA2)" - the lightweight indexer,
                          Top-K per query, attention over the selected entries;
                   一(四)1 "Cross-Layer KV 和 Index Reuse" - Full / Reindex / Reuse modes;
                   一(四)2 "Hierarchical Sparse Indexer" - block max, block selection, pool;
                   一(五)4 "FP4 Main KV Cache" - E2M1 values, one E4M3 scale per 16 channels,
                          no global scale, 448 x 6 = 2688, dequantize before attention;
                   三(二)1 "模型设置" - 512 selected entries, 64 query heads of dim 512,
                          2048 blocks x 8 positions.
  [release note] ModelScope release note, section "压缩稀疏注意力 2（CSA2）" - the same modes,
                 HSI and FP4 format in summary.

Where the pages leave a step open the reading taken is stated at the function (R-n tags match
the list of readings kept with the design notes of this repository).

Parity status: every public function here is pinned by CPU tests against closed forms, library
routines (torch float8_e4m3fn decode / rounding, torch scaled_dot_product_attention, full sorts),
brute force on tiny inputs, hand-built ties, and the structural invariants the pages state.
No function is "parity unpinned".
"""

from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------------------------
# Format constants. [walkthrough] 一(五)4: E2M1 values, one E4M3 scale for every 16 channels.
# ---------------------------------------------------------------------------------------------
GROUP = 16            # channels per E4M3 scale
D_LATENT = 512        # channels of one compressed KV entry (the attention head dim)


def row_bytes(dim: int = D_LATENT) -> int:
    """Bytes of one packed entry: 4 bits per channel plus one byte per 16-channel group.

    For the 512-channel latent this is 256 + 32 = 288 bytes.
    """
    return dim // 2 + dim // GROUP


# ---------------------------------------------------------------------------------------------
# O1 / O2: decoding the two 4- and 8-bit formats from their bit fields.
# ---------------------------------------------------------------------------------------------
def e2m1_decode(codes) -> np.ndarray:
    """O1. Value of E2M1 codes (1 sign, 2 exponent bits with bias 1, 1 mantissa bit).

    [walkthrough] 一(五)4 names E2M1 as the value format. Exponent field 0 is subnormal
    (0.5 * m); otherwise 2^(e-1) * (1 + m/2). Code 8 is -0.
    """
    c = np.asarray(codes).astype(np.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, (e - 1).astype(np.int64)))
    return np.where(s == 1, -mag, mag).astype(np.float64)


def e4m3_decode(codes) -> np.ndarray:
    """O2. Value of OCP E4M3 ("FN") codes: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits.

    [walkthrough] 一(五)4: one E4M3 scale per 16 channels, largest value 448. There is no
    infinity; exponent 15 with mantissa 7 (0x7F, 0xFF) is NaN. Exponent 0 is subnormal
    (m * 2^-9).
    """
    c = np.asarray(codes).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64)))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag).astype(np.float64)


# The 8 E2M1 magnitudes in code order, and the 127 finite non-negative E4M3 values in code
# order (codes 0x00..0x7E); both derived from the decoders above.
E2M1_MAGS = e2m1_decode(np.arange(8))
E4M3_POS = e4m3_decode(np.arange(0x7F))


# ---------------------------------------------------------------------------------------------
# O3 / O4: quantizing and packing one entry.
# ---------------------------------------------------------------------------------------------
def _nearest_even(table: np.ndarray, target: np.ndarray) -> np.ndarray:
    """Index of the table value nearest to each target, ties broken to the even index.

    `table` is ascending. Distances are formed in fp64; for the operands used here (values with
    few significant bits, fp32 targets) the ties are decided exactly.
    """
    hi = np.clip(np.searchsorted(table, target, side="left"), 1, len(table) - 1)
    lo = hi - 1
    d_lo = np.abs(target - table[lo])
    d_hi = np.abs(table[hi] - target)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    # targets beyond either end of the table saturate to that end
    idx = np.where(target <= table[0], 0, idx)
    idx = np.where(target >= table[-1], len(table) - 1, idx)
    return idx


def quantize_groups(x: np.ndarray):
    """O3. Quantize groups of 16 values to 16 E2M1 codes and one E4M3 scale code each.

    [walkthrough] 一(五)4 fixes the format (E2M1 values, one E4M3 scale per 16 channels, NVFP4
    without the global scale) but not the rounding. Readings taken (R-1, R-2):
      * scale = the E4M3 value nearest to amax/6 (round to nearest, ties to the even code,
        saturating at 448), where amax = max |x| over the group; this is the nearest finite
        E4M3 value s to amax/6, found by comparing 6*s with amax exactly;
      * each value's magnitude code is the E2M1 magnitude m_j nearest to |x|/s (ties to even
        j, saturating at 6), found by comparing s*m_j with |x| exactly;
      * the sign bit is the sign bit of x (so -0 and negatives that round to 0 give code 8);
      * a zero scale gives magnitude code 0 for all 16 values.
    x: [..., 16] float array (fp32 or exact fp64). Returns (codes uint8 [..., 16],
    scale codes uint8 [...]).
    """
    x = np.asarray(x, dtype=np.float64)
    assert x.shape[-1] == GROUP
    ax = np.abs(x)
    amax = ax.max(axis=-1)
    sc = _nearest_even(6.0 * E4M3_POS, amax)             # exact compare of amax with 6*s
    s = E4M3_POS[sc]
    # magnitude codes: nearest of s*m_j to |x|, ties to even j
    mj = _nearest_even_scaled(ax, s[..., None])
    mj = np.where(s[..., None] == 0.0, 0, mj)
    sign = np.signbit(x).astype(np.int64)
    codes = (sign << 3) | mj
    return codes.astype(np.uint8), sc.astype(np.uint8)


def _nearest_even_scaled(ax: np.ndarray, s: np.ndarray) -> np.ndarray:
    """argmin_j | ax - s*m_j | over the 8 E2M1 magnitudes m_j, ties to the even j; values at or
    beyond the largest magnitude 6*s saturate to j = 7 (for |x| far above 6*s the fp64 distances
    would all round to the same number, so saturation is decided by a direct compare)."""
    cand = s * E2M1_MAGS                                # [..., 8], exact products
    dist = np.abs(ax[..., None] - cand[..., None, :])    # [..., 16, 8]
    dmin = dist.min(axis=-1, keepdims=True)
    is_min = dist == dmin
    # among the (at most two, adjacent) minimisers prefer the even index
    even = is_min & (np.arange(8) % 2 == 0)
    j = np.where(even.any(axis=-1), even.argmax(axis=-1), is_min.argmax(axis=-1))
    return np.where(ax >= 6.0 * s, 7, j)


def quantize_kv_fp4(src: np.ndarray, chunk_rows: int = 4096) -> np.ndarray:
    """O3 + O4. Quantize and pack entries [rows, D] (fp32 values) into [rows, D/2 + D/16] bytes.

    Layout (reading R-15; the pages give no byte layout): bytes
    0 .. D/2-1 hold the codes, channel 2i in the low nibble of byte i and channel 2i+1 in the
    high nibble; bytes D/2 .. D/2 + D/16 - 1 hold the E4M3 scale codes, group g covering
    channels 16g .. 16g+15. For D = 512 that is 256 + 32 = 288 bytes.
    """
    src = np.asarray(src)
    rows, d = src.shape
    assert d % (2 * GROUP) == 0
    out = np.empty((rows, row_bytes(d)), dtype=np.uint8)
    for r0 in range(0, rows, chunk_rows):
        x = src[r0:r0 + chunk_rows].astype(np.float64).reshape(-1, d // GROUP, GROUP)
        codes, sc = quantize_groups(x)
        codes = codes.reshape(-1, d).astype(np.uint16)
        out[r0:r0 + chunk_rows, : d // 2] = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
        out[r0:r0 + chunk_rows, d // 2:] = sc
    return out


def dequant_kv_fp4(rows: np.ndarray, dim: int = D_LATENT) -> np.ndarray:
    """O5. Unpack and dequantize [n, D/2 + D/16] bytes to fp64 [n, D]: x = E2M1(code) * E4M3(scale).

    [walkthrough] 一(五)4: the cache is dequantized before attention, so attention runs on
    these values. Every product has at most 6 significant bits and is exact.
    """
    rows = np.asarray(rows, dtype=np.uint8)
    n = rows.shape[0]
    assert rows.shape[1] == row_bytes(dim)
    codes = np.empty((n, dim), dtype=np.uint8)
    codes[:, 0::2] = rows[:, : dim // 2] & 0xF
    codes[:, 1::2] = rows[:, : dim // 2] >> 4
    scales = e4m3_decode(rows[:, dim // 2:])             # [n, dim/16]
    return e2m1_decode(codes) * np.repeat(scales, GROUP, axis=1)


# ---------------------------------------------------------------------------------------------
# O14 / O15: producing the caches - the simplified compressor and the indexer-K projection.
# ---------------------------------------------------------------------------------------------
def compress_kv(c: np.ndarray, z: np.ndarray, ratio: int) -> np.ndarray:
    """O14. The CSA2 compressor: every `ratio` consecutive tokens become one main-KV entry.

    [walkthrough] 一(三): each layer's KV entries C and their compression weights Z are
    projections of the same hidden states (C_l = H W^KV_l, Z_l = H W^Z_l). [walkthrough] 一(四):
    CSA builds an entry from 2m overlapping source entries and adds an absolute position
    encoding; CSA2 removes both, so entry j is made from tokens jm .. jm+m-1 alone. The pages give
    no formula for the combination; the reading taken (R-22) is a softmax over the m tokens of the
    group, per channel, weighting the tokens' KV values:
        entry[j, d] = sum_i w[i, d] * c[jm + i, d],  w[:, d] = softmax_i(z[jm + i, d]).
    c, z: [n_tok, D] exact values (bf16 inputs as fp64), n_tok a multiple of ratio.
    Returns fp32 [n_tok / ratio, D]: the exponentials, normalization and weighted sum in fp64,
    rounded once to fp32 (the precision the entry is quantized from).
    """
    c = np.asarray(c, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    n, d = c.shape
    assert z.shape == c.shape and ratio >= 1 and n % ratio == 0
    cg = c.reshape(n // ratio, ratio, d)
    zg = z.reshape(n // ratio, ratio, d)
    e = np.exp(zg - zg.max(axis=1, keepdims=True))     # largest weight of each channel is exp(0) = 1
    w = e / e.sum(axis=1, keepdims=True)
    return (w * cg).sum(axis=1).astype(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp64 values rounded to the nearest bf16 value (8 significant bits, ties to even), as fp64.

    Written from the format: x = m * 2^e with m in [0.5, 1); keep 8 bits of m with
    round-half-to-even (numpy's rint), for values in bf16's normal range (as here).
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def project_index_k(entries: np.ndarray, w_t: np.ndarray, heads: int, dim: int, rounded: bool = True) -> np.ndarray:
    """O15. Indexer keys as a projection of the main-KV entries.

    [walkthrough] 一(四): CSA2 obtains indexer K by projecting the main-KV entries, instead of
    CSA's separate compression path from the hidden states; 一(四)1: a Full layer computes its own
    main KV and indexer K. Reading (R-22): the projection takes the compressed entry (fp32) in
    bf16, like the model's other activations, and a weight w_t [heads * dim, D] whose row o holds
    the D input weights of key channel o; the key is stored in bf16 (the indexer-key format, R-4):
        k[n, h, d] = bf16( sum_c bf16(entries[n, c]) * w_t[h * dim + d, c] ).
    entries: fp32 [N, D]; w_t: exact values [heads * dim, D]. Returns fp64 [N, heads, dim], the
    bf16 values (rounded=True) or the exact sums before the final rounding (rounded=False).
    Products of two bf16 values are exact in fp64 and the sum is fp64.
    """
    x = round_bf16(np.asarray(entries, dtype=np.float32).astype(np.float64))
    w = np.asarray(w_t, dtype=np.float64)
    assert w.shape == (heads * dim, x.shape[1])
    y = x @ w.T
    return (round_bf16(y) if rounded else y).reshape(-1, heads, dim)


# ---------------------------------------------------------------------------------------------
# O6: the lightweight indexer.
# ---------------------------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) to exact fp64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def index_scores(q_idx: np.ndarray, k_idx: np.ndarray, n_vis) -> np.ndarray:
    """O6. Indexer score of every visible entry for each query row, rounded once to fp32.

    [walkthrough] 一(四): indexer Q and indexer K score the main-KV entries, and each query
    keeps its Top-K. The pages print no score formula; the reading taken (R-4) is
    s[r, n] = sum_h sum_d q_idx[r, h, d] * k_idx[n, h', d] with h' = h when keys have one head
    per index head, and h' = 0 when keys have one shared head.
    q_idx: [R, Hi, Di] exact values (fp64); k_idx: [N, Hk, Di] exact values; n_vis: [R] ints.
    Returns fp32 [R, N]; columns n >= n_vis[r] are -inf (they are not part of the result).
    Products of bf16 values are exact in fp64; the sum is fp64; one rounding to fp32 at the end.
    """
    q = np.asarray(q_idx, dtype=np.float64)
    k = np.asarray(k_idx, dtype=np.float64)
    R, Hi, Di = q.shape
    N, Hk, _ = k.shape
    assert Hk in (1, Hi)
    if Hk == 1:
        # sum over the heads of each head's dot product with the one shared key
        s = np.zeros((R, N), dtype=np.float64)
        for h in range(Hi):
            s += q[:, h, :] @ k[:, 0, :].T
    else:
        s = q.reshape(R, Hi * Di) @ k.reshape(N, Hi * Di).T  # [R, N] fp64
    out = s.astype(np.float32)
    n_vis = np.broadcast_to(np.asarray(n_vis), (R,))
    out[np.arange(N)[None, :] >= n_vis[:, None]] = -np.inf
    return out


# ---------------------------------------------------------------------------------------------
# O13: FP4 (OCP MXFP4) indexer query and key.
# ---------------------------------------------------------------------------------------------
MX_BLOCK = 32         # channels per E8M0 scale (OCP MX)
MX_EMAX_E2M1 = 2      # exponent of E2M1's largest power of two (6 = 1.5 * 2^2)


def e8m0_decode(codes) -> np.ndarray:
    """OCP E8M0 scale: code c is 2^(c - 127); c = 255 is NaN."""
    c = np.asarray(codes, dtype=np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, c - 127))


def mxfp4_row_bytes(channels: int) -> int:
    return channels // 2 + channels // MX_BLOCK


def quantize_mxfp4(x: np.ndarray) -> np.ndarray:
    """O13a. Quantize rows [n, C] to MXFP4 rows [n, C/2 + C/32] bytes.

    [walkthrough] 一(五)4: the indexer query and key are FP4 in the OCP MXFP4 format (E2M1
    elements, one E8M0 power-of-two scale per 32). Conversion as the OCP MX rule states it
    (reading R-19): the block's shared exponent is X = floor(log2(max |x|)) - 2 (the largest
    E2M1 power of two is 2^2), clamped to the E8M0 range [-127, 127]; each element is the E2M1
    value nearest to x / 2^X (ties to the even code, saturating at 6) with the sign bit of x.
    A block of zeros takes X = -127. Layout (R-20, as the main KV rows): bytes 0 .. C/2-1 hold
    the codes (channel 2i in the low nibble of byte i), bytes C/2 .. C/2 + C/32 - 1 the E8M0
    codes X + 127 of blocks 0, 1, ...
    """
    x = np.asarray(x).astype(np.float64)
    n, C = x.shape
    assert C % (2 * MX_BLOCK) == 0
    xb = x.reshape(n, C // MX_BLOCK, MX_BLOCK)
    amax = np.abs(xb).max(axis=-1)
    X = np.full(amax.shape, -127, dtype=np.int64)
    nz = amax > 0
    X[nz] = np.frexp(amax[nz])[1] - 1 - MX_EMAX_E2M1      # frexp: amax = m 2^e, m in [0.5, 1)
    X = np.clip(X, -127, 127)
    mj = _nearest_even_scaled(np.abs(xb), np.ldexp(1.0, X)[..., None])
    codes = ((np.signbit(xb).astype(np.int64) << 3) | mj).reshape(n, C).astype(np.uint16)
    out = np.empty((n, mxfp4_row_bytes(C)), dtype=np.uint8)
    out[:, : C // 2] = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    out[:, C // 2:] = (X + 127).astype(np.uint8)
    return out


def dequant_mxfp4(rows: np.ndarray, channels: int) -> np.ndarray:
    """O13b. MXFP4 rows [n, C/2 + C/32] -> exact fp64 values [n, C]: E2M1(code) * 2^(scale - 127)."""
    rows = np.asarray(rows, dtype=np.uint8)
    n = rows.shape[0]
    assert rows.shape[1] == mxfp4_row_bytes(channels)
    codes = np.empty((n, channels), dtype=np.uint8)
    codes[:, 0::2] = rows[:, : channels // 2] & 0xF
    codes[:, 1::2] = rows[:, : channels // 2] >> 4
    return e2m1_decode(codes) * np.repeat(e8m0_decode(rows[:, channels // 2:]), MX_BLOCK, axis=1)


def index_scores_mxfp4(q_rows: np.ndarray, k_rows: np.ndarray, channels: int, n_vis,
                       q_heads: int = 0) -> np.ndarray:
    """O13c. The indexer score (O6) of MXFP4 query rows [R, .] against MXFP4 key rows [N, .].

    q_heads = 0: each row holds all Hi x Di channels of one query or one entry (one key head per
    index head, R-4): s[r, n] = sum_c q[r, c] * k[n, c]. q_heads = Hi: one shared key of
    `channels` channels per entry, query rows of Hi x `channels` (head h = channels
    h*channels .. ), s[r, n] = sum_h q[r, h] . k[n] (R-4, R-16). Over the dequantized values,
    fp64, rounded once to fp32."""
    k = dequant_mxfp4(k_rows, channels)
    if q_heads:
        q = dequant_mxfp4(q_rows, q_heads * channels).reshape(-1, q_heads, channels)
        return index_scores(q, k[:, None, :], n_vis)
    q = dequant_mxfp4(q_rows, channels)
    return index_scores(q[:, None, :], k[:, None, :], n_vis)


def prefill_n_vis(p0: int, T: int, ratio: int) -> np.ndarray:
    """Causal visibility for query tokens at absolute positions p0 .. p0+T-1 (reading R-6).

    A compressed entry covering source tokens [m*j, m*j + m) is visible once its last source
    token is at or before the query position, so n_vis(p) = floor((p + 1) / m).
    """
    p = np.arange(p0, p0 + T, dtype=np.int64)
    return ((p + 1) // ratio).astype(np.int64)


# ---------------------------------------------------------------------------------------------
# O7: Top-K.
# ---------------------------------------------------------------------------------------------
def topk(scores: np.ndarray, k: int, n_valid=None, col_to_pos=None) -> np.ndarray:
    """O7. The k best columns of each row, as positions in ascending order, -1 padded.

    [walkthrough] 一(四): each query selects its Top-K entries. Order used to choose (R-7):
    score descending, then position ascending. Only the first n_valid[r] columns take part; with
    col_to_pos, column c stands for position col_to_pos[r, c] and columns whose position is < 0
    do not take part. The chosen positions are returned sorted ascending and padded with -1 to k
    (R-8). Scores are compared in fp32 (the precision the scores are delivered in).
    """
    scores = np.asarray(scores, dtype=np.float32)
    R, n = scores.shape
    if n_valid is None:
        n_valid = np.full(R, n)
    n_valid = np.broadcast_to(np.asarray(n_valid), (R,))
    out = np.full((R, k), -1, dtype=np.int64)
    for r in range(R):
        cols = np.arange(min(int(n_valid[r]), n))
        pos = cols if col_to_pos is None else np.asarray(col_to_pos[r])[cols].astype(np.int64)
        keep = pos >= 0
        cols, pos = cols[keep], pos[keep]
        s = scores[r, cols]
        order = np.lexsort((pos, -s))                    # primary: -score, secondary: position
        chosen = np.sort(pos[order[:k]])
        out[r, : len(chosen)] = chosen
    return out


# ---------------------------------------------------------------------------------------------
# O8 / O9: Hierarchical Sparse Indexer.
# ---------------------------------------------------------------------------------------------
def block_max(scores: np.ndarray, n_vis, block: int = 8) -> np.ndarray:
    """O8, first half. Block score = the largest index score among the visible positions of the
    block ([walkthrough] 一(四)2: a block's score is the max index score inside it).

    Blocks are aligned runs of `block` positions (R-6). Returns fp32 [R, ceil(N/block)];
    blocks with no visible position are -inf.
    """
    scores = np.asarray(scores, dtype=np.float32)
    R, N = scores.shape
    nb = -(-N // block)
    n_vis = np.broadcast_to(np.asarray(n_vis), (R,))
    padded = np.full((R, nb * block), -np.inf, dtype=np.float32)
    padded[:, :N] = scores
    padded[np.arange(nb * block)[None, :] >= n_vis[:, None]] = -np.inf
    return padded.reshape(R, nb, block).max(axis=2)


def hier_pool(bmax: np.ndarray, n_vis, n_sel_blocks: int, block: int = 8) -> np.ndarray:
    """O8, second half. Choose the n_sel_blocks best blocks and gather their positions.

    [walkthrough] 一(四)2: the highest-scoring blocks are selected and the positions they cover
    form the candidate pool (2048 blocks x 8 positions = 16384 in the model). Block ties break by
    block index (R-7). The pool lists the visible positions of the chosen blocks in ascending
    order and is padded with -1 to n_sel_blocks * block.
    """
    bmax = np.asarray(bmax, dtype=np.float32)
    R, nb = bmax.shape
    n_vis = np.broadcast_to(np.asarray(n_vis), (R,))
    n_valid_blocks = -(-n_vis // block)
    chosen = topk(bmax, n_sel_blocks, n_valid=n_valid_blocks)   # ascending block ids, -1 pad
    pool = np.full((R, n_sel_blocks * block), -1, dtype=np.int64)
    for r in range(R):
        blocks = chosen[r][chosen[r] >= 0]
        pos = (blocks[:, None] * block + np.arange(block)[None, :]).reshape(-1)
        pos = pos[pos < n_vis[r]]
        pool[r, : len(pos)] = pos
    return pool


def pool_scores(q_idx: np.ndarray, k_idx: np.ndarray, pool: np.ndarray) -> np.ndarray:
    """O9. Indexer scores evaluated only at the candidate positions of each query row.

    [walkthrough] 一(四)2: later Reindex layers score only the candidate positions of the
    query. Returns fp32 [R, P]; slots holding -1 are -inf.
    """
    q = np.asarray(q_idx, dtype=np.float64)
    R, P = pool.shape
    out = np.full((R, P), -np.inf, dtype=np.float32)
    for r in range(R):
        valid = pool[r] >= 0
        s = index_scores(q[r:r + 1], np.asarray(k_idx)[pool[r][valid]], [int(valid.sum())])
        out[r, valid] = s[0]
    return out


# ---------------------------------------------------------------------------------------------
# O10: sparse attention over the selected entries.
# ---------------------------------------------------------------------------------------------
def sparse_attn(q: np.ndarray, kv: np.ndarray, idx: np.ndarray, sm_scale: float):
    """O10. Softmax attention of each query head over its selected entries.

    [walkthrough] 一(四): each query attends to its selected main-KV entries; one latent per
    entry serves as key and value (MQA, reading R-5); 一(五)4: entries are dequantized first.
    q: [R, H, D] exact values; kv: [N, D] dequantized fp64 entries; idx: [R, K] positions,
    -1 = no entry. For each (r, h): l_j = sm_scale * q[r,h].kv[j] over selected j,
    o = sum_j softmax(l)_j kv[j], lse = log(sum_j exp(l_j)). No selected entry: o = 0, lse = -inf.
    Returns (out fp32 [R, H, D], lse fp32 [R, H]).
    """
    q = np.asarray(q, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    R, H, D = q.shape
    out = np.zeros((R, H, D), dtype=np.float64)
    lse = np.full((R, H), -np.inf, dtype=np.float64)
    for r in range(R):
        sel = idx[r][idx[r] >= 0]
        if len(sel) == 0:
            continue
        x = kv[sel]                                      # [S, D]
        logits = sm_scale * (q[r] @ x.T)                 # [H, S]
        mx = logits.max(axis=1, keepdims=True)
        w = np.exp(logits - mx)
        den = w.sum(axis=1, keepdims=True)
        out[r] = (w @ x) / den
        lse[r] = mx[:, 0] + np.log(den[:, 0])
    return out.astype(np.float32), lse.astype(np.float32)


# ---------------------------------------------------------------------------------------------
# O12: the sliding-window branch, joined to the selected entries.
# ---------------------------------------------------------------------------------------------
SWA_EXP_MIN, SWA_EXP_MAX = -15, 7   # row exponents: every dequantized value stays exact in f16


def quantize_swa_fp8(x: np.ndarray):
    """O12a. FP8 storage of the layer's own sliding-window KV.

    [walkthrough] 一(五)4: the SWA KV is more sensitive to quantization and keeps FP8 precision.
    The pages give no FP8 layout; reading R-17: every channel is an OCP E4M3 code and every row
    has one power-of-two scale 2^e, e the smallest integer with max|x| <= 448 * 2^e (clamped to
    [SWA_EXP_MIN, SWA_EXP_MAX]; a zero row takes SWA_EXP_MIN). A code is the E4M3 value nearest to
    x / 2^e (exact: a power-of-two scaling), ties to the even code, saturating at 448, with the
    sign bit of x. Returns (codes uint8 [n, D], exps int8 [n]).
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    amax = np.abs(x).max(axis=1)
    e = np.full(amax.shape, SWA_EXP_MIN, dtype=np.int64)
    nz = amax > 0
    est = np.ceil(np.log2(amax[nz] / 448.0)).astype(np.int64)
    # correct the estimate so that 448 * 2^(e-1) < amax <= 448 * 2^e holds exactly
    est = np.where(amax[nz] > 448.0 * np.ldexp(1.0, est), est + 1, est)
    est = np.where(amax[nz] <= 448.0 * np.ldexp(1.0, est - 1), est - 1, est)
    e[nz] = est
    e = np.clip(e, SWA_EXP_MIN, SWA_EXP_MAX)
    y = np.abs(x) * np.ldexp(1.0, -e)[:, None]
    mag = _nearest_even(E4M3_POS, y)
    codes = (mag | (np.signbit(x).astype(np.int64) << 7)).astype(np.uint8)
    return codes, e.astype(np.int8)


def dequant_swa_fp8(codes: np.ndarray, exps: np.ndarray) -> np.ndarray:
    """O12b. x = E4M3(code) * 2^e per row (exact; R-17)."""
    return e4m3_decode(codes) * np.ldexp(1.0, np.asarray(exps, dtype=np.int64))[..., None]


def prefill_windows(buf: np.ndarray, n_win, W: int) -> np.ndarray:
    """O12d. The window rows of each query token of one sequence in prefill.

    [walkthrough] 一(四): each query attends to its own layer's sliding window, which ends at the
    query's own token. Reading R-21: the sequence's window buffer holds T + W - 1 rows, row i
    being token p0 - W + 1 + i (p0 = the first query's position); query t takes its last
    n = min(n_win[t], W) tokens up to its own, buffer rows t + W - n .. t + W - 1 (n < W only near
    the start of the sequence). buf: [T + W - 1, D]; returns win [T, W, D] with those rows first
    (the layout sparse_attn_swa takes)."""
    buf = np.asarray(buf)
    T = buf.shape[0] - W + 1
    win = np.zeros((T, W) + buf.shape[1:], dtype=buf.dtype)
    for t in range(T):
        n = min(int(n_win[t]), W)
        if n > 0:
            win[t, :n] = buf[t + W - n: t + W]
    return win


def sparse_attn_swa(q: np.ndarray, kv: np.ndarray, idx: np.ndarray, win: np.ndarray, n_win, sm_scale: float):
    """O12c. Attention of each query head over its selected entries and its window, as one softmax.

    [walkthrough] 一(四): each query attends both to the selected entries and to its own layer's
    sliding-window KV (reading R-18: one softmax over the union; the window rows are key and value
    like the main entries, R-5). q: [R, H, D]; kv: [N, D] dequantized main entries; idx: [R, K]
    (-1 = none); win: [R, W, D] dequantized window rows, of which the first n_win[r] belong to
    row r. Returns (out fp32 [R, H, D], lse fp32 [R, H]); nothing to attend: 0 and -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    win = np.asarray(win, dtype=np.float64)
    R, H, D = q.shape
    n_win = np.broadcast_to(np.asarray(n_win), (R,))
    out = np.zeros((R, H, D), dtype=np.float64)
    lse = np.full((R, H), -np.inf, dtype=np.float64)
    for r in range(R):
        sel = idx[r][idx[r] >= 0]
        x = np.concatenate([kv[sel], win[r, : int(n_win[r])]], axis=0)   # [S, D]
        if len(x) == 0:
            continue
        logits = sm_scale * (q[r] @ x.T)
        mx = logits.max(axis=1, keepdims=True)
        w = np.exp(logits - mx)
        den = w.sum(axis=1, keepdims=True)
        out[r] = (w @ x) / den
        lse[r] = mx[:, 0] + np.log(den[:, 0])
    return out.astype(np.float32), lse.astype(np.float32)


# ---------------------------------------------------------------------------------------------
# O11: one CSA2 layer step for one sequence.
# ---------------------------------------------------------------------------------------------
FULL, REINDEX, REUSE = 0, 1, 2


def layer_step(mode: int, *, q, kv_deq, k_idx=None, q_idx=None, n_vis=None, k=None,
               shared_topk=None, pool=None, pool_blocks: int = 0, block: int = 8,
               sm_scale: float = 1.0 / np.sqrt(512.0), win=None, n_win=None):
    """O11. One layer of one sequence in the given static mode.

    [walkthrough] 一(四)1: every layer computes its own query; Full scores all visible entries
    with its own indexer query and produces new Top-K; Reindex re-scores the shared keys with
    its own indexer query and produces new Top-K; Reuse attends with the newest Top-K of the
    latest index-producing layer and computes no indexer query and no score. 一(四)2: with the
    hierarchical indexer the Full layer also builds the candidate pool (pool_blocks > 0) and a
    Reindex layer given a pool scores only the pool (reading R-9: the Full layer itself attends
    over its flat Top-K). With a window (win [R, W, D] dequantized rows, n_win [R]) the attention
    is O12c's, over the selected entries and the window as one softmax (一(四), reading R-18).
    Returns dict(out, lse, topk, pool, scores).
    """
    res = {"pool": pool, "scores": None}
    if mode == REUSE:
        sel = shared_topk
    elif mode == FULL or pool is None:
        s = index_scores(q_idx, k_idx, n_vis)
        sel = topk(s, k, n_valid=n_vis)
        res["scores"] = s
        if mode == FULL and pool_blocks > 0:
            res["pool"] = hier_pool(block_max(s, n_vis, block), n_vis, pool_blocks, block)
    else:  # REINDEX on the candidate pool
        s = pool_scores(q_idx, k_idx, pool)
        sel = topk(s, k, col_to_pos=pool)
        res["scores"] = s
    if win is None:
        out, lse = sparse_attn(q, kv_deq, sel, sm_scale)
    else:
        out, lse = sparse_attn_swa(q, kv_deq, sel, win, n_win, sm_scale)
    res.update(out=out, lse=lse, topk=sel)
    return res
