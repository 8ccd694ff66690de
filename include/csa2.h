/*
 * csa2.h - C ABI of the CSA2 sparse-attention hot path with an FP4 main KV cache, for AMD
 * MI355X (gfx950).
 *
 * What is computed follows the model pages on DeepSeek-V4.1-Flash:
 *   [walkthrough]  "DeepSeek-V4.1-Flash" tech-report walkthrough (wkq9411.github.io):
 *                  section 一(四) Compressed Sparse Attention 2 (indexer, Top-K, attention over
 *                  the selected entries), 一(四)1 Cross-Layer KV and Index Reuse (Full / Reindex /
 *                  Reuse), 一(四)2 Hierarchical Sparse Indexer (block max, block selection,
 *                  candidate pool), 一(五)4 FP4 Main KV Cache (E2M1 values, one E4M3 scale per
 *                  16 channels, no global scale, dequantized before attention).
 *   [release note] ModelScope release note, section 压缩稀疏注意力 2（CSA2）.
 *
 * Conventions shared by every call
 *   - Every data pointer is a DEVICE pointer owned by the caller, unless a comment says "host".
 *     The library never allocates, frees or synchronizes; scratch space comes from a caller
 *     buffer `ws` whose size the matching *_workspace_size call returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). Calls only enqueue
 *     work on it and return; results are valid once the caller has synchronized the stream.
 *   - Return codes report synchronous argument / shape / state checks and launch errors only.
 *     Device faults surface at the caller's next synchronization (the HIP convention).
 *     On any non-OK return nothing has been enqueued, except CSA2_E_HIP (a launch failed
 *     part-way).
 *   - bf16 tensors are passed as uint16_t bit patterns. All arrays are dense row-major.
 *   - Scores and query values must be finite (-inf is allowed for scores); this is a
 *     precondition, not checked.
 *   - Calls that overlap on one stream are ordered; the library keeps no state between calls
 *     and is reentrant.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CSA2_OK = 0,
  CSA2_E_ARG = 1,          /* null pointer, negative size, bad enum */
  CSA2_E_SHAPE = 2,        /* unsupported or inconsistent shape */
  CSA2_E_STATE = 3,        /* Reindex/Reuse without the shared state they need */
  CSA2_E_WORKSPACE = 4,    /* workspace missing, smaller than required or misaligned */
  CSA2_E_UNSUPPORTED = 5,  /* valid request the library does not implement */
  CSA2_E_HIP = 6           /* a HIP launch failed */
} csa2_status;

typedef enum { CSA2_FULL = 0, CSA2_REINDEX = 1, CSA2_REUSE = 2 } csa2_mode;
typedef enum { CSA2_F32 = 0, CSA2_BF16 = 1 } csa2_dtype;

/* Packed entry size in bytes for `dim` channels: dim/2 code bytes + dim/16 scale bytes
 * (288 for the 512-channel latent). */
#define CSA2_ROW_BYTES(dim) ((dim) / 2 + (dim) / 16)

const char* csa2_status_string(csa2_status s);

/* ------------------------------------------------------------------------------------------
 * csa2_quantize_kv_fp4 - pack entries into the FP4 main-KV format.
 * [walkthrough] 一(五)4: E2M1 values with one E4M3 scale per 16 channels, no global scale,
 * quantized after RoPE (so all channels are treated alike).
 *
 * src       [n_rows, dim] fp32 or bf16 (src_dtype) values, finite.
 * rows      [n_rows, dim/2 + dim/16] bytes, written. Byte i < dim/2 holds channel 2i in its low
 *           nibble and channel 2i+1 in its high nibble; byte dim/2 + g holds the E4M3 scale of
 *           channels 16g .. 16g+15.
 * Rounding: per group, scale = the E4M3 value nearest to amax/6 (ties to the even code,
 *           saturating at 448; amax = largest |x|); each code = sign bit of x and the E2M1
 *           magnitude nearest to |x|/scale (ties to even, saturating at 6); a zero scale gives
 *           zero magnitudes. All decisions are exact comparisons.
 * dim       multiple of 64, at most 4096.  n_rows >= 0 (0 enqueues nothing).
 * ------------------------------------------------------------------------------------------ */
csa2_status csa2_quantize_kv_fp4(const void* src, csa2_dtype src_dtype, int64_t n_rows,
                                 int32_t dim, uint8_t* rows, void* stream);

/* csa2_dequant_kv_fp4 - inverse of the packing: out[r, c] = E2M1(code) * E4M3(scale), exact.
 * [walkthrough] 一(五)4: the cache is dequantized before attention. The attention kernel
 * dequantizes in registers/LDS; this stand-alone form writes fp32 [n_rows, dim]. */
csa2_status csa2_dequant_kv_fp4(const uint8_t* rows, int64_t n_rows, int32_t dim, float* out,
                                void* stream);

/* ------------------------------------------------------------------------------------------
 * csa2_compress_kv - producing the caches: compressor, FP4 packing and indexer-K projection.
 * [walkthrough] 一(三): a layer's KV entries C and their compression weights Z are projections
 * of the hidden states (C = H W^KV, Z = H W^Z); 一(四): CSA2's compressor turns every `ratio`
 * consecutive tokens into one main-KV entry, without CSA's overlap between neighbouring entries
 * and without an absolute position encoding, and indexer K is obtained by projecting the main-KV
 * entries; 一(五)4: the entries are stored as FP4 (E2M1 + one E4M3 scale per 16 channels).
 *
 * For sequence b, new entry j (j < n_tok / ratio) is made from tokens j*ratio .. j*ratio+ratio-1:
 *   e[d] = sum_i w_i[d] c[b, j*ratio + i, d],   w_.[d] = softmax over the group's z[b, ., d]
 * (fp32; reading of the pages: softmax weights per channel). It is written, packed as
 * csa2_quantize_kv_fp4 packs an fp32 row, to rows[b, entry0[b] + j], and its indexer key
 *   k_idx[b, entry0[b] + j, o] = bf16( sum_d bf16(e[d]) * w_t[o, d] ),  o < Hk * Di
 * (bf16 products, fp32 accumulation, rounded to nearest even). Entries whose index
 * entry0[b] + j falls outside [0, n_max) are not written.
 *
 * c, z     [B, n_tok, D] bf16 (16-byte aligned): the new tokens' KV values and compression weights.
 * ratio    tokens per entry: 1, 2, 4 or 8; n_tok a multiple of it. D == 512.
 * entry0   [B] int32 (device): index of each sequence's first new entry in its cache.
 * rows     [B, n_max, D/2 + D/16] bytes: the FP4 cache, new entries written.
 * w_t      [Hk*Di, D] bf16 projection weight (row o: the D input weights of key channel o), and
 * k_idx    [B, n_max, Hk, Di] bf16 indexer keys, new entries written; both NULL: no projection.
 *          Hk*Di a multiple of 128, at most 1024.
 * entries  NULL, or [B, n_tok/ratio, D] fp32: the compressed entries before packing (for checks).
 * ------------------------------------------------------------------------------------------ */
csa2_status csa2_compress_kv(const uint16_t* c, const uint16_t* z, int32_t B, int32_t n_tok, int32_t D,
                             int32_t ratio, const int32_t* entry0, int32_t n_max, uint8_t* rows,
                             const uint16_t* w_t, int32_t Hk, int32_t Di, uint16_t* k_idx, float* entries,
                             void* stream);

/* ------------------------------------------------------------------------------------------
 * csa2_index_scores - the lightweight indexer.
 * [walkthrough] 一(四): indexer Q and indexer K score the main-KV entries; 一(四)2: later
 * layers may score only a candidate pool.
 *
 * score[r, n] = sum_{h < Hi} sum_{d < Di} q_idx[r, h, d] * k_idx[b(r), n, h', d]
 *   with r = b*T + t, h' = h if Hk == Hi, h' = 0 if Hk == 1. Products are exact, the sum is
 *   fp32 (so results match an exact sum to about 1e-6 of sum |q*k|).
 *
 * q_idx     [B, T, Hi, Di] bf16.
 * k_idx     [B, n_max, Hk, Di] bf16.
 * n_vis     [B*T] int32 visible entries per query row (device), or NULL for all n_max.
 *           Entries n >= n_vis[r] are not scored; their score slots are left unwritten.
 * cand      NULL: flat mode, scores is [B*T, n_max].
 *           else [B*T, P] int32 positions per query row (pool mode, -1 = empty slot);
 *           scores is [B*T, P] and slot p holds the score of position cand[r, p]
 *           (-inf for an empty slot or a position outside [0, n_max)).
 * block_max NULL, or (flat mode only) [B*T, ceil(n_max / block)]: the max score over the
 *           visible positions of each aligned block of `block` entries ([walkthrough]
 *           一(四)2, a block's score is the max index score inside it). Blocks with no visible
 *           position are left unwritten. block must be 8 when block_max is given.
 * Requires Hk in {1, Hi}, Di % 8 == 0, and Hi*Di <= 1024 when Hk == Hi, or Di <= 1024 and
 * Hi*Di <= 8192 when Hk == 1 (one shared key: the query heads are summed in fp32 first, so the
 * score is (sum_h q_idx[r, h]) . k_idx[n, 0]).
 * Prefill calls (T >= 16, flat mode without block_max, Hk == Hi, Hi*Di % 64 == 0) run as MFMA
 * tiles with causal tile skipping. Every other call streams the keys once per query row and
 * needs a key row of Hk*Di in {64, 128, 256, 512, 1024} channels. Other shapes: CSA2_E_SHAPE.
 * ------------------------------------------------------------------------------------------ */
csa2_status csa2_index_scores(const uint16_t* q_idx, const uint16_t* k_idx, int32_t B, int32_t T,
                              int32_t Hi, int32_t Hk, int32_t Di, int32_t n_max,
                              const int32_t* n_vis, const int32_t* cand, int32_t P,
                              float* scores, float* block_max, int32_t block, void* stream);

/* ------------------------------------------------------------------------------------------
 * csa2_prefill_visibility - causal visibility of the compressed entries for a prefill chunk.
 * [walkthrough] 一(四): a query scores only the compressed entries it may see. An entry
 * compresses `ratio` consecutive tokens and becomes visible once its last source token is at or
 * before the query's own position p, so the query sees entries n < floor((p + 1) / ratio).
 *
 * p0     [B] int64 (device): absolute position of the first query token of each sequence.
 * n_vis  [B*T] int32 (device), written: n_vis[b*T + t] = min(n_max, floor((p0[b] + t + 1) / ratio)),
 *        and 0 where that is negative. Feeds the n_vis argument of the indexer, Top-K and layer calls.
 * ratio > 0; B, T, n_max >= 0 (B*T == 0 enqueues nothing).
 * ------------------------------------------------------------------------------------------ */
csa2_status csa2_prefill_visibility(const int64_t* p0, int32_t B, int32_t T, int32_t ratio, int32_t n_max,
                                    int32_t* n_vis, void* stream);

/* ------------------------------------------------------------------------------------------
 * csa2_index_scores_mxfp4 - the lightweight indexer over FP4 query and key rows.
 * [walkthrough] 一(五)4: the indexer query and key are FP4 in the OCP MXFP4 format (E2M1
 * elements, one E8M0 power-of-two scale per 32 channels); 一(四): the indexer scores every
 * main-KV entry.
 *
 * An MXFP4 row of C channels is C/2 code bytes (channel 2i in the low nibble of byte i)
 * followed by C/32 E8M0 scale codes (value 2^(code - 127)) of channels 32j .. 32j+31.
 * Key rows hold an entry's Hk * Di channels, query rows a query's Hi * Di channels (head h at
 * channels h*Di ..). score[r, n] = sum_h q[r, h] . k[b(r), n, h'] over the dequantized values,
 * h' = h (Hk == Hi) or 0 (Hk == 1, one shared key), r = b*T + t. With Hk == Hi each 32-channel
 * block's sum is exact and the blocks' scaled sums are added in fp32; with a shared key the
 * heads are summed in fp32 first.
 *
 * q_rows  [B*T, Hi*Di/2 + Hi*Di/32] bytes, k_rows [B, n_max, Hk*Di/2 + Hk*Di/32] bytes (8-byte
 *         aligned bases).
 * n_vis   [B*T] int32 visible entries per query row (device), or NULL for all n_max; entries
 *         n >= n_vis[r] are not scored and their slots are left unwritten (flat mode).
 * cand, P, block_max, block: as csa2_index_scores (pool mode: scores [B*T, P], slot p holds the
 *         score of position cand[r, p] or -inf; flat mode: the max of every aligned block of 8
 *         visible entries, block == 8; CSA2_E_UNSUPPORTED for block_max with cand or another
 *         block).
 * scores  [B*T, n_max] fp32 (flat) or [B*T, P] (pool).
 * Requires Hk == Hi with Hi * Di in {256, 512}, or Hk == 1, Di == 128 and Hi <= 64
 * (CSA2_E_SHAPE otherwise); finite scales (code 255 is NaN).
 * Decode-shaped calls stream the keys once per query row on the vector ALUs. Prefill calls (T >= 16,
 * flat mode without block_max, Hk == Hi) run as tiles on the scaled FP4 matrix cores
 * (v_mfma_scale_f32_32x32x64_f8f6f4: the rows' 32-channel blocks and E8M0 scales are its operand
 * format), exact products accumulated in fp32, with causal tile skipping.
 * ------------------------------------------------------------------------------------------ */
csa2_status csa2_index_scores_mxfp4(const uint8_t* q_rows, const uint8_t* k_rows, int32_t B,
                                    int32_t T, int32_t Hi, int32_t Hk, int32_t Di, int32_t n_max,
                                    const int32_t* n_vis, const int32_t* cand, int32_t P,
                                    float* scores, float* block_max, int32_t block, void* stream);

/* ------------------------------------------------------------------------------------------
 * csa2_topk - Top-K selection per row.
 * [walkthrough] 一(四): each query keeps its Top-K entries (512 in the model, 三(二)1).
 *
 * Chooses, for each row r, the k best columns among c < n_valid[r] (all n_cols if n_valid is
 * NULL) whose position is >= 0, ordered by score descending then position ascending, and
 * writes their positions in ASCENDING order to idx[r, 0 ..), padding with -1 up to k.
 * position(c) = c, or col_to_pos[r, c] when col_to_pos is given (pool slot -> global position;
 * the pool must be ascending in its valid slots, which csa2_hier_pool guarantees).
 * -0.0 and +0.0 are equal scores. The result is deterministic.
 *
 * scores     [rows, n_cols] fp32.     idx  [rows, k] int32, written.
 * Limits     k <= 4096, n_cols <= 2^26 (CSA2_E_SHAPE otherwise).
 * ws         scratch of csa2_topk_workspace_size() bytes (may be NULL if that size is 0).
 * ------------------------------------------------------------------------------------------ */
size_t csa2_topk_workspace_size(int64_t rows, int32_t n_cols, int32_t k);
csa2_status csa2_topk(const float* scores, int64_t rows, int32_t n_cols, const int32_t* n_valid,
                      const int32_t* col_to_pos, int32_t k, int32_t* idx, void* ws,
                      size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * csa2_hier_pool - candidate pool of the Hierarchical Sparse Indexer.
 * [walkthrough] 一(四)2: the first Full layer scores every visible position, takes each
 * block's max, selects the highest-scoring blocks, and the positions they cover form the pool
 * that later Reindex layers score (2048 blocks x 8 = 16384 positions in the model).
 *
 * block_max  [rows, n_blocks] fp32 (from csa2_index_scores).
 * n_vis      [rows] visible positions per row (device) or NULL (= n_blocks * block).
 *            Blocks at or beyond ceil(n_vis / block) do not take part.
 * pool       [rows, n_sel_blocks * block] int32, written: the visible positions of the chosen
 *            blocks (block ties broken by block index) in ascending order, then -1.
 * ws         scratch of csa2_hier_pool_workspace_size() bytes.
 * Limits     n_sel_blocks <= 4096, block <= 64.
 * ------------------------------------------------------------------------------------------ */
size_t csa2_hier_pool_workspace_size(int64_t rows, int32_t n_blocks, int32_t n_sel_blocks);
csa2_status csa2_hier_pool(const float* block_max, int64_t rows, int32_t n_blocks,
                           const int32_t* n_vis, int32_t block, int32_t n_sel_blocks,
                           int32_t* pool, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * csa2_sparse_attn - attention of each query over its selected FP4 entries.
 * [walkthrough] 一(四): each query attends to its selected main-KV entries; one 512-channel
 * latent per entry is both key and value (MQA over H heads); 一(五)4: entries are dequantized
 * before attention.
 *
 * For each (b, t, h): l_j = sm_scale * q[b,t,h,:] . x_j over selected j, out = sum softmax(l)_j
 * x_j, lse = ln sum_j exp(l_j), with x_j the dequantized entry idx[b,t,j] of sequence b.
 * Indices < 0 or >= n_max are skipped; with nothing selected out = 0 and lse = -inf.
 * q K^T and P V run on f16 MFMA with fp32 accumulation: dequantized entries are exact in f16
 * (at most 6 significant bits, magnitudes 2^-10 .. 2688); each head's bf16 query is scaled by a
 * power of two that puts its largest |q| in [2^14, 2^15) and then converted to f16, which is exact
 * for every component within 2^31 of that largest one (smaller ones round to f16 subnormals, an
 * error below 2^-24 of the head's largest |q|); the power of two is folded back into the softmax
 * scale. Softmax in fp32; probabilities are rounded to f16 for P V.
 *
 * q     [B, T, H, D] bf16.        rows [B, n_max, D/2 + D/16] bytes (16-byte aligned base).
 * idx   [B, T, K] int32.          out  [B, T, H, D] fp32.   lse [B, T, H] fp32 or NULL.
 * Requires D == 512, H % 16 == 0, K <= 4096 (the Top-K limit; CSA2_E_SHAPE otherwise).
 * ws    scratch of csa2_sparse_attn_workspace_size() bytes (split-K partial results).
 * ------------------------------------------------------------------------------------------ */
size_t csa2_sparse_attn_workspace_size(int32_t B, int32_t T, int32_t H, int32_t D, int32_t K);
csa2_status csa2_sparse_attn(const uint16_t* q, const uint8_t* rows, int32_t n_max,
                             const int32_t* idx, int32_t B, int32_t T, int32_t H, int32_t D,
                             int32_t K, float sm_scale, float* out, float* lse, void* ws,
                             size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * csa2_sparse_attn_swa - decode attention over the selected FP4 entries joined with the
 * layer's own sliding window of FP8 rows, as one softmax.
 * [walkthrough] 一(四): each query attends to its selected entries and to its own layer's
 * sliding-window KV; 一(五)4: that KV stays in FP8; 三(二)1: the window is 128 tokens.
 *
 * One query token per sequence (T = 1). For each (b, h) the softmax runs over the selected
 * entries of idx[b] (as csa2_sparse_attn) and the window rows 0 .. n_win[b]-1 of sequence b:
 *   window row value = E4M3(swa_codes[b, w, c]) * 2^swa_exp[b, w]   (exact in f16)
 * out = sum over the union of softmax(l) * x, lse = ln sum exp(l); nothing to attend: 0, -inf.
 * The selected entries are split over workgroups as in the decode form of csa2_sparse_attn,
 * the window over up to two more slots of 64 rows, or up to four of 32 rows when fewer than 256
 * workgroups would run otherwise; their partial softmaxes meet in one combine pass.
 *
 * q         [B, H, D] bf16.          rows, n_max, idx [B, K], K: as csa2_sparse_attn with T = 1.
 * swa_codes [B, W, D] uint8 OCP E4M3 codes (16-byte aligned base); swa_exp [B, W] int8 row
 *           exponents in [-15, 7] (outside that range the f16 products are not exact).
 * n_win     [B] int32 (device): window rows of each sequence, clamped to [0, W].
 * W         rows reserved per sequence, W <= 128 (CSA2_E_SHAPE otherwise).
 * out       [B, H, D] fp32.          lse [B, H] fp32 or NULL.
 * ws        scratch of csa2_sparse_attn_swa_workspace_size() bytes (never NULL; partial
 *           results of every split, independent of W).
 * Requires D == 512, H % 16 == 0, K <= 4096.
 * ------------------------------------------------------------------------------------------ */
size_t csa2_sparse_attn_swa_workspace_size(int32_t B, int32_t H, int32_t D, int32_t K);
csa2_status csa2_sparse_attn_swa(const uint16_t* q, const uint8_t* rows, int32_t n_max,
                                 const int32_t* idx, int32_t B, int32_t H, int32_t D, int32_t K,
                                 const uint8_t* swa_codes, const int8_t* swa_exp,
                                 const int32_t* n_win, int32_t W, float sm_scale, float* out,
                                 float* lse, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * csa2_sparse_attn_swa_prefill - attention of many query tokens over their selected FP4
 * entries joined with each token's own sliding window of FP8 rows, as one softmax.
 * [walkthrough] 一(四): each query attends to its selected entries and to its own layer's
 * sliding-window KV, which ends at the query's own token; 一(五)4: that KV is FP8.
 *
 * For each (b, t, h) the softmax runs over the selected entries of idx[b, t] (as
 * csa2_sparse_attn) and the window of query t: the sequence's buffer holds T + W - 1 rows (row i
 * = token p0 - W + 1 + i, p0 = position of query 0), and query t takes its last
 * n = min(n_win[b, t], W) tokens up to its own, rows t + W - n .. t + W - 1 (n < W near the start
 * of the sequence). Row values as csa2_sparse_attn_swa. out / lse as csa2_sparse_attn.
 *
 * q [B, T, H, D] bf16; rows, n_max, idx [B, T, K], K <= 4096: as csa2_sparse_attn.
 * swa_codes [B, T + W - 1, D] uint8 E4M3 codes (16-byte aligned); swa_exp [B, T + W - 1] int8
 *           exponents in [-15, 7]; n_win [B, T] int32 (device); W <= 128.
 * out [B, T, H, D] fp32; lse [B, T, H] fp32 or NULL.
 * ws        scratch of csa2_sparse_attn_swa_prefill_workspace_size() bytes, 256-byte aligned;
 *           may be NULL when that size is 0 (B * T >= 512, H % 64 == 0 and 0 < K <= 1024: the
 *           window runs as further chunks of the selected entries' own pass).
 * Requires D == 512, H % 16 == 0.
 * ------------------------------------------------------------------------------------------ */
size_t csa2_sparse_attn_swa_prefill_workspace_size(int32_t B, int32_t T, int32_t H, int32_t D,
                                                   int32_t K);
csa2_status csa2_sparse_attn_swa_prefill(const uint16_t* q, const uint8_t* rows, int32_t n_max,
                                         const int32_t* idx, int32_t B, int32_t T, int32_t H,
                                         int32_t D, int32_t K, const uint8_t* swa_codes,
                                         const int8_t* swa_exp, const int32_t* n_win, int32_t W,
                                         float sm_scale, float* out, float* lse, void* ws,
                                         size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * csa2_layer_step - one CSA2 layer in its static mode.
 * [walkthrough] 一(四)1: every layer computes its own query. Full scores every visible entry
 * with its own indexer query and produces new Top-K; Reindex re-scores the latest shared keys
 * with its own indexer query and produces new Top-K; Reuse attends with the newest Top-K of
 * the latest index-producing layer and computes no indexer query and no score. Main KV and
 * indexer K come from the most recent Full layer. 一(四)2: with the hierarchical indexer the
 * (first) Full layer also builds the candidate pool and later Reindex layers score only it.
 *
 * Shared state is described by plain host structs pointing at caller-owned device buffers:
 *   csa2_shared_kv   the cache of the most recent Full layer. The caller fills the pointers
 *                    and shapes before the Full layer; FULL marks it valid.
 *   csa2_shared_idx  the newest Top-K (and pool). FULL and REINDEX write topk and set
 *                    topk_valid; FULL with use_pool writes pool and sets pool_valid.
 * Modes:
 *   FULL     (compress the layer's new tokens into the caches ->) index scores over all visible
 *            entries -> Top-K (-> block max -> pool) -> attention.
 *   REINDEX  needs kv->valid. With use_pool and idx->pool_valid it scores only the pool;
 *            otherwise all visible entries. -> Top-K -> attention.
 *   REUSE    needs kv->valid and idx->topk_valid. Attention over idx->topk only.
 * Errors: CSA2_E_STATE when the needed shared state is not valid.
 * ------------------------------------------------------------------------------------------ */
typedef struct {
  const uint8_t* rows;     /* [B, n_max, D/2 + D/16] FP4 entries */
  const uint16_t* k_idx;   /* [B, n_max, Hk, Di] bf16 indexer keys */
  const int32_t* n_vis;    /* [B*T] visible entries per query row, or NULL (= n_max) */
  int32_t B, n_max, D, Hk, Di;
  int32_t valid;           /* set by FULL */
  /* FP4 indexer keys ([walkthrough] 一(五)4, OCP MXFP4): [B, n_max, C/2 + C/32] rows of
   * C = Hk * Di channels (layout of csa2_index_scores_mxfp4), or NULL. When given, Full and
   * Reindex layers score them against the layer's q_idx_mx instead of k_idx / q_idx (shapes as
   * csa2_index_scores_mxfp4, with or without the hierarchical pool). */
  const uint8_t* k_mx;
} csa2_shared_kv;

typedef struct {
  int32_t* topk;           /* [B*T, K] positions, ascending, -1 padded */
  int32_t K;
  int32_t* pool;           /* [B*T, P] candidate positions or NULL */
  int32_t P;               /* pool capacity = pool_blocks * block */
  int32_t topk_valid, pool_valid;
} csa2_shared_idx;

typedef struct {
  const uint16_t* q;       /* [B, T, H, D] bf16 attention query of this layer */
  const uint16_t* q_idx;   /* [B, T, Hi, Di] bf16 indexer query (Full / Reindex) */
  int32_t T, H, Hi;
  float sm_scale;
  int32_t use_pool;        /* Full: build the pool; Reindex: score only the pool */
  int32_t pool_blocks;     /* blocks kept in the pool (Full with use_pool) */
  int32_t block;           /* positions per block (8) */
  float* out;              /* [B, T, H, D] fp32 */
  float* lse;              /* [B, T, H] fp32 or NULL */
  void* ws;                /* scratch of csa2_layer_workspace_size() bytes, 256-byte aligned */
  size_t ws_bytes;
  /* The layer's sliding window, joined to the selected entries as one softmax: as
   * csa2_sparse_attn_swa when T == 1, as csa2_sparse_attn_swa_prefill when T > 1 (the buffer then
   * holds T + swa_W - 1 rows per sequence and swa_n one count per query row).
   * swa_codes NULL: no window (a zero-initialized struct has none). */
  const uint8_t* swa_codes; /* [B, swa_W, D] (T == 1) or [B, T + swa_W - 1, D] E4M3 codes */
  const int8_t* swa_exp;    /* [B, swa_W] or [B, T + swa_W - 1] row exponents in [-15, 7] */
  const int32_t* swa_n;     /* [B] or [B*T] window rows (device), clamped to [0, swa_W] */
  int32_t swa_W;            /* rows reserved per sequence, <= 128 */
  const uint8_t* q_idx_mx;  /* [B*T, Hi*Di/2 + Hi*Di/32] MXFP4 indexer query, with shared_kv.k_mx */
  /* Producing the caches ([walkthrough] 一(四)1: a Full layer computes its own main KV and then
   * its indexer K from it). FULL only, with new_kv != NULL: the layer first compresses its new
   * tokens into entries new_entry0[b] .. new_entry0[b] + new_tokens/ratio - 1 of shared_kv->rows
   * and shared_kv->k_idx (written in place, as csa2_compress_kv; bf16 indexer keys only), then
   * scores every visible entry as usual. new_kv NULL (a zero-initialized struct): no production. */
  const uint16_t* new_kv;   /* [B, new_tokens, D] bf16 KV values of the new tokens */
  const uint16_t* new_z;    /* [B, new_tokens, D] bf16 compression weights */
  int32_t new_tokens;       /* a multiple of ratio */
  int32_t ratio;            /* tokens per entry: 1, 2, 4 or 8 */
  const int32_t* new_entry0; /* [B] int32 (device): first new entry of each sequence */
  const uint16_t* w_ik;     /* [Hk*Di, D] bf16 indexer-K projection weight */
} csa2_layer_args;

/* csa2_layer_workspace_size - scratch bytes csa2_layer_step needs for this layer (index scores,
 * block maxima, Top-K scratch, attention partials). It takes the shared index state too, since the
 * sizes depend on its Top-K and pool capacity. The workspace passed in a->ws must be 256-byte
 * aligned (hipMalloc and torch allocations are); csa2_layer_step returns CSA2_E_WORKSPACE for a
 * NULL, short or misaligned one. */
csa2_status csa2_layer_workspace_size(csa2_mode mode, const csa2_layer_args* a,
                                      const csa2_shared_kv* kv, const csa2_shared_idx* idx,
                                      size_t* bytes);
csa2_status csa2_layer_step(csa2_mode mode, const csa2_layer_args* a, csa2_shared_kv* kv,
                            csa2_shared_idx* idx, void* stream);

/* ------------------------------------------------------------------------------------------
 * csa2_layer_step_noalloc - csa2_layer_step for callers that cannot allocate device memory or
 * pass a workspace: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same arguments, kernels and results as csa2_layer_step, except that a->ws and
 * a->ws_bytes are ignored: the scratch comes from a fixed device array inside the library of
 * CSA2_NOALLOC_SCRATCH_BYTES (64 MiB), one copy per GPU, held until the process ends. The caller
 * still passes every input and output buffer.
 *   - CSA2_E_WORKSPACE when the layer needs more scratch than that (csa2_layer_workspace_size
 *     gives the need: every decode layer of B <= 32 sequences x 65536 entries fits; a 4096-token
 *     prefill chunk does not). Checked before anything is enqueued.
 *   - The first call on a device looks up that device's copy of the array (hipGetSymbolAddress)
 *     and keeps its address; no call allocates or frees memory.
 *   - Every call on one GPU shares that GPU's scratch, which keeps the last call's contents:
 *     calls that may overlap on one GPU (different streams without ordering between them, or
 *     several host threads) race and must be serialized by the caller. Calls in order on one
 *     stream are safe. No kernel relies on the scratch starting at zero.
 * ------------------------------------------------------------------------------------------ */
#define CSA2_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
csa2_status csa2_layer_step_noalloc(csa2_mode mode, const csa2_layer_args* a, csa2_shared_kv* kv,
                                    csa2_shared_idx* idx, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_H */
