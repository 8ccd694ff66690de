// Internal launchers of the CSA2 kernels (host side). Each validates nothing: the C-ABI layer in
// csa2_api.cpp checks arguments before calling these.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/csa2.h"

namespace csa2 {

// fp4_codec.hip
hipError_t launch_quantize(const void* src, bool bf16, int64_t n_rows, int dim, uint8_t* rows,
                           hipStream_t s);
hipError_t launch_dequant(const uint8_t* rows, int64_t n_rows, int dim, float* out, hipStream_t s);

// Compute units of the current device (queried once per device; 256 if the query fails).
int device_cu_count();

// index_decode.hip: streaming indexer (flat or pool), optional fused 8-block max
hipError_t launch_index_stream(const uint16_t* q, const uint16_t* k, int B, int T, int Hi, int Hk,
                               int Di, int n_max, const int32_t* n_vis, const int32_t* cand, int P,
                               float* scores, float* block_max, hipStream_t s);

// index_mxfp4.hip: streaming indexer over MXFP4 query and key rows: Hk == Hi with Hi*Di = 256
// or 512, or one shared key of Di = 128 channels (Hk == 1) and Hi query heads
// (the shared-key form also scores a candidate pool, or writes the 8-entry block max)
hipError_t launch_index_mxfp4(const uint8_t* q, const uint8_t* k, int B, int T, int Hi, int Hk, int Di,
                              int n_max, const int32_t* n_vis, const int32_t* cand, int P, float* scores,
                              float* block_max, hipStream_t s);

// index_mxfp4_prefill.hip: many query rows on the scaled FP4 MFMA (Hk == Hi, 256 or 512 channels)
bool index_mxfp4_prefill_supported(int T, int Hi, int Hk, int Di);
hipError_t launch_index_mxfp4_prefill(const uint8_t* q, const uint8_t* k, int B, int T, int Hi, int Di, int n_max,
                                      const int32_t* n_vis, float* scores, hipStream_t s);

// index_prefill.hip: MFMA tiles for many query rows, causal tile skipping
bool index_prefill_supported(int T, int Hi, int Hk, int Di);
hipError_t launch_index_prefill(const uint16_t* q, const uint16_t* k, int B, int T, int Hi, int Di,
                                int n_max, const int32_t* n_vis, float* scores, hipStream_t s);
hipError_t launch_prefill_visibility(const int64_t* p0, int B, int T, int ratio, int n_max, int32_t* n_vis,
                                     hipStream_t s);

// compress.hip: compressor (ratio 1, 2, 4 or 8 tokens per entry) + FP4 packing + indexer-K
// projection (c_out = Hk * Di key channels; k_idx may be null: no projection)
bool compress_ratio_supported(int ratio);
hipError_t launch_compress_kv(const uint16_t* c, const uint16_t* z, int B, int n_tok, int ratio,
                              const int32_t* entry0, int n_max, uint8_t* rows, const uint16_t* w_t, int c_out,
                              uint16_t* k_idx, float* entries, hipStream_t s);

// topk.hip
size_t topk_workspace(int64_t rows, int n_cols, int k);
// n_valid[r] (nullable) counts valid entries; ceil(n_valid[r] / valid_div) columns take part.
// expand_block > 0 writes each chosen column c as positions c*b .. c*b+b-1 (those >= expand_n_vis[r]
// become -1, or >= expand_limit when expand_n_vis is null); the candidate-pool form.
hipError_t launch_topk(const float* scores, int64_t rows, int n_cols, const int32_t* n_valid,
                       int valid_div, const int32_t* col_to_pos, int k, int32_t* idx,
                       int expand_block, const int32_t* expand_n_vis, int expand_limit, void* ws,
                       hipStream_t s);
// Top-K over the positions listed in cand [rows, P] (-1 = empty), scored from the full score rows
// scores [rows, n_max]; the chosen positions are written ascending. Scratch as topk_workspace(rows, P, k).
hipError_t launch_topk_gather(const float* scores, int n_max, int64_t rows, const int32_t* cand, int P, int k,
                              int32_t* idx, void* ws, hipStream_t s);
// Both selections of an HSI Full layer in one kernel (one workgroup per row): the pool of the
// pool_blocks best blocks of block_max [rows, n_blocks] (as launch_topk with expand 8), then the
// k best of the scores [rows, n_max] at the pool's positions (as launch_topk_gather). Returns
// hipErrorNotSupported for sizes it does not cover (4096 < n_blocks <= 40960, 256 < pool_blocks
// <= 2048); the caller then uses the two launches.
hipError_t launch_pool_topk(const float* block_max, int64_t rows, int n_blocks, const int32_t* n_vis,
                            int pool_blocks, int32_t* pool, const float* scores, int n_max, int k, int32_t* idx,
                            hipStream_t s);

// sparse_attn.hip
size_t attn_workspace(int B, int T, int H, int D, int K);
size_t attn_swa_workspace(int B, int H, int D, int K);
size_t attn_swa_prefill_workspace(int B, int T, int H, int D, int K);
hipError_t launch_sparse_attn_swa_prefill(const uint16_t* q, const uint8_t* rows, int n_max, const int32_t* idx,
                                          int B, int T, int H, int D, int K, const uint8_t* swa_codes,
                                          const int8_t* swa_exp, const int32_t* n_win, int W, float sm_scale,
                                          float* out, float* lse, void* ws, hipStream_t s);
hipError_t launch_sparse_attn_swa(const uint16_t* q, const uint8_t* rows, int n_max, const int32_t* idx, int B,
                                  int H, int D, int K, const uint8_t* swa_codes, const int8_t* swa_exp,
                                  const int32_t* n_win, int W, float sm_scale, float* out, float* lse, void* ws,
                                  hipStream_t s);
hipError_t launch_sparse_attn(const uint16_t* q, const uint8_t* rows, int n_max, const int32_t* idx,
                              int B, int T, int H, int D, int K, float sm_scale, float* out,
                              float* lse, void* ws, hipStream_t s);

}  // namespace csa2
