// C ABI of the CSA2 hot path: argument and state validation, workspace layout, dispatch to the
// HIP kernels, and the per-layer mode logic of CSA2 (Full / Reindex / Reuse; DeepSeek-V4.1-Flash
// walkthrough, wkq9411.github.io, 一(四)1 and 一(四)2). No call allocates, frees or
// synchronizes; every launch goes to the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "../../include/csa2.h"
#include "launch.h"

using namespace csa2;

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

csa2_status hip_status(hipError_t e) { return e == hipSuccess ? CSA2_OK : CSA2_E_HIP; }

bool index_shape_ok(int32_t Hi, int32_t Hk, int32_t Di) {
  // per-head keys: the query and the key row are Hi*Di channels, at most 1024; one shared key:
  // the key row is Di channels (at most 1024) and the query heads are summed first (up to 8192)
  return Hi >= 1 && (Hk == Hi || Hk == 1) && Di > 0 && Di % 8 == 0 && (Hk * Di) % 64 == 0 &&
         (Hk == 1 ? Di <= 1024 && Hi * Di <= 8192 : Hi * Di <= 1024);
}

// The streaming kernel is instantiated for key rows of 64, 128, 256, 512 and 1024 channels; the
// MFMA prefill kernel takes any per-head channel count that index_shape_ok admits.
bool index_call_ok(int32_t T, int32_t Hi, int32_t Hk, int32_t Di, bool pool, bool bmax) {
  if (!index_shape_ok(Hi, Hk, Di)) return false;
  if (!pool && !bmax && index_prefill_supported(T, Hi, Hk, Di)) return true;
  const int32_t c = Hk * Di;
  return c == 64 || c == 128 || c == 256 || c == 512 || c == 1024;
}

constexpr int32_t kMaxSwaWindow = 128;   // window rows per sequence (n_win of the model)

bool attn_shape_ok(int32_t H, int32_t D) { return D == 512 && H > 0 && H % 16 == 0 && (H <= 64 || H % 64 == 0); }

constexpr int kMaxK = 4096;
constexpr int64_t kMaxCols = 1 << 26;

}  // namespace

extern "C" {

const char* csa2_status_string(csa2_status s) {
  switch (s) {
    case CSA2_OK: return "ok";
    case CSA2_E_ARG: return "invalid argument (null pointer, negative size or bad enum)";
    case CSA2_E_SHAPE: return "unsupported or inconsistent shape";
    case CSA2_E_STATE: return "shared state needed by this mode is not valid";
    case CSA2_E_WORKSPACE: return "workspace missing, too small or misaligned";
    case CSA2_E_UNSUPPORTED: return "not supported by this library";
    case CSA2_E_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

csa2_status csa2_quantize_kv_fp4(const void* src, csa2_dtype src_dtype, int64_t n_rows, int32_t dim,
                                 uint8_t* rows, void* stream) {
  if (n_rows < 0 || (src_dtype != CSA2_F32 && src_dtype != CSA2_BF16)) return CSA2_E_ARG;
  if (dim <= 0 || dim % 64 != 0 || dim > 4096) return CSA2_E_SHAPE;
  if (n_rows == 0) return CSA2_OK;
  if (!src || !rows) return CSA2_E_ARG;
  if (reinterpret_cast<uintptr_t>(src) % 16 || reinterpret_cast<uintptr_t>(rows) % 4) return CSA2_E_ARG;
  return hip_status(launch_quantize(src, src_dtype == CSA2_BF16, n_rows, dim, rows, as_stream(stream)));
}

csa2_status csa2_dequant_kv_fp4(const uint8_t* rows, int64_t n_rows, int32_t dim, float* out, void* stream) {
  if (n_rows < 0) return CSA2_E_ARG;
  if (dim <= 0 || dim % 64 != 0 || dim > 4096) return CSA2_E_SHAPE;
  if (n_rows == 0) return CSA2_OK;
  if (!rows || !out) return CSA2_E_ARG;
  if (reinterpret_cast<uintptr_t>(rows) % 4 || reinterpret_cast<uintptr_t>(out) % 16) return CSA2_E_ARG;
  return hip_status(launch_dequant(rows, n_rows, dim, out, as_stream(stream)));
}

csa2_status csa2_index_scores(const uint16_t* q_idx, const uint16_t* k_idx, int32_t B, int32_t T, int32_t Hi,
                              int32_t Hk, int32_t Di, int32_t n_max, const int32_t* n_vis, const int32_t* cand,
                              int32_t P, float* scores, float* block_max, int32_t block, void* stream) {
  if (B < 0 || T < 0 || n_max < 0 || (cand && P < 0)) return CSA2_E_ARG;
  if (!index_call_ok(T, Hi, Hk, Di, cand != nullptr, block_max != nullptr)) return CSA2_E_SHAPE;
  if (block_max && (cand || block != 8)) return CSA2_E_UNSUPPORTED;
  const int64_t rows = (int64_t)B * T;
  const int32_t ncols = cand ? P : n_max;
  if (rows == 0 || ncols == 0) return CSA2_OK;
  if (!q_idx || !k_idx || !scores) return CSA2_E_ARG;
  if (rows > INT32_MAX || ncols > kMaxCols) return CSA2_E_SHAPE;
  if (reinterpret_cast<uintptr_t>(q_idx) % 16 || reinterpret_cast<uintptr_t>(k_idx) % 16) return CSA2_E_ARG;
  hipStream_t s = as_stream(stream);
  if (!cand && !block_max && index_prefill_supported(T, Hi, Hk, Di))
    return hip_status(launch_index_prefill(q_idx, k_idx, B, T, Hi, Di, n_max, n_vis, scores, s));
  return hip_status(launch_index_stream(q_idx, k_idx, B, T, Hi, Hk, Di, n_max, n_vis, cand, P, scores,
                                        block_max, s));
}

csa2_status csa2_compress_kv(const uint16_t* c, const uint16_t* z, int32_t B, int32_t n_tok, int32_t D,
                             int32_t ratio, const int32_t* entry0, int32_t n_max, uint8_t* rows, const uint16_t* w_t,
                             int32_t Hk, int32_t Di, uint16_t* k_idx, float* entries, void* stream) {
  if (B < 0 || n_tok < 0 || n_max < 0 || ratio <= 0 || Hk < 0 || Di < 0) return CSA2_E_ARG;
  if (D != 512 || !compress_ratio_supported(ratio) || n_tok % ratio != 0) return CSA2_E_SHAPE;
  if ((w_t == nullptr) != (k_idx == nullptr)) return CSA2_E_ARG;
  const int32_t c_out = Hk * Di;
  if (k_idx && (c_out <= 0 || c_out % 128 != 0 || c_out > 1024)) return CSA2_E_SHAPE;
  if ((int64_t)B * (n_tok / ratio) > INT32_MAX) return CSA2_E_SHAPE;
  if (B == 0 || n_tok == 0) return CSA2_OK;
  if (!c || !z || !entry0 || !rows) return CSA2_E_ARG;
  if (reinterpret_cast<uintptr_t>(c) % 16 || reinterpret_cast<uintptr_t>(z) % 16 ||
      reinterpret_cast<uintptr_t>(rows) % 4 || reinterpret_cast<uintptr_t>(w_t) % 16 ||
      reinterpret_cast<uintptr_t>(k_idx) % 2 || reinterpret_cast<uintptr_t>(entries) % 16)
    return CSA2_E_ARG;
  return hip_status(launch_compress_kv(c, z, B, n_tok, ratio, entry0, n_max, rows, w_t, c_out, k_idx, entries,
                                       as_stream(stream)));
}

csa2_status csa2_prefill_visibility(const int64_t* p0, int32_t B, int32_t T, int32_t ratio, int32_t n_max,
                                    int32_t* n_vis, void* stream) {
  if (B < 0 || T < 0 || n_max < 0 || ratio <= 0) return CSA2_E_ARG;
  if ((int64_t)B * T > INT32_MAX) return CSA2_E_SHAPE;
  if (B == 0 || T == 0) return CSA2_OK;
  if (!p0 || !n_vis) return CSA2_E_ARG;
  return hip_status(launch_prefill_visibility(p0, B, T, ratio, n_max, n_vis, as_stream(stream)));
}

static bool mxfp4_shape_ok(int32_t Hi, int32_t Hk, int32_t Di) {
  if (Hi <= 0 || Hk <= 0 || Di <= 0) return false;
  if (Hk == 1 && Di == 128) return Hi <= 64;                       // one shared 128-channel key
  return Hk == Hi && (Hi * Di == 256 || Hi * Di == 512);
}

csa2_status csa2_index_scores_mxfp4(const uint8_t* q_rows, const uint8_t* k_rows, int32_t B, int32_t T,
                                    int32_t Hi, int32_t Hk, int32_t Di, int32_t n_max, const int32_t* n_vis,
                                    const int32_t* cand, int32_t P, float* scores, float* block_max,
                                    int32_t block, void* stream) {
  if (B < 0 || T < 0 || n_max < 0 || (cand && P < 0)) return CSA2_E_ARG;
  if (!mxfp4_shape_ok(Hi, Hk, Di)) return CSA2_E_SHAPE;
  if (block_max && (cand || block != 8)) return CSA2_E_UNSUPPORTED;
  const int64_t rows = (int64_t)B * T;
  const int32_t ncols = cand ? P : n_max;
  if (rows == 0 || ncols == 0) return CSA2_OK;
  if (!q_rows || !k_rows || !scores) return CSA2_E_ARG;
  if (rows > INT32_MAX || ncols > kMaxCols || n_max > kMaxCols) return CSA2_E_SHAPE;
  if (reinterpret_cast<uintptr_t>(q_rows) % 8 || reinterpret_cast<uintptr_t>(k_rows) % 8 ||
      reinterpret_cast<uintptr_t>(scores) % 4)
    return CSA2_E_ARG;
  if (!cand && !block_max && index_mxfp4_prefill_supported(T, Hi, Hk, Di))
    return hip_status(launch_index_mxfp4_prefill(q_rows, k_rows, B, T, Hi, Di, n_max, n_vis, scores, as_stream(stream)));
  return hip_status(launch_index_mxfp4(q_rows, k_rows, B, T, Hi, Hk, Di, n_max, n_vis, cand, P, scores, block_max,
                                       as_stream(stream)));
}

size_t csa2_topk_workspace_size(int64_t rows, int32_t n_cols, int32_t k) {
  if (rows <= 0 || n_cols <= 0 || k <= 0 || k > kMaxK || n_cols > kMaxCols) return 0;
  return topk_workspace(rows, n_cols, k);
}

csa2_status csa2_topk(const float* scores, int64_t rows, int32_t n_cols, const int32_t* n_valid,
                      const int32_t* col_to_pos, int32_t k, int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  if (rows < 0 || n_cols < 0 || k < 0) return CSA2_E_ARG;
  if (k > kMaxK || n_cols > kMaxCols || rows > INT32_MAX) return CSA2_E_SHAPE;
  if (rows == 0 || k == 0) return CSA2_OK;
  if (!idx || (n_cols > 0 && !scores)) return CSA2_E_ARG;
  const size_t need = csa2_topk_workspace_size(rows, std::max(n_cols, 1), k);
  if (need > 0 && (!ws || ws_bytes < need)) return CSA2_E_WORKSPACE;
  return hip_status(launch_topk(scores, rows, n_cols, n_valid, 1, col_to_pos, k, idx, 0, nullptr, 0, ws,
                                as_stream(stream)));
}

size_t csa2_hier_pool_workspace_size(int64_t rows, int32_t n_blocks, int32_t n_sel_blocks) {
  return csa2_topk_workspace_size(rows, n_blocks, n_sel_blocks);
}

csa2_status csa2_hier_pool(const float* block_max, int64_t rows, int32_t n_blocks, const int32_t* n_vis,
                           int32_t block, int32_t n_sel_blocks, int32_t* pool, void* ws, size_t ws_bytes,
                           void* stream) {
  if (rows < 0 || n_blocks < 0 || n_sel_blocks < 0 || block <= 0) return CSA2_E_ARG;
  if (block > 64 || n_sel_blocks > kMaxK || n_blocks > kMaxCols || rows > INT32_MAX) return CSA2_E_SHAPE;
  if ((int64_t)n_blocks * block > INT32_MAX) return CSA2_E_SHAPE;
  if (rows == 0 || n_sel_blocks == 0) return CSA2_OK;
  if (!pool || (n_blocks > 0 && !block_max)) return CSA2_E_ARG;
  const size_t need = csa2_hier_pool_workspace_size(rows, std::max(n_blocks, 1), n_sel_blocks);
  if (need > 0 && (!ws || ws_bytes < need)) return CSA2_E_WORKSPACE;
  return hip_status(launch_topk(block_max, rows, n_blocks, n_vis, block, nullptr, n_sel_blocks, pool, block,
                                n_vis, n_blocks * block, ws, as_stream(stream)));
}

size_t csa2_sparse_attn_workspace_size(int32_t B, int32_t T, int32_t H, int32_t D, int32_t K) {
  if (B <= 0 || T <= 0 || !attn_shape_ok(H, D) || K <= 0 || K > kMaxK) return 0;
  return attn_workspace(B, T, H, D, K);
}

csa2_status csa2_sparse_attn(const uint16_t* q, const uint8_t* rows, int32_t n_max, const int32_t* idx, int32_t B,
                             int32_t T, int32_t H, int32_t D, int32_t K, float sm_scale, float* out, float* lse,
                             void* ws, size_t ws_bytes, void* stream) {
  if (B < 0 || T < 0 || n_max < 0 || K < 0 || H < 0) return CSA2_E_ARG;
  // a split stages at most 1024 entry positions and the combine pass reads at most 64 splits
  if (!attn_shape_ok(H, D) || K > kMaxK) return CSA2_E_SHAPE;
  if ((int64_t)B * T > INT32_MAX) return CSA2_E_SHAPE;
  if (B == 0 || T == 0) return CSA2_OK;
  if (!q || !out || (K > 0 && (!idx || (n_max > 0 && !rows)))) return CSA2_E_ARG;
  if (reinterpret_cast<uintptr_t>(q) % 16 || reinterpret_cast<uintptr_t>(rows) % 16 ||
      reinterpret_cast<uintptr_t>(out) % 16)
    return CSA2_E_ARG;
  const size_t need = csa2_sparse_attn_workspace_size(B, T, H, D, K);
  if (need > 0 && (!ws || ws_bytes < need)) return CSA2_E_WORKSPACE;
  return hip_status(launch_sparse_attn(q, rows, n_max, idx, B, T, H, D, K, sm_scale, out, lse, ws,
                                       as_stream(stream)));
}

size_t csa2_sparse_attn_swa_workspace_size(int32_t B, int32_t H, int32_t D, int32_t K) {
  if (B <= 0 || !attn_shape_ok(H, D) || K < 0 || K > kMaxK) return 0;
  return attn_swa_workspace(B, H, D, K);
}

csa2_status csa2_sparse_attn_swa(const uint16_t* q, const uint8_t* rows, int32_t n_max, const int32_t* idx,
                                 int32_t B, int32_t H, int32_t D, int32_t K, const uint8_t* swa_codes,
                                 const int8_t* swa_exp, const int32_t* n_win, int32_t W, float sm_scale,
                                 float* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (B < 0 || n_max < 0 || K < 0 || H < 0 || W < 0) return CSA2_E_ARG;
  if (!attn_shape_ok(H, D) || W > kMaxSwaWindow || K > kMaxK) return CSA2_E_SHAPE;
  if (B == 0) return CSA2_OK;
  if (!q || !out || !n_win || (W > 0 && (!swa_codes || !swa_exp)) || (K > 0 && (!idx || (n_max > 0 && !rows))))
    return CSA2_E_ARG;
  if (reinterpret_cast<uintptr_t>(q) % 16 || reinterpret_cast<uintptr_t>(rows) % 16 ||
      reinterpret_cast<uintptr_t>(out) % 16 || reinterpret_cast<uintptr_t>(swa_codes) % 16)
    return CSA2_E_ARG;
  const size_t need = csa2_sparse_attn_swa_workspace_size(B, H, D, K);
  if (!ws || ws_bytes < need) return CSA2_E_WORKSPACE;
  return hip_status(launch_sparse_attn_swa(q, rows, n_max, idx, B, H, D, K, swa_codes, swa_exp, n_win, W, sm_scale,
                                           out, lse, ws, as_stream(stream)));
}

size_t csa2_sparse_attn_swa_prefill_workspace_size(int32_t B, int32_t T, int32_t H, int32_t D, int32_t K) {
  if (B <= 0 || T <= 0 || !attn_shape_ok(H, D) || K < 0 || K > kMaxK) return 0;
  return attn_swa_prefill_workspace(B, T, H, D, K);
}

csa2_status csa2_sparse_attn_swa_prefill(const uint16_t* q, const uint8_t* rows, int32_t n_max, const int32_t* idx,
                                         int32_t B, int32_t T, int32_t H, int32_t D, int32_t K,
                                         const uint8_t* swa_codes, const int8_t* swa_exp, const int32_t* n_win,
                                         int32_t W, float sm_scale, float* out, float* lse, void* ws,
                                         size_t ws_bytes, void* stream) {
  if (B < 0 || T < 0 || n_max < 0 || K < 0 || H < 0 || W < 0) return CSA2_E_ARG;
  if (!attn_shape_ok(H, D) || W > kMaxSwaWindow || K > kMaxK) return CSA2_E_SHAPE;
  if ((int64_t)B * T > INT32_MAX) return CSA2_E_SHAPE;
  if (B == 0 || T == 0) return CSA2_OK;
  if (!q || !out || !n_win || (W > 0 && (!swa_codes || !swa_exp)) || (K > 0 && (!idx || (n_max > 0 && !rows))))
    return CSA2_E_ARG;
  if (reinterpret_cast<uintptr_t>(q) % 16 || reinterpret_cast<uintptr_t>(rows) % 16 ||
      reinterpret_cast<uintptr_t>(out) % 16 || reinterpret_cast<uintptr_t>(swa_codes) % 16)
    return CSA2_E_ARG;
  const size_t need = csa2_sparse_attn_swa_prefill_workspace_size(B, T, H, D, K);
  if (need > 0 && (!ws || ws_bytes < need || reinterpret_cast<uintptr_t>(ws) % 256)) return CSA2_E_WORKSPACE;
  return hip_status(launch_sparse_attn_swa_prefill(q, rows, n_max, idx, B, T, H, D, K, swa_codes, swa_exp, n_win, W,
                                                   sm_scale, out, lse, ws, as_stream(stream)));
}

// ---------------------------------------------------------------------------------------------
// Layer step. Workspace layout: [scores][block_max][top-k / pool scratch][attention partials].
// ---------------------------------------------------------------------------------------------
namespace {

struct LayerPlan {
  bool score;           // runs the indexer (Full / Reindex)
  bool on_pool;         // Reindex restricted to the candidate pool
  bool build_pool;      // Full with the hierarchical indexer
  int64_t rows;
  int32_t ncols;        // score columns (n_max, or pool capacity)
  int32_t n_blocks;
  size_t off_scores, off_bmax, off_sel, off_attn, total;
};

csa2_status plan_layer(csa2_mode mode, const csa2_layer_args* a, const csa2_shared_kv* kv,
                       const csa2_shared_idx* idx, LayerPlan* p) {
  if (!a || !kv || !idx) return CSA2_E_ARG;
  if (mode != CSA2_FULL && mode != CSA2_REINDEX && mode != CSA2_REUSE) return CSA2_E_ARG;
  if (kv->B < 0 || kv->n_max < 0 || a->T < 0 || idx->K < 0) return CSA2_E_ARG;
  if (!attn_shape_ok(a->H, kv->D)) return CSA2_E_SHAPE;
  if (idx->K > kMaxK) return CSA2_E_SHAPE;
  const bool window = a->swa_codes != nullptr;
  if (window && (a->swa_W < 0 || a->swa_W > kMaxSwaWindow)) return CSA2_E_SHAPE;
  *p = LayerPlan{};
  p->rows = (int64_t)kv->B * a->T;
  p->score = mode != CSA2_REUSE;
  p->build_pool = mode == CSA2_FULL && a->use_pool;
  p->on_pool = mode == CSA2_REINDEX && a->use_pool && idx->pool_valid;
  if (p->score) {
    if (kv->k_mx) {
      // FP4 (MXFP4) indexer keys
      if (!mxfp4_shape_ok(a->Hi, kv->Hk, kv->Di)) return CSA2_E_SHAPE;
    } else if (!index_call_ok(a->T, a->Hi, kv->Hk, kv->Di, p->on_pool, p->build_pool)) {
      return CSA2_E_SHAPE;
    }
    p->ncols = p->on_pool ? idx->P : kv->n_max;
  }
  if (p->build_pool) {
    if (a->block != 8) return CSA2_E_UNSUPPORTED;
    if (a->pool_blocks <= 0 || a->pool_blocks > kMaxK) return CSA2_E_SHAPE;
    if (!idx->pool || idx->P != a->pool_blocks * a->block) return CSA2_E_SHAPE;
    if (idx->K > a->pool_blocks * a->block) return CSA2_E_SHAPE;  // pool smaller than Top-K
    p->n_blocks = (kv->n_max + 7) / 8;
  }
  if (p->on_pool && (!idx->pool || idx->P <= 0)) return CSA2_E_SHAPE;
  if (a->new_kv) {
    // producing the caches: Full layers with bf16 indexer keys
    if (mode != CSA2_FULL) return CSA2_E_ARG;
    if (kv->k_mx) return CSA2_E_UNSUPPORTED;
    if (kv->D != 512 || a->new_tokens < 0 || !compress_ratio_supported(a->ratio) || a->new_tokens % a->ratio)
      return CSA2_E_SHAPE;
    const int32_t c_out = kv->Hk * kv->Di;
    if (c_out <= 0 || c_out % 128 != 0 || c_out > 1024) return CSA2_E_SHAPE;
  }
  size_t off = 0;
  p->off_scores = off;
  if (p->score) off = align_up(off + (size_t)p->rows * p->ncols * 4);
  p->off_bmax = off;
  if (p->build_pool) off = align_up(off + (size_t)p->rows * p->n_blocks * 4);
  p->off_sel = off;
  // scratch of the Top-K / pool / attention calls (they run one after another)
  size_t sel = 0, attn = 0;
  const int64_t rows = p->rows;
  if (rows > 0) {
    if (p->score && p->ncols > 0 && idx->K > 0) sel = std::max(sel, csa2_topk_workspace_size(rows, p->ncols, idx->K));
    if (p->build_pool && p->n_blocks > 0)
      sel = std::max(sel, csa2_hier_pool_workspace_size(rows, p->n_blocks, a->pool_blocks));
    if (p->build_pool && idx->P > 0 && idx->K > 0)  // Top-K taken from the pool's positions
      sel = std::max(sel, csa2_topk_workspace_size(rows, idx->P, idx->K));
    if (window && a->T == 1)
      attn = csa2_sparse_attn_swa_workspace_size(kv->B, a->H, kv->D, idx->K);
    else if (window)
      attn = csa2_sparse_attn_swa_prefill_workspace_size(kv->B, a->T, a->H, kv->D, idx->K);
    else if (idx->K > 0)
      attn = csa2_sparse_attn_workspace_size(kv->B, a->T, a->H, kv->D, idx->K);
  }
  off = align_up(off + sel);
  p->off_attn = off;
  off = align_up(off + attn);
  p->total = off;
  return CSA2_OK;
}

}  // namespace

csa2_status csa2_layer_workspace_size(csa2_mode mode, const csa2_layer_args* a, const csa2_shared_kv* kv,
                                      const csa2_shared_idx* idx, size_t* bytes) {
  if (!bytes) return CSA2_E_ARG;
  LayerPlan p;
  const csa2_status st = plan_layer(mode, a, kv, idx, &p);
  if (st != CSA2_OK) return st;
  *bytes = p.total;
  return CSA2_OK;
}

}  // extern "C"

namespace {

// Argument and state checks of a layer step that do not concern its workspace.
csa2_status check_layer(csa2_mode mode, const csa2_layer_args* a, const csa2_shared_kv* kv,
                        const csa2_shared_idx* idx, const LayerPlan& p) {
  if (mode != CSA2_FULL && !kv->valid) return CSA2_E_STATE;
  if (mode == CSA2_REUSE && !idx->topk_valid) return CSA2_E_STATE;
  if (!a->out || !idx->topk || !kv->rows || !a->q) return CSA2_E_ARG;
  if (p.score && (kv->k_mx ? !a->q_idx_mx : (!a->q_idx || !kv->k_idx))) return CSA2_E_ARG;
  if (a->swa_codes && (!a->swa_exp || !a->swa_n)) return CSA2_E_ARG;
  if (a->new_kv && (!a->new_z || !a->new_entry0 || !a->w_ik || !kv->k_idx)) return CSA2_E_ARG;
  return CSA2_OK;
}

// Enqueues the kernels of a validated layer step; `ws_base` holds at least p.total bytes and is
// 256-byte aligned.
csa2_status run_layer(csa2_mode mode, const csa2_layer_args* a, csa2_shared_kv* kv, csa2_shared_idx* idx,
                      const LayerPlan& p, void* ws_base, void* stream) {
  csa2_status st = CSA2_OK;
  uint8_t* ws = static_cast<uint8_t*>(ws_base);
  float* scores = reinterpret_cast<float*>(ws + p.off_scores);
  float* bmax = p.build_pool ? reinterpret_cast<float*>(ws + p.off_bmax) : nullptr;
  void* sel_ws = ws + p.off_sel;
  void* attn_ws = ws + p.off_attn;
  const size_t sel_bytes = p.off_attn - p.off_sel;
  const size_t attn_bytes = p.total - p.off_attn;
  const int T = a->T;

  hipStream_t hs = as_stream(stream);
  const int B = kv->B;
  const int64_t rows = p.rows;
  const int32_t* n_vis = kv->n_vis;
  int32_t* pool = idx->pool;
  if (a->new_kv) {
    // the Full layer's own main KV and indexer keys, written into the shared caches first
    st = csa2_compress_kv(a->new_kv, a->new_z, B, a->new_tokens, kv->D, a->ratio, a->new_entry0, kv->n_max,
                          const_cast<uint8_t*>(kv->rows), a->w_ik, kv->Hk, kv->Di, const_cast<uint16_t*>(kv->k_idx),
                          nullptr, stream);
    if (st != CSA2_OK) return st;
  }
  if (p.score) {
    if (kv->k_mx) {
      st = csa2_index_scores_mxfp4(a->q_idx_mx, kv->k_mx, B, T, a->Hi, kv->Hk, kv->Di, kv->n_max, n_vis,
                                   p.on_pool ? pool : nullptr, p.on_pool ? idx->P : 0, scores, bmax, 8, stream);
    } else {
      st = csa2_index_scores(a->q_idx, kv->k_idx, B, T, a->Hi, kv->Hk, kv->Di, kv->n_max, n_vis,
                             p.on_pool ? pool : nullptr, p.on_pool ? idx->P : 0, scores, bmax, 8, stream);
    }
    if (st != CSA2_OK) return st;
    if (p.build_pool && a->pool_blocks >= idx->K) {
      // The pool of the best pool_blocks >= K blocks holds the layer's own flat Top-K: each Top-K
      // position's block max is at least its score, so a block left out would be outranked by
      // >= K block maxima. The pool is chosen first and the Top-K taken from its positions.
      hipError_t e = launch_pool_topk(bmax, rows, p.n_blocks, n_vis, a->pool_blocks, pool, scores, p.ncols, idx->K,
                                      idx->topk, hs);
      if (e == hipErrorNotSupported) {
        (void)hipGetLastError();
        e = launch_topk(bmax, rows, p.n_blocks, n_vis, 8, nullptr, a->pool_blocks, pool, 8, n_vis, kv->n_max, sel_ws,
                        hs);
        if (e != hipSuccess) return CSA2_E_HIP;
        e = launch_topk_gather(scores, p.ncols, rows, pool, idx->P, idx->K, idx->topk, sel_ws, hs);
      }
      if (e != hipSuccess) return CSA2_E_HIP;
    } else {
      st = csa2_topk(scores, rows, p.ncols, p.on_pool ? nullptr : n_vis, p.on_pool ? pool : nullptr, idx->K, idx->topk,
                     sel_ws, sel_bytes, stream);
      if (st != CSA2_OK) return st;
      if (p.build_pool && a->pool_blocks > 0) {
        const hipError_t e = launch_topk(bmax, rows, p.n_blocks, n_vis, 8, nullptr, a->pool_blocks, pool, 8, n_vis,
                                         kv->n_max, sel_ws, hs);
        if (e != hipSuccess) return CSA2_E_HIP;
      }
    }
  }
  if (a->swa_codes && T > 1)
    st = csa2_sparse_attn_swa_prefill(a->q, kv->rows, kv->n_max, idx->topk, B, T, a->H, kv->D, idx->K, a->swa_codes,
                                      a->swa_exp, a->swa_n, a->swa_W, a->sm_scale, a->out, a->lse, attn_ws, attn_bytes,
                                      stream);
  else if (a->swa_codes)
    st = csa2_sparse_attn_swa(a->q, kv->rows, kv->n_max, idx->topk, B, a->H, kv->D, idx->K, a->swa_codes, a->swa_exp,
                              a->swa_n, a->swa_W, a->sm_scale, a->out, a->lse, attn_ws, attn_bytes, stream);
  else
    st = csa2_sparse_attn(a->q, kv->rows, kv->n_max, idx->topk, B, T, a->H, kv->D, idx->K, a->sm_scale, a->out,
                          a->lse, attn_ws, attn_bytes, stream);
  if (st != CSA2_OK) return st;
  if (p.score) idx->topk_valid = 1;
  if (p.build_pool) idx->pool_valid = 1;
  if (mode == CSA2_FULL) kv->valid = 1;
  return CSA2_OK;
}

// Scratch of csa2_layer_step_noalloc: one copy per device, held until the process ends. Host code
// never uses the array's name as an address: each device's copy is looked up once with
// hipGetSymbolAddress (with that device current) and the pointer kept per device.
static __device__ __align__(256) unsigned char scratch[CSA2_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_for_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr || reinterpret_cast<uintptr_t>(ptr) % kAlign) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

csa2_status csa2_layer_step(csa2_mode mode, const csa2_layer_args* a, csa2_shared_kv* kv, csa2_shared_idx* idx,
                            void* stream) {
  LayerPlan p;
  csa2_status st = plan_layer(mode, a, kv, idx, &p);
  if (st != CSA2_OK) return st;
  if ((st = check_layer(mode, a, kv, idx, p)) != CSA2_OK) return st;
  if (p.total > 0 && (!a->ws || a->ws_bytes < p.total || reinterpret_cast<uintptr_t>(a->ws) % kAlign))
    return CSA2_E_WORKSPACE;
  return run_layer(mode, a, kv, idx, p, a->ws, stream);
}

csa2_status csa2_layer_step_noalloc(csa2_mode mode, const csa2_layer_args* a, csa2_shared_kv* kv,
                                    csa2_shared_idx* idx, void* stream) {
  LayerPlan p;
  csa2_status st = plan_layer(mode, a, kv, idx, &p);
  if (st != CSA2_OK) return st;
  if ((st = check_layer(mode, a, kv, idx, p)) != CSA2_OK) return st;
  if (p.total > CSA2_NOALLOC_SCRATCH_BYTES) return CSA2_E_WORKSPACE;
  void* ws = nullptr;
  if (scratch_for_current_device(&ws) != hipSuccess) return CSA2_E_HIP;
  return run_layer(mode, a, kv, idx, p, ws, stream);
}

}  // extern "C"
