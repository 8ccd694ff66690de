// Lightweight indexer over FP4 query and key rows (OCP MXFP4), streaming form.
// Source: DeepSeek-V4.1-Flash walkthrough (wkq9411.github.io), 一(五)4 "FP4 Main KV Cache": the
// indexer query and key are FP4 in the OCP MXFP4 format (E2M1 elements, one power-of-two E8M0
// scale per 32 channels); 一(四): the indexer scores every main-KV entry.
//
// A row (one query's or one entry's Hi x Di channels, C = Hi*Di) is C/2 code bytes (channel 2i
// in the low nibble of byte i) followed by C/32 E8M0 bytes. score[r, n] = sum_c q[r,c] k[n,c].
// HBM-bound: every key row is read once (C = 512: 272 bytes instead of 1024 in bf16). L = C/32
// lanes own one key row, lane j its 32-channel block j: 16 code bytes and one scale byte. The
// block's E2M1 values of query and key are converted to f16 (exact) and multiplied with v_dot2
// into an fp32 sum that is exact (products are multiples of 1/4 below 36, 32 of them), which is
// then scaled by 2^(eq + ek - 254) (one rounding) and the L block sums meet in a butterfly.
#include "common.h"
#include "launch.h"

namespace csa2 {

typedef _Float16 f16x2_mx_t __attribute__((ext_vector_type(2)));
typedef float f32x2_mx_t __attribute__((ext_vector_type(2)));

constexpr int kMxThreads = 256;
constexpr int kMxInFlight = 4;          // row steps whose loads a lane issues before using them
constexpr int kMxSharedInFlight = 4;    // the same for the shared-key form (68-byte rows; 4 beat 8 and 16)

// 8 E2M1 codes (one 32-bit word, channel 2i in the low nibble of byte i) -> 4 f16 pairs, exact.
__device__ __forceinline__ void mx_e2m1x8(uint32_t w, f16x2_mx_t* out) {
  out[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
  out[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
  out[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
  out[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
}

// kPool: column c of a query row scores position cand[r, c] (-inf for an empty slot or a position
// outside [0, n_max)); kBlockMax: the max score of each aligned block of 8 visible entries goes to
// block_max (a block spans two waves here, so an iteration's scores meet in LDS).
template <int L, bool kPool, bool kBlockMax>
__global__ __launch_bounds__(kMxThreads) void index_mxfp4_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k, int T, int n_max,
    const int32_t* __restrict__ n_vis, const int32_t* __restrict__ cand, int P, int tile_rows,
    float* __restrict__ scores, float* __restrict__ block_max) {
  static_assert(L == 8 || L == 16, "rows of 256 or 512 channels");
  constexpr int C = 32 * L;
  constexpr int RB = C / 2 + C / 32;            // bytes per row
  constexpr int ROWS = kMxThreads / L;          // rows per workgroup step
  const int r = blockIdx.x;                     // query row = b * T + t
  const int b = r / T;
  const int tid = threadIdx.x;
  const int j = tid % L;                        // the lane's 32-channel block
  const int grp = tid / L;                      // the lane group's row within a step
  const int ncols = kPool ? P : n_max;
  const int nv = (!kPool && n_vis) ? min(n_vis[r], n_max) : n_max;
  const int tile0 = blockIdx.y * tile_rows;
  const int tile_end = min(tile0 + tile_rows, kPool ? ncols : nv);
  if (tile0 >= tile_end) return;               // uniform over the workgroup
  __shared__ float sbm[kBlockMax ? ROWS * kMxInFlight : 1];
  const int32_t* crow = kPool ? cand + (int64_t)r * P : nullptr;
  const int n_blocks = (n_max + 7) >> 3;

  // the query's block j as 16 f16 pairs and its exponent
  f16x2_mx_t qv[16];
  int eq;
  {
    const uint8_t* qp = q + (int64_t)r * RB;
    const uint2 a = *reinterpret_cast<const uint2*>(qp + 16 * j);
    const uint2 c = *reinterpret_cast<const uint2*>(qp + 16 * j + 8);
    mx_e2m1x8(a.x, qv);
    mx_e2m1x8(a.y, qv + 4);
    mx_e2m1x8(c.x, qv + 8);
    mx_e2m1x8(c.y, qv + 12);
    eq = qp[C / 2 + j];
  }
  const uint8_t* kb = k + (int64_t)b * n_max * RB;
  float* srow = scores + (int64_t)r * ncols;

  for (int base = tile0; base < tile_end; base += ROWS * kMxInFlight) {
    uint2 ca[kMxInFlight], cb[kMxInFlight];
    int ek[kMxInFlight];
    bool valid[kMxInFlight];
#pragma unroll
    for (int u = 0; u < kMxInFlight; ++u) {
      const int col = base + u * ROWS + grp;
      int n = col;
      if (kPool) {
        n = col < tile_end ? crow[col] : -1;
        valid[u] = n >= 0 && n < n_max;
      } else {
        valid[u] = col < tile_end;
      }
      ca[u] = cb[u] = make_uint2(0, 0);
      ek[u] = 127;
      if (valid[u]) {
        const uint8_t* p = kb + (int64_t)n * RB;
        ca[u] = *reinterpret_cast<const uint2*>(p + 16 * j);
        cb[u] = *reinterpret_cast<const uint2*>(p + 16 * j + 8);
        ek[u] = p[C / 2 + j];
      }
    }
#pragma unroll
    for (int u = 0; u < kMxInFlight; ++u) {
      f16x2_mx_t kv[16];
      mx_e2m1x8(ca[u].x, kv);
      mx_e2m1x8(ca[u].y, kv + 4);
      mx_e2m1x8(cb[u].x, kv + 8);
      mx_e2m1x8(cb[u].y, kv + 12);
      float part = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) part = __builtin_amdgcn_fdot2(qv[i], kv[i], part, false);
      float v = ldexpf(part, eq + ek[u] - 254);
#pragma unroll
      for (int m = L / 2; m >= 1; m /= 2) v += shfl_xor_f(v, m);
      const int col = base + u * ROWS + grp;
      if (j == 0 && col < tile_end) srow[col] = valid[u] ? v : -INFINITY;
      if (kBlockMax && j == 0) sbm[u * ROWS + grp] = valid[u] ? v : -INFINITY;
    }
    if (kBlockMax) {
      // sbm[i] is the score of row base + i (base and the tile are multiples of 8 rows)
      __syncthreads();
      if (tid < ROWS * kMxInFlight / 8) {
        float m = sbm[8 * tid];
#pragma unroll
        for (int e = 1; e < 8; ++e) m = fmaxf(m, sbm[8 * tid + e]);
        const int blk = (base >> 3) + tid;
        if (blk < n_blocks && blk * 8 < tile_end) block_max[(int64_t)r * n_blocks + blk] = m;
      }
      __syncthreads();                          // sbm is rewritten by the next iteration
    }
  }
}

// One shared key of 128 channels per entry (68-byte rows, 4 lanes per row) and Hi query heads:
// score = (sum_h q_h) . k. The workgroup first sums the heads' dequantized query values in fp32,
// then each entry's 32-channel block j (lane j) is 32 fp32 products with the key's E2M1 values,
// scaled by the key's exponent; the 4 block sums meet in a butterfly.
// kPool: column c of a query row scores position cand[r, c] (-inf for an empty slot or a position
// outside [0, n_max)); kBlockMax: the max score of each aligned block of 8 visible entries (the 8
// row groups of a half-wave are one block) goes to block_max ([walkthrough] 一(四)2).
constexpr int kMaxSharedHeads = 64;      // query heads of the shared-key form
template <bool kPool, bool kBlockMax>
__global__ __launch_bounds__(kMxThreads) void index_mxfp4_shared_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k, int T, int Hi, int n_max,
    const int32_t* __restrict__ n_vis, const int32_t* __restrict__ cand, int P, int tile_rows,
    float* __restrict__ scores, float* __restrict__ block_max) {
  constexpr int L = 4, RB = 68;                 // 128 channels: 64 code bytes + 4 scale bytes
  constexpr int ROWS = kMxThreads / L;
  const int r = blockIdx.x;
  const int b = r / T;
  const int tid = threadIdx.x;
  const int j = tid % L;
  const int grp = tid / L;
  const int lane = tid & 63;
  const int ncols = kPool ? P : n_max;
  const int nv = (!kPool && n_vis) ? min(n_vis[r], n_max) : n_max;
  const int tile0 = blockIdx.y * tile_rows;
  const int tile_end = min(tile0 + tile_rows, kPool ? ncols : nv);
  if (tile0 >= tile_end) return;

  // The query summed over its heads, (sum_h q_h)[c] for the 128 channels. The query row is
  // Hi*64 code bytes (head h at 64 h) followed by Hi*4 scale bytes (head h at 4 h); it is staged
  // in LDS with one load per thread (at most 64 x 68 bytes), then thread t sums channel t % 128
  // over every other head and the two halves meet in LDS, so each workgroup spends a few hundred
  // instructions per thread on it instead of every lane summing all heads of its block.
  __shared__ uint32_t qsm[kMaxSharedHeads * RB / 4];
  __shared__ float qsum[2][128];
  {
    const uint32_t* qw = reinterpret_cast<const uint32_t*>(q + (int64_t)r * Hi * RB);
    for (int i = tid; i < Hi * (RB / 4); i += kMxThreads) qsm[i] = qw[i];
  }
  __syncthreads();
  {
    const uint8_t* qp = reinterpret_cast<const uint8_t*>(qsm);
    const int c = tid & 127, half = tid >> 7;
    float acc = 0.0f;
    for (int h = half; h < Hi; h += 2) {
      const uint32_t nib = (qp[64 * h + (c >> 1)] >> (4 * (c & 1))) & 0xFu;
      const uint32_t e = (nib >> 1) & 3u, m = nib & 1u;
      const float mag = e ? ldexpf(1.0f + 0.5f * (float)m, (int)e - 1) : 0.5f * (float)m;   // E2M1
      const float sc = ldexpf(1.0f, (int)qp[Hi * 64 + 4 * h + (c >> 5)] - 127);
      acc = fmaf((nib & 8u) ? -mag : mag, sc, acc);
    }
    qsum[half][c] = acc;
  }
  __syncthreads();
  float qs[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) qs[i] = qsum[0][32 * j + i] + qsum[1][32 * j + i];
  const uint8_t* kb = k + (int64_t)b * n_max * RB;
  float* srow = scores + (int64_t)r * ncols;
  const int32_t* crow = kPool ? cand + (int64_t)r * P : nullptr;
  const int n_blocks = (n_max + 7) >> 3;

  for (int base = tile0; base < tile_end; base += ROWS * kMxSharedInFlight) {
    uint32_t cw[kMxSharedInFlight][4];
    int ek[kMxSharedInFlight];
    bool valid[kMxSharedInFlight];
#pragma unroll
    for (int u = 0; u < kMxSharedInFlight; ++u) {
      const int col = base + u * ROWS + grp;
      int n = col;
      if (kPool) {
        n = col < tile_end ? crow[col] : -1;
        valid[u] = n >= 0 && n < n_max;
      } else {
        valid[u] = col < tile_end;
      }
#pragma unroll
      for (int w = 0; w < 4; ++w) cw[u][w] = 0u;
      ek[u] = 127;
      if (valid[u]) {
        const uint8_t* p = kb + (int64_t)n * RB;
        const uint32_t* pw = reinterpret_cast<const uint32_t*>(p + 16 * j);
#pragma unroll
        for (int w = 0; w < 4; ++w) cw[u][w] = pw[w];
        ek[u] = p[64 + j];
      }
    }
#pragma unroll
    for (int u = 0; u < kMxSharedInFlight; ++u) {
      float part = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const f32x2_mx_t v[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[u][w], 1.0f, 0),
                                 __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[u][w], 1.0f, 1),
                                 __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[u][w], 1.0f, 2),
                                 __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[u][w], 1.0f, 3)};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          part = fmaf(qs[8 * w + 2 * e], v[e][0], part);
          part = fmaf(qs[8 * w + 2 * e + 1], v[e][1], part);
        }
      }
      float v = ldexpf(part, ek[u] - 127);
      v += shfl_xor_f(v, 2);
      v += shfl_xor_f(v, 1);
      const int col = base + u * ROWS + grp;
      if (j == 0 && col < tile_end) srow[col] = valid[u] ? v : -INFINITY;
      if (kBlockMax) {
        // the 8 row groups of a half-wave are one aligned block of 8 entries (tiles and steps are
        // multiples of 8 rows)
        float m = valid[u] ? v : -INFINITY;
        m = fmaxf(m, shfl_xor_f(m, 4));
        m = fmaxf(m, shfl_xor_f(m, 8));
        m = fmaxf(m, shfl_xor_f(m, 16));
        const int blk = (base + u * ROWS + (grp & ~7)) >> 3;
        if ((lane & 31) == 0 && blk < n_blocks && blk * 8 < tile_end) block_max[(int64_t)r * n_blocks + blk] = m;
      }
    }
  }
}

template <int L>
static hipError_t launch_mx_modes(dim3 grid, hipStream_t s, const uint8_t* q, const uint8_t* k, int T, int n_max,
                                  const int32_t* n_vis, const int32_t* cand, int P, int tile, float* scores,
                                  float* block_max) {
  if (cand)
    hipLaunchKernelGGL((index_mxfp4_kernel<L, true, false>), grid, dim3(kMxThreads), 0, s, q, k, T, n_max, n_vis,
                       cand, P, tile, scores, block_max);
  else if (block_max)
    hipLaunchKernelGGL((index_mxfp4_kernel<L, false, true>), grid, dim3(kMxThreads), 0, s, q, k, T, n_max, n_vis,
                       cand, P, tile, scores, block_max);
  else
    hipLaunchKernelGGL((index_mxfp4_kernel<L, false, false>), grid, dim3(kMxThreads), 0, s, q, k, T, n_max, n_vis,
                       cand, P, tile, scores, block_max);
  return hipGetLastError();
}

hipError_t launch_index_mxfp4(const uint8_t* q, const uint8_t* k, int B, int T, int Hi, int Hk, int Di,
                              int n_max, const int32_t* n_vis, const int32_t* cand, int P, float* scores,
                              float* block_max, hipStream_t s) {
  const int64_t rows = (int64_t)B * T;
  const int ncols = cand ? P : n_max;
  if (rows == 0 || ncols == 0) return hipSuccess;
  if (Hk == 1 && Di == 128) {                   // one shared key per entry
    // larger tiles than the per-head form: each workgroup first sums the query heads (about 1024
    // workgroups measured best against 512 .. 4096 at 4 x 262144, 32 x 16384 and 1 x 1048576)
    const int step = (kMxThreads / 4) * kMxSharedInFlight;
    int tile = step;
    while (tile < 8192 && rows * ((ncols + 2 * tile - 1) / (2 * tile)) >= 1024) tile *= 2;
    dim3 grid((unsigned)rows, (unsigned)((ncols + tile - 1) / tile));
    if (cand)
      hipLaunchKernelGGL((index_mxfp4_shared_kernel<true, false>), grid, dim3(kMxThreads), 0, s, q, k, T, Hi, n_max,
                         n_vis, cand, P, tile, scores, block_max);
    else if (block_max)
      hipLaunchKernelGGL((index_mxfp4_shared_kernel<false, true>), grid, dim3(kMxThreads), 0, s, q, k, T, Hi, n_max,
                         n_vis, cand, P, tile, scores, block_max);
    else
      hipLaunchKernelGGL((index_mxfp4_shared_kernel<false, false>), grid, dim3(kMxThreads), 0, s, q, k, T, Hi, n_max,
                         n_vis, cand, P, tile, scores, block_max);
    return hipGetLastError();
  }

  const int C = Hi * Di;
  // tiles of rows per workgroup: about 16384 workgroups or more, each at least one step of rows in
  // flight (four steps of 8-byte loads per lane and this target measured best against 8 or 16
  // steps and 4096 / 8192 workgroups at 4 x 262144, 16 x 65536 and 32 x 16384 entries)
  const int step = (kMxThreads / (C / 32)) * kMxInFlight;
  int tile = step;
  while (tile < 8192 && rows * ((ncols + 2 * tile - 1) / (2 * tile)) >= 16384) tile *= 2;
  dim3 grid((unsigned)rows, (unsigned)((ncols + tile - 1) / tile));
  if (C == 256) return launch_mx_modes<8>(grid, s, q, k, T, n_max, n_vis, cand, P, tile, scores, block_max);
  return launch_mx_modes<16>(grid, s, q, k, T, n_max, n_vis, cand, P, tile, scores, block_max);
}

}  // namespace csa2
