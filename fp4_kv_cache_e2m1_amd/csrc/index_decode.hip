// Lightweight indexer, streaming form (decode and candidate-pool scoring).
// Source: DeepSeek-V4.1-Flash walkthrough (wkq9411.github.io), 一(四) (indexer Q x indexer K
// scores every main-KV entry) and 一(四)2 (later layers score only the candidate pool; a
// block's score is the max index score inside it).
//
// score[r, n] = sum_h sum_d q[r, h, d] * k[b, n, h', d]. This pass is HBM-bound: every key row
// (Hk*Di bf16) is read once and contributes one fp32 score, so the kernel is laid out for
// streaming, not for MFMA. Eight lanes own one key row; on each load instruction they read 128
// contiguous bytes of it (a wave covers 8 consecutive rows = 8 x 128 B), and after NCH such
// loads each lane has NCH*8 channels of the row. Products of bf16 pairs go through v_dot2
// (exact products, fp32 accumulation), the 8 partial sums meet in a 3-step DPP reduction, and
// the 8 rows of a wave form one aligned 8-entry block, whose max is the fused block score.
#include "common.h"
#include "launch.h"

#include <atomic>

namespace csa2 {

constexpr int kIdxThreads = 256;           // 4 waves, 32 rows per row step
constexpr int kRowsPerIter = kIdxThreads / 8;
template <int NCH> constexpr int kRowsPerGroup = NCH >= 8 ? 1 : 8 / NCH;

// RPI rows per lane group and iteration (short key rows: 8 / NCH), so every lane keeps 8 loads in
// flight whatever the row length; row u of an iteration is 32 u rows after row 0, so the 8 row
// groups of a wave still cover one aligned 8-entry block for each u.
template <int NCH, bool kSharedKey, bool kPool, bool kBlockMax, int RPI>
__global__ __launch_bounds__(kIdxThreads) void index_stream_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, int T, int Hi, int Di, int n_max,
    const int32_t* __restrict__ n_vis, const int32_t* __restrict__ cand, int P, int tile_rows,
    float* __restrict__ scores, float* __restrict__ block_max) {
  const int r = blockIdx.x;                 // query row = b * T + t
  const int b = r / T;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int j = tid & 7;                    // lane within the 8-lane row group
  const int grp = tid >> 3;                 // row group within the workgroup (0..31)
  const int CH = NCH * 8;                   // 16-byte chunks per key row
  const int ncols = kPool ? P : n_max;
  const int nv = (!kPool && n_vis) ? min(n_vis[r], n_max) : n_max;
  const int tile0 = blockIdx.y * tile_rows;
  const int tile_end = min(tile0 + tile_rows, ncols);

  // this lane's share of the query: chunks j + 8i (8 channels each)
  uint32_t qw[NCH][4];
  float qf[kSharedKey ? NCH : 1][8];
  if (!kSharedKey) {
    const uint4* qp = reinterpret_cast<const uint4*>(q + (int64_t)r * Hi * Di);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const uint4 v = qp[j + 8 * i];
      qw[i][0] = v.x; qw[i][1] = v.y; qw[i][2] = v.z; qw[i][3] = v.w;
    }
  } else {
    // one shared key head: the score is (sum_h q_h) . k, with the head sum in fp32
#pragma unroll
    for (int i = 0; i < NCH; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[kSharedKey ? i : 0][e] = 0.0f;
    for (int h = 0; h < Hi; ++h) {
      const uint4* qp = reinterpret_cast<const uint4*>(q + ((int64_t)r * Hi + h) * Di);
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const uint4 v = qp[j + 8 * i];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qf[kSharedKey ? i : 0][2 * e] += __uint_as_float(w[e] << 16);
          qf[kSharedKey ? i : 0][2 * e + 1] += __uint_as_float(w[e] & 0xFFFF0000u);
        }
      }
    }
  }

  const u32x4_t* kbase = reinterpret_cast<const u32x4_t*>(k) + (int64_t)b * n_max * CH;
  const int32_t* crow = kPool ? cand + (int64_t)r * P : nullptr;
  const int n_blocks = (n_max + 7) >> 3;

  for (int it = 0; it < tile_rows; it += kRowsPerIter * RPI) {
    int col[RPI];
    bool valid[RPI];
    u32x4_t kv[RPI][NCH];
#pragma unroll
    for (int u = 0; u < RPI; ++u) {
      col[u] = tile0 + it + kRowsPerIter * u + grp;
      int pos = col[u];
      if (kPool) {
        pos = col[u] < tile_end ? crow[col[u]] : -1;
        valid[u] = pos >= 0 && pos < n_max;
      } else {
        valid[u] = col[u] < tile_end && col[u] < nv;
      }
      if (valid[u]) {
        const u32x4_t* kp = kbase + (int64_t)pos * CH + j;
#pragma unroll
        for (int i = 0; i < NCH; ++i) kv[u][i] = __builtin_nontemporal_load(kp + 8 * i);
      } else {
#pragma unroll
        for (int i = 0; i < NCH; ++i) kv[u][i] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < RPI; ++u) {
      float acc = 0.0f;
      if (!kSharedKey) {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
          const uint32_t w[4] = {kv[u][i].x, kv[u][i].y, kv[u][i].z, kv[u][i].w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qw[i][e]),
                                                  __builtin_bit_cast(bf16x2_t, w[e]), acc, false);
        }
      } else {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
          const uint32_t w[4] = {kv[u][i].x, kv[u][i].y, kv[u][i].z, kv[u][i].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc = fmaf(qf[kSharedKey ? i : 0][2 * e], __uint_as_float(w[e] << 16), acc);
            acc = fmaf(qf[kSharedKey ? i : 0][2 * e + 1], __uint_as_float(w[e] & 0xFFFF0000u), acc);
          }
        }
      }
      acc = sum8(acc);
      if (j == 0 && col[u] < tile_end) {
        if (kPool)
          scores[(int64_t)r * ncols + col[u]] = valid[u] ? acc : -INFINITY;
        else if (valid[u])
          scores[(int64_t)r * ncols + col[u]] = acc;
      }
      if (kBlockMax) {
        // the wave's 8 row groups are one aligned block of 8 entries
        float m = valid[u] ? acc : -INFINITY;
        m = fmaxf(m, shfl_xor_f(m, 8));
        m = fmaxf(m, shfl_xor_f(m, 16));
        m = fmaxf(m, shfl_xor_f(m, 32));
        const int blk = (tile0 + it + kRowsPerIter * u + (grp & ~7)) >> 3;  // first column of the wave / 8
        if (lane == 0 && blk < n_blocks && blk * 8 < min(nv, tile_end))
          block_max[(int64_t)r * n_blocks + blk] = m;
      }
    }
  }
}

template <int NCH>
static hipError_t launch_nch(bool shared, bool pool, bool bmax, dim3 grid, hipStream_t s,
                             const uint16_t* q, const uint16_t* k, int T, int Hi, int Di, int n_max,
                             const int32_t* n_vis, const int32_t* cand, int P, int tile_rows,
                             float* scores, float* block_max) {
  dim3 block(kIdxThreads);
#define CSA2_IDX_LAUNCH(SK, PL, BM)                                                                  \
  hipLaunchKernelGGL((index_stream_kernel<NCH, SK, PL, BM, kRowsPerGroup<NCH>>), grid, block, 0, s, q, k, T, Hi, Di, n_max, \
                     n_vis, cand, P, tile_rows, scores, block_max)
  if (shared) {
    if (pool) CSA2_IDX_LAUNCH(true, true, false);
    else if (bmax) CSA2_IDX_LAUNCH(true, false, true);
    else CSA2_IDX_LAUNCH(true, false, false);
  } else {
    if (pool) CSA2_IDX_LAUNCH(false, true, false);
    else if (bmax) CSA2_IDX_LAUNCH(false, false, true);
    else CSA2_IDX_LAUNCH(false, false, false);
  }
#undef CSA2_IDX_LAUNCH
  return hipGetLastError();
}

int device_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
      (void)hipGetLastError();
      n = 256;
    }
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

hipError_t launch_index_stream(const uint16_t* q, const uint16_t* k, int B, int T, int Hi, int Hk,
                               int Di, int n_max, const int32_t* n_vis, const int32_t* cand, int P,
                               float* scores, float* block_max, hipStream_t s) {
  const int rows = B * T;
  const int ncols = cand ? P : n_max;
  if (rows == 0 || ncols == 0) return hipSuccess;
  const int ch = Hk * Di * 2 / 16;  // 16-byte chunks per key row (multiple of 8)
  const int nch = ch / 8;
  // Tile size. Flat scoring of rows of 1 KiB or more: one workgroup per CU when the rows split
  // evenly enough, each streaming one contiguous tile (4 x 262144 and 16 x 65536 entries:
  // 165 -> 151 us, 7.1 TB/s; a grid just over one workgroup per CU is much slower, its second
  // round running on a few CUs, and two per CU are no faster than many). Otherwise enough
  // workgroups to cover the chip several times over, in whole iterations (short key rows take
  // 8 / nch rows per lane group and iteration).
  const int cus = device_cu_count();
  const int per_row = rows <= cus ? cus / rows : 0;
  int tile_rows = kRowsPerIter * (nch >= 8 ? 1 : 8 / nch);
  if (!cand && nch >= 8 && per_row > 0 && 4 * (int64_t)rows * per_row >= 3 * (int64_t)cus &&
      ncols >= per_row * kRowsPerIter) {
    tile_rows = ((ncols + per_row - 1) / per_row + kRowsPerIter - 1) / kRowsPerIter * kRowsPerIter;
  } else {
    while (tile_rows < 1024 && (int64_t)((ncols + 2 * tile_rows - 1) / (2 * tile_rows)) * rows >= 2048)
      tile_rows *= 2;
    // short key rows: a workgroup streams as many bytes as it would with 1 KiB rows when the grid
    // keeps at least 512 workgroups (measured: 256-byte rows, 4 x 262144 entries, 54 -> 47 us)
    if (nch < 8) {
      const int big = tile_rows * (8 / nch);
      if ((int64_t)((ncols + big - 1) / big) * rows >= 512) tile_rows = big;
    }
  }
  while ((ncols + tile_rows - 1) / tile_rows > 65535) tile_rows *= 2;  // grid.y limit
  dim3 grid((unsigned)rows, (unsigned)((ncols + tile_rows - 1) / tile_rows));
  const bool shared = Hk == 1, pool = cand != nullptr, bmax = block_max != nullptr && !pool;
  switch (nch) {
    case 1: return launch_nch<1>(shared, pool, bmax, grid, s, q, k, T, Hi, Di, n_max, n_vis, cand, P, tile_rows, scores, block_max);
    case 2: return launch_nch<2>(shared, pool, bmax, grid, s, q, k, T, Hi, Di, n_max, n_vis, cand, P, tile_rows, scores, block_max);
    case 4: return launch_nch<4>(shared, pool, bmax, grid, s, q, k, T, Hi, Di, n_max, n_vis, cand, P, tile_rows, scores, block_max);
    case 8: return launch_nch<8>(shared, pool, bmax, grid, s, q, k, T, Hi, Di, n_max, n_vis, cand, P, tile_rows, scores, block_max);
    case 16: return launch_nch<16>(shared, pool, bmax, grid, s, q, k, T, Hi, Di, n_max, n_vis, cand, P, tile_rows, scores, block_max);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace csa2
