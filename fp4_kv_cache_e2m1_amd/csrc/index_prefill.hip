// Lightweight indexer, prefill form: many query tokens against the same keys.
// Source: DeepSeek-V4.1-Flash walkthrough (wkq9411.github.io), 一(四) (indexer Q x indexer K
// scores every causally visible main-KV entry for each query).
//
// With T query rows the scores are a dense [T x (Hi*Di)] x [(Hi*Di) x N] contraction, so this
// form runs on v_mfma_f32_16x16x32_bf16 (exact bf16 products, fp32 accumulation). A workgroup
// (4 waves in a 2 x 2 arrangement) computes a 128 x 128 score tile, walking the 512 contraction
// channels in LDS-staged slices of 64. Tiles whose keys are all beyond every row's visible range
// are skipped whole; partially visible tiles mask their stores. The grid runs query tiles
// fastest, so the workgroups sharing a key tile are dispatched together and each XCD keeps the
// same few query tiles resident in its L2.
#include "common.h"
#include "launch.h"

namespace csa2 {

constexpr int kPBM = 128, kPBN = 128, kPBK = 64;
constexpr int kPPitch = kPBK + 8;  // bf16 elements per LDS row

__global__ __launch_bounds__(256) void index_prefill_kernel(const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ k, int T,
                                                            int C, int n_max,
                                                            const int32_t* __restrict__ n_vis,
                                                            float* __restrict__ scores) {
  __shared__ __attribute__((aligned(16))) uint16_t qs[kPBM * kPPitch];
  __shared__ __attribute__((aligned(16))) uint16_t ks[kPBN * kPPitch];
  __shared__ int tile_vis;

  const int t0 = blockIdx.x * kPBM, n0 = blockIdx.y * kPBN, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;

  // skip tiles with no visible (query, key) pair
  if (tid == 0) tile_vis = 0;
  __syncthreads();
  if (tid < kPBM && t0 + tid < T) {
    const int nv = n_vis ? n_vis[(int64_t)b * T + t0 + tid] : n_max;
    if (nv > n0) atomicMax(&tile_vis, 1);
  }
  __syncthreads();
  if (!tile_vis) return;

  const uint16_t* qb = q + ((int64_t)b * T) * C;
  const uint16_t* kb = k + ((int64_t)b * n_max) * C;
  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int c0 = 0; c0 < C; c0 += kPBK) {
    // stage 128 x 64 slices of Q and K (8 x 16 B per row)
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int e = tid + it * 256;
      const int row = e >> 3, part = e & 7;
      uint4 vq = make_uint4(0, 0, 0, 0), vk = make_uint4(0, 0, 0, 0);
      if (t0 + row < T) vq = *reinterpret_cast<const uint4*>(qb + (int64_t)(t0 + row) * C + c0 + 8 * part);
      if (n0 + row < n_max) vk = *reinterpret_cast<const uint4*>(kb + (int64_t)(n0 + row) * C + c0 + 8 * part);
      *reinterpret_cast<uint4*>(qs + row * kPPitch + 8 * part) = vq;
      *reinterpret_cast<uint4*>(ks + row * kPPitch + 8 * part) = vk;
    }
    __syncthreads();
#pragma unroll
    for (int ks32 = 0; ks32 < kPBK; ks32 += 32) {
      bf16x8_t a[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qs + (wm + 16 * i + l16) * kPPitch + ks32 + 8 * g));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bv[j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(ks + (wn + 16 * j + l16) * kPPitch + ks32 + 8 * g));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bv[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }

  // store: lane holds rows wm + 16 i + 4 g + r, column wn + 16 j + l16
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + wm + 16 * i + 4 * g + r;
      if (t >= T) continue;
      const int nv = n_vis ? min(n_vis[(int64_t)b * T + t], n_max) : n_max;
      float* srow = scores + ((int64_t)b * T + t) * n_max;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + wn + 16 * j + l16;
        if (n < nv) srow[n] = acc[i][j][r];
      }
    }
}

bool index_prefill_supported(int T, int Hi, int Hk, int Di) {
  return T >= 16 && Hk == Hi && (Hi * Di) % kPBK == 0;
}

hipError_t launch_index_prefill(const uint16_t* q, const uint16_t* k, int B, int T, int Hi, int Di,
                                int n_max, const int32_t* n_vis, float* scores, hipStream_t s) {
  if (B == 0 || T == 0 || n_max == 0) return hipSuccess;
  dim3 grid((unsigned)((T + kPBM - 1) / kPBM), (unsigned)((n_max + kPBN - 1) / kPBN), (unsigned)B);
  hipLaunchKernelGGL(index_prefill_kernel, grid, dim3(256), 0, s, q, k, T, Hi * Di, n_max, n_vis, scores);
  return hipGetLastError();
}

}  // namespace csa2
