// Lightweight indexer over FP4 query and key rows (OCP MXFP4), prefill form on the scaled FP4
// matrix cores.
// Source: DeepSeek-V4.1-Flash walkthrough (wkq9411.github.io), 一(五)4 "FP4 Main KV Cache": the
// indexer query and key are FP4 in the OCP MXFP4 format (E2M1 elements, one power-of-two E8M0
// scale per 32 channels), to speed up index computation; 一(四): each query scores every
// causally visible main-KV entry.
//
// With T query rows the scores are a dense [T x C] x [C x N] contraction whose operands already
// are MX blocks of 32 channels, which is exactly the operand format of gfx950's
// v_mfma_scale_f32_32x32x64_f8f6f4 with E2M1 inputs: per MFMA, 32 query rows x 32 keys x 64
// channels, lane l holding 32 channels (16 code bytes) of row or key l % 32, block l / 32 of the
// step, and that block's E8M0 scale byte. Products of E2M1 values times the two powers of two
// are exact; the sum is accumulated in fp32.
//
// Query-stationary, as the bf16 prefill indexer: each wave keeps its 64 query rows (two 32-row
// blocks) as MFMA A fragments and E8M0 scales in registers for the whole kernel (FP4 rows are a
// quarter of the bf16 bytes, so a workgroup of 8 waves holds 512 rows); key tiles of 32 rows
// stream through double-buffered LDS as contiguous byte ranges (C/2 + C/32 bytes per key).
// Every key tile read from L2 serves 512 query rows, so the kernel's traffic is almost only the
// fp32 score writes, which leave the accumulators after every tile through buffer stores whose
// masked lanes get an out-of-range offset (dropped by the hardware).
//
// Visibility: row t sees keys n < n_vis[t]; tiles past a slab's largest n_vis are skipped and
// stores are masked per row. Placement: workgroup i runs on XCD i mod 8 and the workgroups that
// share a key chunk sit on one XCD.
#include "common.h"
#include "launch.h"

#include <algorithm>
#include <type_traits>

namespace csa2 {

typedef int i32x8_mx_t __attribute__((ext_vector_type(8)));
typedef float f32x16_mx_t __attribute__((ext_vector_type(16)));

template <int C, int NW, int RB, bool kBufStore>
__global__ __launch_bounds__(64 * NW) void index_mxfp4_prefill_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k, int T, int n_max,
    const int32_t* __restrict__ n_vis, float* __restrict__ scores, int m_slabs, int n_chunks, int chunk_keys,
    int per_xcd) {
  constexpr int NT = 64 * NW, WR = 32 * RB, BM = WR * NW;
  constexpr int RBYTES = C / 2 + C / 32;          // bytes per MXFP4 row: 272 (C = 512) or 136 (C = 256)
  constexpr int KS = C / 64;                      // MFMA steps per row
  constexpr int KT = 32;                          // keys per tile
  constexpr int TILE = KT * RBYTES;               // bytes per key tile (contiguous in memory)
  constexpr int LW = C == 512 ? 16 : 8;           // bytes per staging load (row pitch 272 or 136)
  constexpr int LOADS = (TILE / LW + NT - 1) / NT;
  static_assert(TILE % LW == 0, "tile of whole loads");
  __shared__ __attribute__((aligned(16))) uint8_t ks[2][TILE];
  __shared__ int row_nv[BM];
  __shared__ int slab_nv;

  const int u = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (u >= m_slabs * n_chunks) return;
  const int t0 = (u % m_slabs) * BM, n_begin = (u / m_slabs) * chunk_keys, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, lh = lane >> 5;
  if (tid == 0) slab_nv = 0;
  __syncthreads();
  for (int r = tid; r < BM; r += NT) {
    int nv = 0;
    if (t0 + r < T) nv = n_vis ? min(n_vis[(int64_t)b * T + t0 + r], n_max) : n_max;
    row_nv[r] = nv;
    atomicMax(&slab_nv, nv);
  }
  __syncthreads();
  const int n_end = min(n_begin + chunk_keys, slab_nv);
  if (n_end <= n_begin) return;  // uniform: nothing visible in this chunk

  // A fragments: block rb holds rows WR*wave + 32 rb + lane%32; step s takes code bytes
  // 32 s + 16 (lane/32) .. +15 (channels 64 s + 32 (lane/32) ..) and scale byte 2 s + lane/32
  u32x4_t qa[RB][KS];
  int qs[RB][KS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int t = t0 + WR * wave + 32 * rb + lr;
    const uint8_t* qr = q + ((int64_t)b * T + t) * RBYTES;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qa[rb][s] = u32x4_t{0u, 0u, 0u, 0u};
      qs[rb][s] = 127;
      if (t < T) {
        const uint2 lo = *reinterpret_cast<const uint2*>(qr + 32 * s + 16 * lh);
        const uint2 hi = *reinterpret_cast<const uint2*>(qr + 32 * s + 16 * lh + 8);
        qa[rb][s] = u32x4_t{lo.x, lo.y, hi.x, hi.y};
        qs[rb][s] = qr[C / 2 + 2 * s + lh];
      }
    }
  }
  const uint8_t* kb = k + (int64_t)b * n_max * RBYTES;
  typedef typename std::conditional<LW == 16, u32x4_t, uint2>::type chunk_t;
  chunk_t stg[LOADS];
  auto gload = [&](int n0) {
    const int64_t base = (int64_t)n0 * RBYTES;
    const int avail = (n_end - n0) * RBYTES;      // bytes of visible keys in this tile
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int e = (tid + i * NT) * LW;
      stg[i] = chunk_t{};
      if (e < TILE && e < avail) stg[i] = *reinterpret_cast<const chunk_t*>(kb + base + e);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int e = (tid + i * NT) * LW;
      if (e < TILE) *reinterpret_cast<chunk_t*>(&ks[buf][e]) = stg[i];
    }
  };

  float* sw = scores + ((int64_t)b * T + t0 + WR * wave) * n_max;  // this wave's first row
  __amdgpu_buffer_rsrc_t srsrc;
  {
    const uint64_t a = reinterpret_cast<uint64_t>(sw);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a), hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const int bytes = __builtin_amdgcn_readfirstlane(kBufStore ? max(0, min(WR, T - t0 - WR * wave)) * n_max * 4 : 0);
    srsrc = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), 0, bytes, 0x00020000);
  }
  gload(n_begin);
  lstore(0);
  __syncthreads();
  int buf = 0;
  for (int n0 = n_begin; n0 < n_end; n0 += KT) {
    const bool more = n0 + KT < n_end;
    if (more) gload(n0 + KT);
    // B fragments of the tile: key lane%32, the same channel split as the A fragments
    const uint8_t* kr = &ks[buf][lr * RBYTES];
    u32x4_t kf[KS];
    int ksc[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (C == 512) {
        kf[s] = *reinterpret_cast<const u32x4_t*>(kr + 32 * s + 16 * lh);
      } else {
        const uint2 lo = *reinterpret_cast<const uint2*>(kr + 32 * s + 16 * lh);
        const uint2 hi = *reinterpret_cast<const uint2*>(kr + 32 * s + 16 * lh + 8);
        kf[s] = u32x4_t{lo.x, lo.y, hi.x, hi.y};
      }
      ksc[s] = kr[C / 2 + 2 * s + lh];
    }
    f32x16_mx_t acc[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][r] = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const i32x8_mx_t bv = {(int)kf[s][0], (int)kf[s][1], (int)kf[s][2], (int)kf[s][3], 0, 0, 0, 0};
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const i32x8_mx_t av = {(int)qa[rb][s][0], (int)qa[rb][s][1], (int)qa[rb][s][2], (int)qa[rb][s][3], 0, 0, 0, 0};
        // E2M1 x E2M1 (format code 4 for both operands), E8M0 scales in byte 0 of the scale operands
        acc[rb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc[rb], 4, 4, 0, qs[rb][s], 0, ksc[s]);
      }
    }
    // accumulator r of block rb: row 32 rb + 8(r/4) + 4(lane/32) + r%4 of the wave, key n0 + lane%32
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * rb + 8 * (r >> 2) + 4 * lh + (r & 3);
        const int nv = row_nv[WR * wave + row];  // 0 for rows past T
        const int n = n0 + lr;
        if (kBufStore) {
          const int off = n < nv ? (row * n_max + n) * 4 : (int)0x80000000;
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[rb][r]), srsrc, off, 0, 0);
        } else if (n < nv) {
          sw[(int64_t)row * n_max + n] = acc[rb][r];
        }
      }
    if (more) lstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
}

bool index_mxfp4_prefill_supported(int T, int Hi, int Hk, int Di) {
  return T >= 16 && Hk == Hi && (Hi * Di == 256 || Hi * Di == 512);
}

template <int C>
static hipError_t launch_mx_prefill_c(const uint8_t* q, const uint8_t* k, int B, int T, int n_max,
                                      const int32_t* n_vis, float* scores, hipStream_t s) {
  constexpr int NW = 8, RB = 2, KT = 32, BM = 32 * RB * NW;
  const int m_slabs = (T + BM - 1) / BM;
  // about one workgroup per CU: split the keys into chunks of whole tiles
  int n_chunks = std::max(1, 256 / m_slabs);
  int chunk_keys = (n_max + n_chunks - 1) / n_chunks;
  chunk_keys = (chunk_keys + KT - 1) / KT * KT;
  n_chunks = (n_max + chunk_keys - 1) / chunk_keys;
  const int64_t items = (int64_t)m_slabs * n_chunks;
  const int per_xcd = (int)((items + 7) / 8);
  const dim3 grid((unsigned)(8 * per_xcd), (unsigned)B), block(64 * NW);
  if ((int64_t)32 * RB * n_max * 4 <= ((int64_t)1 << 31) - 4)
    hipLaunchKernelGGL((index_mxfp4_prefill_kernel<C, NW, RB, true>), grid, block, 0, s, q, k, T, n_max, n_vis,
                       scores, m_slabs, n_chunks, chunk_keys, per_xcd);
  else
    hipLaunchKernelGGL((index_mxfp4_prefill_kernel<C, NW, RB, false>), grid, block, 0, s, q, k, T, n_max, n_vis,
                       scores, m_slabs, n_chunks, chunk_keys, per_xcd);
  return hipGetLastError();
}

hipError_t launch_index_mxfp4_prefill(const uint8_t* q, const uint8_t* k, int B, int T, int Hi, int Di, int n_max,
                                      const int32_t* n_vis, float* scores, hipStream_t s) {
  if (B == 0 || T == 0 || n_max == 0) return hipSuccess;
  if (Hi * Di == 512) return launch_mx_prefill_c<512>(q, k, B, T, n_max, n_vis, scores, s);
  return launch_mx_prefill_c<256>(q, k, B, T, n_max, n_vis, scores, s);
}

}  // namespace csa2
