// Lightweight indexer, prefill form: many query tokens against the same keys.
// Source: DeepSeek-V4.1-Flash walkthrough (wkq9411.github.io), 一(四) (indexer Q x indexer K
// scores every causally visible main-KV entry for each query).
//
// With T query rows the scores are a dense [T x C] x [C x N] contraction (C = Hi*Di), so this
// form runs on v_mfma_f32_32x32x16_bf16: bf16 products are exact and accumulate in fp32.
//
// Main form (C = 256 or 512): query-stationary. Each wave keeps its 32 query rows, all C
// channels, in registers as MFMA A fragments for the whole kernel; a workgroup of 8 waves owns a
// slab of 256 query rows and a contiguous chunk of keys, and streams the chunk through LDS in
// tiles of 32 keys (double-buffered: the next tile is loaded from global memory while the
// current one is multiplied). Each MFMA takes its key fragment from LDS; the fragments are read
// eight steps ahead so LDS latency stays hidden behind the matrix core. Global traffic is the
// keys once per slab plus the queries once. Scores leave the accumulators after every key tile,
// so stores are spread over the whole kernel: in the 32x32 accumulator layout the 32 lanes of a
// half-wave hold 32 consecutive keys of one query row, and each store writes whole 128-byte
// lines.
//
// Other C: a tiled form (256 x 256 score tiles, 8 waves of 128 x 64) with both operands staged
// through double-buffered LDS.
//
// Visibility. Row t sees keys n < n_vis[t]; work past the largest n_vis of a slab (or tile) is
// skipped, key rows past it are not loaded, and stores are masked per row.
//
// Placement. Workgroup i runs on XCD i mod 8. Work items are numbered query-slab-fastest and
// each XCD takes a contiguous range of them, so the workgroups sharing a key chunk run on one XCD
// and the chunk is fetched into that XCD's L2 about once.
#include "common.h"
#include "launch.h"

#include <algorithm>

namespace csa2 {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int WM, int WN, int FM, int FN, int BK>
struct PrefillTile {
  static constexpr int kThreads = 64 * WM * WN;
  static constexpr int kBM = 32 * FM * WM;
  static constexpr int kBN = 32 * FN * WN;
  static constexpr int kPitch = BK + 8;                 // bf16 elements per LDS row
  static constexpr int kStage = (kBM + kBN) * kPitch;   // bf16 elements per buffer
  static constexpr int kChunks = BK / 8;                // 16-byte chunks per row and slice
  static constexpr int kLoadsQ = kBM * kChunks / kThreads;
  static constexpr int kLoadsK = kBN * kChunks / kThreads;
  static_assert(kBM * kChunks % kThreads == 0 && kBN * kChunks % kThreads == 0, "staging split");
  static_assert(BK % 16 == 0, "slice of whole MFMA k-steps");
  static_assert(2 * kStage * 2 + 4 * kBM + 64 <= 160 * 1024, "LDS budget");
};

template <int WM, int WN, int FM, int FN, int BK>
__global__ __launch_bounds__(64 * WM * WN) void index_prefill_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, int T, int C, int n_max,
    const int32_t* __restrict__ n_vis, float* __restrict__ scores, int m_tiles, int n_tiles,
    int per_xcd) {
  using Cfg = PrefillTile<WM, WN, FM, FN, BK>;
  constexpr int NT = Cfg::kThreads, BM = Cfg::kBM, BN = Cfg::kBN, P = Cfg::kPitch;
  constexpr int CH = Cfg::kChunks;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * Cfg::kStage];
  __shared__ int row_nv[BM];
  __shared__ int tile_nv;

  const int u = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (u >= m_tiles * n_tiles) return;
  const int t0 = (u % m_tiles) * BM, n0 = (u / m_tiles) * BN, b = blockIdx.y;
  const int tid = threadIdx.x;

  if (tid == 0) tile_nv = 0;
  __syncthreads();
  for (int r = tid; r < BM; r += NT) {
    int nv = 0;
    if (t0 + r < T) nv = n_vis ? min(n_vis[(int64_t)b * T + t0 + r], n_max) : n_max;
    row_nv[r] = nv;
    if (nv > n0) atomicMax(&tile_nv, nv);
  }
  __syncthreads();
  const int key_end = tile_nv;          // keys n0 .. key_end-1 are visible to some row
  if (key_end <= n0) return;            // uniform: no visible pair in this tile

  const uint16_t* qb = q + (int64_t)b * T * C;
  const uint16_t* kb = k + (int64_t)b * n_max * C;

  u32x4_t rq[Cfg::kLoadsQ], rk[Cfg::kLoadsK];
  auto gload = [&](int c0) {
#pragma unroll
    for (int i = 0; i < Cfg::kLoadsQ; ++i) {
      const int e = tid + i * NT, row = e / CH, ch = e % CH;
      rq[i] = u32x4_t{0u, 0u, 0u, 0u};
      if (t0 + row < T) rq[i] = *reinterpret_cast<const u32x4_t*>(qb + (int64_t)(t0 + row) * C + c0 + 8 * ch);
    }
#pragma unroll
    for (int i = 0; i < Cfg::kLoadsK; ++i) {
      const int e = tid + i * NT, row = e / CH, ch = e % CH;
      rk[i] = u32x4_t{0u, 0u, 0u, 0u};
      if (n0 + row < key_end) rk[i] = *reinterpret_cast<const u32x4_t*>(kb + (int64_t)(n0 + row) * C + c0 + 8 * ch);
    }
  };
  auto lstore = [&](int buf) {
    uint16_t* s = lds + buf * Cfg::kStage;
#pragma unroll
    for (int i = 0; i < Cfg::kLoadsQ; ++i) {
      const int e = tid + i * NT, row = e / CH, ch = e % CH;
      *reinterpret_cast<u32x4_t*>(s + row * P + 8 * ch) = rq[i];
    }
#pragma unroll
    for (int i = 0; i < Cfg::kLoadsK; ++i) {
      const int e = tid + i * NT, row = e / CH, ch = e % CH;
      *reinterpret_cast<u32x4_t*>(s + (BM + row) * P + 8 * ch) = rk[i];
    }
  };

  const int wave = tid >> 6, lane = tid & 63;
  const int wm = (wave / WN) * FM * 32, wn = (wave % WN) * FN * 32;
  const int lr = lane & 31, lh = lane >> 5;

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  gload(0);
  lstore(0);
  __syncthreads();
  const int nk = C / BK;
  for (int ks = 0; ks < nk; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < nk) gload((ks + 1) * BK);
    const uint16_t* s = lds + buf * Cfg::kStage;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      // 32x32x16 operands: lane holds row/column (lane % 32), channels 8*(lane/32) .. +7
      bf16x8_t a[FM], bv[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        a[i] = *reinterpret_cast<const bf16x8_t*>(s + (wm + 32 * i + lr) * P + kk + 8 * lh);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bv[j] = *reinterpret_cast<const bf16x8_t*>(s + (BM + wn + 32 * j + lr) * P + kk + 8 * lh);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bv[j], acc[i][j], 0, 0, 0);
    }
    if (ks + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // accumulator r of block (i, j): query row wm + 32i + 8(r/4) + 4(lane/32) + r%4, key wn + 32j + lane%32
  float* sb = scores + (int64_t)b * T * n_max;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
      const int nv = row_nv[row];  // 0 for rows past T
      float* srow = sb + (int64_t)(t0 + row) * n_max;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = n0 + wn + 32 * j + lr;
        if (n < nv) srow[n] = acc[i][j][r];
      }
    }
}


template <int C, int KT, int PD, int NW, int RB, bool kBufStore>
__global__ __launch_bounds__(64 * NW) void index_prefill_qs_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, int T, int n_max,
    const int32_t* __restrict__ n_vis, float* __restrict__ scores, int m_slabs, int n_chunks,
    int chunk_keys, int per_xcd) {
  constexpr int NT = 64 * NW, WR = 32 * RB, BM = WR * NW, KS = C / 16;
  constexpr int P = C + 8;                        // bf16 per LDS key row (16-byte pad)
  constexpr int LOADS = KT * (C / 8) / NT;        // 16-byte loads per thread per key tile
  constexpr int NS = KS * (KT / 32);              // key-fragment steps per tile: step = s * (KT/32) + j
  static_assert(KT % 32 == 0 && KT * (C / 8) % NT == 0, "key tile split");
  __shared__ __attribute__((aligned(16))) uint16_t ks[2][KT * P];
  __shared__ int row_nv[BM];
  __shared__ int slab_nv;

  const int u = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (u >= m_slabs * n_chunks) return;
  const int t0 = (u % m_slabs) * BM, n_begin = (u / m_slabs) * chunk_keys, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: row bases stay scalar
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

  // A fragments: row block rb holds rows WR*wave + 32 rb + lane%32, channels 16s + 8*(lane/32) .. +7
  bf16x8_t qa[RB][KS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int t = t0 + WR * wave + 32 * rb + lr;
    const uint16_t* qr = q + ((int64_t)b * T + t) * C + 8 * lh;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (t < T) v = *reinterpret_cast<const u32x4_t*>(qr + 16 * s);
      qa[rb][s] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  const uint16_t* kb = k + (int64_t)b * n_max * C;
  u32x4_t stg[LOADS];
  auto gload = [&](int n0) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int e = tid + i * NT, row = e / (C / 8), ch = e % (C / 8);
      stg[i] = u32x4_t{0u, 0u, 0u, 0u};
      if (n0 + row < n_end) stg[i] = *reinterpret_cast<const u32x4_t*>(kb + (int64_t)(n0 + row) * C + 8 * ch);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int e = tid + i * NT, row = e / (C / 8), ch = e % (C / 8);
      *reinterpret_cast<u32x4_t*>(&ks[buf][row * P + 8 * ch]) = stg[i];
    }
  };

  float* sw = scores + ((int64_t)b * T + t0 + WR * wave) * n_max;  // this wave's first row
  // this wave's rows as one buffer range (used when WR rows fit in 2^31 bytes)
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
    f32x16_t acc[RB][KT / 32];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int j = 0; j < KT / 32; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[rb][j][r] = 0.f;
    // B fragments: key 32j + lane%32 of the tile, channels 16s + 8*(lane/32) .. +7; each feeds RB MFMAs
    const uint16_t* kt = &ks[buf][lr * P + 8 * lh];
    auto bload = [&](int step) {
      return *reinterpret_cast<const bf16x8_t*>(kt + 32 * (step % (KT / 32)) * P + 16 * (step / (KT / 32)));
    };
    bf16x8_t bq[PD];
#pragma unroll
    for (int d = 0; d < PD; ++d) bq[d] = bload(d);
#pragma unroll
    for (int step = 0; step < NS; ++step) {
      const bf16x8_t cur = bq[step % PD];
      if (step + PD < NS) bq[step % PD] = bload(step + PD);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        acc[rb][step % (KT / 32)] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            qa[rb][step / (KT / 32)], cur, acc[rb][step % (KT / 32)], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);  // keep the reads PD steps ahead of their MFMAs
    }
    // accumulator r of block (rb, j): row 32 rb + 8(r/4) + 4(lane/32) + r%4 of the wave, key n0 + 32j + lane%32
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * rb + 8 * (r >> 2) + 4 * lh + (r & 3);
        const int nv = row_nv[WR * wave + row];  // 0 for rows past T
#pragma unroll
        for (int j = 0; j < KT / 32; ++j) {
          const int n = n0 + 32 * j + lr;
          if (kBufStore) {
            // unconditional: masked lanes get an offset past the range, which the hardware drops,
            // so the compiler can count the stores and never waits for them
            const int off = n < nv ? (row * n_max + n) * 4 : (int)0x80000000;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[rb][j][r]), srsrc, off, 0, 0);
          } else if (n < nv) {
            sw[(int64_t)row * n_max + n] = acc[rb][j][r];
          }
        }
      }
    if (more) lstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
}

namespace {

template <int WM, int WN, int FM, int FN, int BK>
hipError_t launch_prefill_cfg(const uint16_t* q, const uint16_t* k, int B, int T, int C, int n_max,
                              const int32_t* n_vis, float* scores, hipStream_t s) {
  using Cfg = PrefillTile<WM, WN, FM, FN, BK>;
  const int m_tiles = (T + Cfg::kBM - 1) / Cfg::kBM;
  const int n_tiles = (n_max + Cfg::kBN - 1) / Cfg::kBN;
  const int64_t tiles = (int64_t)m_tiles * n_tiles;
  const int per_xcd = (int)((tiles + 7) / 8);
  dim3 grid((unsigned)(8 * per_xcd), (unsigned)B);
  hipLaunchKernelGGL((index_prefill_kernel<WM, WN, FM, FN, BK>), grid, dim3(Cfg::kThreads), 0, s, q, k, T, C,
                     n_max, n_vis, scores, m_tiles, n_tiles, per_xcd);
  return hipGetLastError();
}


template <int C, int NW, int RB>
hipError_t launch_prefill_qs(const uint16_t* q, const uint16_t* k, int B, int T, int n_max,
                             const int32_t* n_vis, float* scores, hipStream_t s) {
  constexpr int KT = 32, BM = 32 * RB * NW;
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
    hipLaunchKernelGGL((index_prefill_qs_kernel<C, KT, 8, NW, RB, true>), grid, block, 0, s, q, k, T, n_max, n_vis,
                       scores, m_slabs, n_chunks, chunk_keys, per_xcd);
  else
    hipLaunchKernelGGL((index_prefill_qs_kernel<C, KT, 8, NW, RB, false>), grid, block, 0, s, q, k, T, n_max, n_vis,
                       scores, m_slabs, n_chunks, chunk_keys, per_xcd);
  return hipGetLastError();
}
}  // namespace

// Causal visibility of the compressed entries for a chunk of query tokens: the query at absolute
// position p sees entry n once the entry's last source token is at or before p, i.e. n < (p+1) / ratio
// (floor), capped at n_max. One thread per query row.
__global__ void prefill_visibility_kernel(const int64_t* __restrict__ p0, int T, int ratio, int n_max,
                                          int64_t rows, int32_t* __restrict__ n_vis) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  const int64_t pos = p0[r / T] + r % T;
  const int64_t v = (pos + 1) / ratio;
  n_vis[r] = (int32_t)(v < 0 ? 0 : (v > n_max ? n_max : v));
}

hipError_t launch_prefill_visibility(const int64_t* p0, int B, int T, int ratio, int n_max, int32_t* n_vis,
                                     hipStream_t s) {
  const int64_t rows = (int64_t)B * T;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_visibility_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, p0, T, ratio,
                     n_max, rows, n_vis);
  return hipGetLastError();
}

bool index_prefill_supported(int T, int Hi, int Hk, int Di) {
  return T >= 16 && Hk == Hi && (Hi * Di) % 64 == 0;
}

hipError_t launch_index_prefill(const uint16_t* q, const uint16_t* k, int B, int T, int Hi, int Di,
                                int n_max, const int32_t* n_vis, float* scores, hipStream_t s) {
  if (B == 0 || T == 0 || n_max == 0) return hipSuccess;
  const int C = Hi * Di;
  if (C == 512) return launch_prefill_qs<512, 8, 1>(q, k, B, T, n_max, n_vis, scores, s);
  if (C == 256) return launch_prefill_qs<256, 8, 1>(q, k, B, T, n_max, n_vis, scores, s);
  // 8 waves of 128 x 64, 256 x 256 tiles, 64-channel slices
  return launch_prefill_cfg<2, 4, 4, 2, 64>(q, k, B, T, C, n_max, n_vis, scores, s);
}

}  // namespace csa2
