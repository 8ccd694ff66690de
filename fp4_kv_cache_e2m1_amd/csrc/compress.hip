// Producing the caches: the CSA2 compressor, the FP4 packing of its entries and the indexer-K
// projection, fused in one kernel.
// Source: DeepSeek-V4.1-Flash walkthrough (wkq9411.github.io), 一(三) (a layer's KV entries C and
// their compression weights Z are projections of the hidden states), 一(四) (CSA2's simplified
// compressor turns m tokens into one entry with no overlap between entries and no absolute
// position encoding; indexer K is a projection of the main-KV entries) and 一(五)4 (the main KV
// is stored as E2M1 values with one E4M3 scale per 16 channels).
//
// Entry j of a sequence combines its tokens jm .. jm+m-1 channel by channel with softmax weights
// over their compression weights: e[d] = sum_i softmax_i(z_i[d]) c_i[d] (fp32; exponentials with
// the group's largest weight subtracted). The entry is packed to FP4 with the same exact-compare
// quantizer as the stand-alone packing call, and its bf16 rounding is multiplied by the
// projection weight on v_mfma_f32_32x32x16_bf16 (exact products, fp32 accumulation), giving the
// entry's indexer key in bf16.
//
// Work split: workgroup (x, y) of 8 waves owns NE (8, 16 or 32) consecutive entries x of the
// flattened (sequence, entry) list and key channels [256 y, 256 y + 256), NE the smallest that
// keeps the grid to one workgroup per CU (the call is a chain of memory round trips, so spreading
// it over the CUs shortens it: 1024 entries 24.2 -> 15.0 us, 2048 entries 25.1 -> 18.6 us). A
// wave compresses NE / 8 of the entries with a lane holding 8 consecutive channels; the 16-byte
// loads of every token of its entries are issued together (two rounds for 8 tokens per entry).
// The 8 channels are half of a 16-channel scale group, so the group maximum needs one lane
// exchange, and the lane's eight 4-bit codes are one 32-bit word of the packed row (written by
// the y = 0 workgroups only). The bf16 entries meet in LDS as the A operand of the projection
// (rows past NE unused); wave w then computes the 32 key channels 256 y + 32 w .. for the
// entries, its 32 weight fragments (one 32 x 512 slice of the weight) all loaded at once, so the
// whole call costs about two memory round trips when only a few entries are new (decode appends
// one entry per sequence).
#include "common.h"
#include "launch.h"

namespace csa2 {

constexpr int kCmpEntries = 32;          // entries per workgroup
constexpr int kCmpD = 512;               // channels of an entry
constexpr int kCmpPitch = kCmpD + 8;     // bf16 per LDS entry row (16-byte pad)

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// fp32 -> bf16 bits, round to nearest even (finite values)
CSA2_DEV uint32_t f32_to_bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

constexpr int kCmpWaves = 8;
constexpr int kCmpCols = 32 * kCmpWaves;          // key channels per workgroup

// One entry's 8 channels of this lane from its M tokens' KV values and compression weights
// (16-byte rows of 8 bf16 each): softmax over the tokens per channel, weighted sum.
template <int M>
CSA2_DEV void compress_lane(const u32x4_t (&cv)[M], const u32x4_t (&zv)[M], float (&e)[8]) {
#pragma unroll
  for (int ch = 0; ch < 8; ++ch) {
    float cf[M], zf[M];
#pragma unroll
    for (int i = 0; i < M; ++i) {
      const uint32_t wc = cv[i][ch >> 1], wz = zv[i][ch >> 1];
      cf[i] = __uint_as_float((ch & 1) ? (wc & 0xFFFF0000u) : (wc << 16));
      zf[i] = __uint_as_float((ch & 1) ? (wz & 0xFFFF0000u) : (wz << 16));
    }
    if (M == 1) {
      e[ch] = cf[0];
    } else {
      float zm = zf[0];
#pragma unroll
      for (int i = 1; i < M; ++i) zm = fmaxf(zm, zf[i]);
      float s = 0.0f, a = 0.0f;
#pragma unroll
      for (int i = 0; i < M; ++i) {
        const float w = __expf(zf[i] - zm);
        s += w;
        a = fmaf(w, cf[i], a);
      }
      e[ch] = a / s;
    }
  }
}

// FP4 packing of the lane's 8 channels (half of a 16-channel scale group, lanes 2g and 2g+1
// together) into row `row` (null: not written); the wave's 64 lanes cover the 512 channels.
CSA2_DEV void pack_lane(const float (&e)[8], uint8_t* row, int lane) {
  float amax = 0.0f;
#pragma unroll
  for (int ch = 0; ch < 8; ++ch) amax = fmaxf(amax, fabsf(e[ch]));
  amax = fmaxf(amax, shfl_xor_f(amax, 1));
  const uint32_t sc = e4m3_scale_code(amax);
  const float s = e4m3_mag(sc);
  uint32_t word = 0;
#pragma unroll
  for (int ch = 0; ch < 8; ++ch) {
    const uint32_t j = s > 0.0f ? e2m1_mag_code(fabsf(e[ch]), s) : 0u;
    word |= (((__float_as_uint(e[ch]) >> 28) & 8u) | j) << (4 * ch);
  }
  if (row) {
    reinterpret_cast<uint32_t*>(row)[lane] = word;                 // codes of channels 8 lane ..
    if ((lane & 1) == 0) row[kCmpD / 2 + (lane >> 1)] = (uint8_t)sc;
  }
}

CSA2_DEV u32x4_t bf16x8_of(const float (&e)[8]) {
  u32x4_t packed;
#pragma unroll
  for (int h = 0; h < 4; ++h) packed[h] = f32_to_bf16_rne(e[2 * h]) | (f32_to_bf16_rne(e[2 * h + 1]) << 16);
  return packed;
}

template <int M, int NE>
__global__ __launch_bounds__(64 * kCmpWaves) void compress_kv_kernel(
    const uint16_t* __restrict__ c, const uint16_t* __restrict__ z, int n_tok, int n_new, int64_t n_entries,
    const int32_t* __restrict__ entry0, int n_max, uint8_t* __restrict__ rows, const uint16_t* __restrict__ w_t,
    int c_out, uint16_t* __restrict__ k_idx, float* __restrict__ entries) {
  constexpr int EPW = NE / kCmpWaves;              // entries per wave
  static_assert(EPW >= 1 && NE <= kCmpEntries, "entries per workgroup");
  constexpr int EB = M <= 2 ? EPW : (M == 4 ? (EPW < 2 ? EPW : 2) : 1);   // entries whose tokens are loaded together
  __shared__ __attribute__((aligned(16))) uint16_t ebf[kCmpEntries * kCmpPitch];
  __shared__ int64_t dest[kCmpEntries];            // b * n_max + entry index, or -1 (not written)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t q0 = (int64_t)blockIdx.x * NE;
  const bool first_cols = blockIdx.y == 0;         // writes the packed rows and fp32 entries

  // rows NE .. 31 of the projection's A operand are never written: their products land in
  // accumulator rows that are not stored (dest -1)
  if (tid < kCmpEntries) {
    const int64_t q = q0 + tid;
    int64_t d = -1;
    if (tid < NE && q < n_entries) {
      const int b = (int)(q / n_new), j = (int)(q % n_new);
      const int n = entry0[b] + j;
      if (n >= 0 && n < n_max) d = (int64_t)b * n_max + n;
    }
    dest[tid] = d;
  }
  // the wave's 32 x 512 slice of the projection weight: 32 fragments, loaded first so that their
  // latency overlaps the compression
  const int lr = lane & 31, lh = lane >> 5;
  const int o0 = kCmpCols * (int)blockIdx.y + 32 * wave;
  const bool project = k_idx != nullptr && o0 < c_out;   // uniform per wave
  const int o = o0 + lr;                                  // this lane's key channel (B column)
  bf16x8_t bw[kCmpD / 16];
  if (project) {
    const uint16_t* wrow = w_t + (int64_t)o * kCmpD + 8 * lh;
#pragma unroll
    for (int s = 0; s < kCmpD / 16; ++s) bw[s] = *reinterpret_cast<const bf16x8_t*>(wrow + 16 * s);
  }
  __builtin_amdgcn_sched_barrier(0);   // keep every weight load ahead of the compression
  __syncthreads();

  // ---- compress, pack, stage the bf16 entry for the projection ----
#pragma unroll
  for (int p = 0; p < EPW; p += EB) {
    int loc[EB];
    bool ok[EB];
    u32x4_t cv[EB][M], zv[EB][M];
#pragma unroll
    for (int u = 0; u < EB; ++u) {
      loc[u] = wave + kCmpWaves * (p + u);
      const int64_t q = q0 + loc[u];
      ok[u] = q < n_entries;
      const int64_t b = ok[u] ? q / n_new : 0, j = ok[u] ? q % n_new : 0;
      const int64_t tok = b * n_tok + j * M;
#pragma unroll
      for (int i = 0; i < M; ++i) {
        cv[u][i] = u32x4_t{0u, 0u, 0u, 0u};
        zv[u][i] = u32x4_t{0u, 0u, 0u, 0u};
        if (ok[u]) {
          cv[u][i] = *reinterpret_cast<const u32x4_t*>(c + (tok + i) * kCmpD + 8 * lane);
          zv[u][i] = *reinterpret_cast<const u32x4_t*>(z + (tok + i) * kCmpD + 8 * lane);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < EB; ++u) {
      float e[8];
      compress_lane<M>(cv[u], zv[u], e);
      if (first_cols) {
        const int64_t d = dest[loc[u]];
        pack_lane(e, ok[u] && d >= 0 ? rows + d * CSA2_ROW_BYTES(kCmpD) : nullptr, lane);
        if (entries && ok[u]) {
          float4* ep = reinterpret_cast<float4*>(entries + (q0 + loc[u]) * kCmpD + 8 * lane);
          ep[0] = make_float4(e[0], e[1], e[2], e[3]);
          ep[1] = make_float4(e[4], e[5], e[6], e[7]);
        }
      }
      *reinterpret_cast<u32x4_t*>(&ebf[loc[u] * kCmpPitch + 8 * lane]) = bf16x8_of(e);
    }
  }
  if (!k_idx) return;                              // uniform: no projection asked for
  __syncthreads();                                 // every wave's bf16 entries are in LDS

  // ---- indexer keys: [32 entries x 512] x [512 x 32] per wave, key channels o0 .. o0 + 31 ----
  if (!project) return;
  const uint16_t* arow = &ebf[lr * kCmpPitch + 8 * lh];
  f32x16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
  for (int s = 0; s < kCmpD / 16; ++s)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8_t*>(arow + 16 * s), bw[s], acc,
                                                  0, 0, 0);
  // accumulator r: entry 8 (r/4) + 4 (lane/32) + r%4, key channel o
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t d = dest[8 * (r >> 2) + 4 * lh + (r & 3)];
    if (d >= 0) k_idx[d * c_out + o] = (uint16_t)f32_to_bf16_rne(acc[r]);
  }
}

// Few new entries (decode appends one per sequence): workgroup (x, y) of 4 waves owns 4 entries
// and the 32 key channels 32 y ..; wave w compresses entry w (every workgroup of the row of
// column groups recomputes it; those with y = 0 write the rows) and multiplies the 4 entries by
// input channels 128 w .. 128 w + 127 of the weight slice; the 4 partial tiles are added in LDS.
// Each workgroup then reads 32 KB of weights and 32 KB of tokens, so the call is about two memory
// round trips on as many CUs as there are column groups times entry groups.
constexpr int kCmpSmallEntries = 4;

template <int M>
__global__ __launch_bounds__(256) void compress_kv_small_kernel(
    const uint16_t* __restrict__ c, const uint16_t* __restrict__ z, int n_tok, int n_new, int64_t n_entries,
    const int32_t* __restrict__ entry0, int n_max, uint8_t* __restrict__ rows, const uint16_t* __restrict__ w_t,
    int c_out, uint16_t* __restrict__ k_idx, float* __restrict__ entries) {
  __shared__ __attribute__((aligned(16))) uint16_t ebf[kCmpEntries * kCmpPitch];
  __shared__ float part[4][16][64];                // per wave: its partial 32 x 32 tile, accumulator layout
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t q = (int64_t)blockIdx.x * kCmpSmallEntries + wave;   // this wave's entry
  const bool ok = q < n_entries;
  const int b = ok ? (int)(q / n_new) : 0, j = ok ? (int)(q % n_new) : 0;
  const int n = ok ? entry0[b] + j : -1;
  const int64_t d = (n >= 0 && n < n_max) ? (int64_t)b * n_max + n : -1;
  const int lr = lane & 31, lh = lane >> 5;
  const int o = 32 * (int)blockIdx.y + lr;         // this lane's key channel
  const bool project = k_idx != nullptr;
  // loads: the entry's M token rows of 16 bytes per lane, and the weight fragments of key channel
  // o over input channels 128 wave + 16 s + 8 (lane/32)
  u32x4_t cv[M], zv[M];
  const int64_t tok = (int64_t)b * n_tok + (int64_t)j * M;
#pragma unroll
  for (int i = 0; i < M; ++i) {
    cv[i] = u32x4_t{0u, 0u, 0u, 0u};
    zv[i] = u32x4_t{0u, 0u, 0u, 0u};
    if (ok) {
      cv[i] = *reinterpret_cast<const u32x4_t*>(c + (tok + i) * kCmpD + 8 * lane);
      zv[i] = *reinterpret_cast<const u32x4_t*>(z + (tok + i) * kCmpD + 8 * lane);
    }
  }
  bf16x8_t bw[8];
  if (project) {
    const uint16_t* wrow = w_t + (int64_t)o * kCmpD + 128 * wave + 8 * lh;
#pragma unroll
    for (int s = 0; s < 8; ++s) bw[s] = *reinterpret_cast<const bf16x8_t*>(wrow + 16 * s);
  }
  float e[8];
  compress_lane<M>(cv, zv, e);
  if (blockIdx.y == 0) {
    pack_lane(e, ok && d >= 0 ? rows + d * CSA2_ROW_BYTES(kCmpD) : nullptr, lane);
    if (entries && ok) {
      float4* ep = reinterpret_cast<float4*>(entries + q * kCmpD + 8 * lane);
      ep[0] = make_float4(e[0], e[1], e[2], e[3]);
      ep[1] = make_float4(e[4], e[5], e[6], e[7]);
    }
  }
  if (!project) return;                            // uniform
  // A operand rows: the 4 entries, then zeros
  *reinterpret_cast<u32x4_t*>(&ebf[wave * kCmpPitch + 8 * lane]) = bf16x8_of(e);
  for (int r = kCmpSmallEntries + wave; r < kCmpEntries; r += 4)
    *reinterpret_cast<u32x4_t*>(&ebf[r * kCmpPitch + 8 * lane]) = u32x4_t{0u, 0u, 0u, 0u};
  __syncthreads();
  const uint16_t* arow = &ebf[lr * kCmpPitch + 128 * wave + 8 * lh];
  f32x16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
  for (int s = 0; s < 8; ++s)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8_t*>(arow + 16 * s), bw[s], acc, 0, 0,
                                                  0);
  // rows 0..3 of the tile are accumulator registers 0..3 of lanes 0..31 (entry 4 (lane/32) + r%4)
#pragma unroll
  for (int r = 0; r < 4; ++r) part[wave][r][lane] = acc[r];
  __syncthreads();
  if (wave == 0 && lh == 0) {
#pragma unroll
    for (int r = 0; r < kCmpSmallEntries; ++r) {
      // the four waves' partial sums, added in wave order
      const float v = ((part[0][r][lane] + part[1][r][lane]) + part[2][r][lane]) + part[3][r][lane];
      const int64_t qr = (int64_t)blockIdx.x * kCmpSmallEntries + r;
      if (qr < n_entries) {
        const int br = (int)(qr / n_new), jr = (int)(qr % n_new);
        const int nr = entry0[br] + jr;
        if (nr >= 0 && nr < n_max) k_idx[((int64_t)br * n_max + nr) * c_out + o] = (uint16_t)f32_to_bf16_rne(v);
      }
    }
  }
}

bool compress_ratio_supported(int ratio) { return ratio == 1 || ratio == 2 || ratio == 4 || ratio == 8; }

hipError_t launch_compress_kv(const uint16_t* c, const uint16_t* z, int B, int n_tok, int ratio,
                              const int32_t* entry0, int n_max, uint8_t* rows, const uint16_t* w_t, int c_out,
                              uint16_t* k_idx, float* entries, hipStream_t s) {
  const int n_new = n_tok / ratio;
  const int64_t n_entries = (int64_t)B * n_new;
  if (n_entries == 0) return hipSuccess;
  // few entries: 4 per workgroup and 32 key channels per workgroup, so the weight and the tokens
  // are spread over many CUs; many entries: 32 per workgroup, 256 key channels per workgroup
  const bool small = n_entries <= 512;
  const int col_groups = k_idx ? (c_out + (small ? 32 : kCmpCols) - 1) / (small ? 32 : kCmpCols) : 1;
  int ne = kCmpEntries;
  for (int cand = 8; cand < kCmpEntries; cand *= 2)
    if ((n_entries + cand - 1) / cand * col_groups <= device_cu_count()) {
      ne = cand;
      break;
    }
  const int per = small ? kCmpSmallEntries : ne;
  const dim3 grid((unsigned)((n_entries + per - 1) / per), (unsigned)col_groups), block(small ? 256 : 64 * kCmpWaves);
#define CSA2_CMP(M)                                                                                                \
  if (small)                                                                                                       \
    hipLaunchKernelGGL((compress_kv_small_kernel<M>), grid, block, 0, s, c, z, n_tok, n_new, n_entries, entry0,    \
                       n_max, rows, w_t, c_out, k_idx, entries);                                                   \
  else if (ne == 8)                                                                                                \
    hipLaunchKernelGGL((compress_kv_kernel<M, 8>), grid, block, 0, s, c, z, n_tok, n_new, n_entries, entry0, n_max, \
                       rows, w_t, c_out, k_idx, entries);                                                            \
  else if (ne == 16)                                                                                               \
    hipLaunchKernelGGL((compress_kv_kernel<M, 16>), grid, block, 0, s, c, z, n_tok, n_new, n_entries, entry0,       \
                       n_max, rows, w_t, c_out, k_idx, entries);                                                     \
  else                                                                                                             \
    hipLaunchKernelGGL((compress_kv_kernel<M, 32>), grid, block, 0, s, c, z, n_tok, n_new, n_entries, entry0,       \
                       n_max, rows, w_t, c_out, k_idx, entries)
  switch (ratio) {
    case 1: CSA2_CMP(1); break;
    case 2: CSA2_CMP(2); break;
    case 4: CSA2_CMP(4); break;
    case 8: CSA2_CMP(8); break;
    default: return hipErrorInvalidValue;
  }
#undef CSA2_CMP
  return hipGetLastError();
}

}  // namespace csa2
