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
// Work split: a workgroup of 4 waves owns 32 consecutive entries of the flattened (sequence,
// entry) list. A wave compresses 8 of them, two at a time, with a lane holding 8 consecutive
// channels (16-byte loads of every token of both entries are in flight together); the 8 channels
// are half of a 16-channel scale group, so the group maximum needs one lane exchange, and the
// lane's eight 4-bit codes are one 32-bit word of the packed row. The bf16 entries meet in LDS as
// the A operand of the projection; wave w then computes the keys' channel columns
// [w C/4, (w+1) C/4) for all 32 entries, with the weight rows as B fragments read from global
// memory (the weight is shared by every workgroup and stays in L2).
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

template <int M>
__global__ __launch_bounds__(256) void compress_kv_kernel(
    const uint16_t* __restrict__ c, const uint16_t* __restrict__ z, int n_tok, int n_new, int64_t n_entries,
    const int32_t* __restrict__ entry0, int n_max, uint8_t* __restrict__ rows, const uint16_t* __restrict__ w_t,
    int c_out, uint16_t* __restrict__ k_idx, float* __restrict__ entries) {
  __shared__ __attribute__((aligned(16))) uint16_t ebf[kCmpEntries * kCmpPitch];
  __shared__ int64_t dest[kCmpEntries];    // b * n_max + entry index, or -1 (not written)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t q0 = (int64_t)blockIdx.x * kCmpEntries;

  if (tid < kCmpEntries) {
    const int64_t q = q0 + tid;
    int64_t d = -1;
    if (q < n_entries) {
      const int b = (int)(q / n_new), j = (int)(q % n_new);
      const int n = entry0[b] + j;
      if (n >= 0 && n < n_max) d = (int64_t)b * n_max + n;
    }
    dest[tid] = d;
  }
  __syncthreads();

  // ---- compress, pack, stage the bf16 entry for the projection ----
#pragma unroll 1
  for (int p = 0; p < kCmpEntries / 4; p += 2) {
    int loc[2];
    bool ok[2];
    u32x4_t cv[2][M], zv[2][M];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      loc[u] = wave + 4 * (p + u);
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
    for (int u = 0; u < 2; ++u) {
      float e[8];
#pragma unroll
      for (int ch = 0; ch < 8; ++ch) {
        float cf[M], zf[M];
#pragma unroll
        for (int i = 0; i < M; ++i) {
          const uint32_t wc = cv[u][i][ch >> 1], wz = zv[u][i][ch >> 1];
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
      // FP4: the lane's 8 channels are half of a 16-channel scale group (lanes 2g, 2g+1)
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
      const int64_t d = dest[loc[u]];
      if (ok[u] && d >= 0) {
        uint8_t* row = rows + d * CSA2_ROW_BYTES(kCmpD);
        reinterpret_cast<uint32_t*>(row)[lane] = word;               // codes of channels 8 lane ..
        if ((lane & 1) == 0) row[kCmpD / 2 + (lane >> 1)] = (uint8_t)sc;
      }
      if (entries && ok[u]) {
        float4* ep = reinterpret_cast<float4*>(entries + (q0 + loc[u]) * kCmpD + 8 * lane);
        ep[0] = make_float4(e[0], e[1], e[2], e[3]);
        ep[1] = make_float4(e[4], e[5], e[6], e[7]);
      }
      u32x4_t packed;
#pragma unroll
      for (int h = 0; h < 4; ++h) packed[h] = f32_to_bf16_rne(e[2 * h]) | (f32_to_bf16_rne(e[2 * h + 1]) << 16);
      *reinterpret_cast<u32x4_t*>(&ebf[loc[u] * kCmpPitch + 8 * lane]) = packed;
    }
  }
  if (!k_idx) return;                      // uniform: no projection asked for
  __syncthreads();

  // ---- indexer keys: [32 entries x 512] x [512 x c_out], wave w owns columns [w c_out/4, ..) ----
  const int lr = lane & 31, lh = lane >> 5;
  const int cols = c_out / 4, tiles = cols / 32;
  for (int t = 0; t < tiles; ++t) {
    const int o = wave * cols + 32 * t + lr;             // this lane's key channel (B column)
    const uint16_t* wrow = w_t + (int64_t)o * kCmpD + 8 * lh;
    const uint16_t* arow = &ebf[lr * kCmpPitch + 8 * lh];
    f32x16_t acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    bf16x8_t bw[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) bw[s] = *reinterpret_cast<const bf16x8_t*>(wrow + 16 * s);
#pragma unroll
    for (int s = 0; s < kCmpD / 16; ++s) {
      const bf16x8_t b = bw[s & 3];
      if (s + 4 < kCmpD / 16) bw[s & 3] = *reinterpret_cast<const bf16x8_t*>(wrow + 16 * (s + 4));
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(arow + 16 * s);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
    }
    // accumulator r: entry 8 (r/4) + 4 (lane/32) + r%4, key channel o
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ent = 8 * (r >> 2) + 4 * lh + (r & 3);
      const int64_t d = dest[ent];
      if (d >= 0) k_idx[d * c_out + o] = (uint16_t)f32_to_bf16_rne(acc[r]);
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
  const dim3 grid((unsigned)((n_entries + kCmpEntries - 1) / kCmpEntries)), block(256);
#define CSA2_CMP(M)                                                                                            \
  hipLaunchKernelGGL((compress_kv_kernel<M>), grid, block, 0, s, c, z, n_tok, n_new, n_entries, entry0, n_max, \
                     rows, w_t, c_out, k_idx, entries)
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
