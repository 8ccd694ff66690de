// FP4 main-KV codec: E2M1 values with one E4M3 scale per 16 channels (no global scale).
// Source: DeepSeek-V4.1-Flash walkthrough (wkq9411.github.io), 一(五)4 FP4 Main KV Cache.
//
// Quantize: one wave per entry. Lane l holds 8 consecutive channels of a 512-channel slice, so a
// 16-channel scale group is a lane pair and its amax needs one xor-1 exchange. The packed entry
// (dim/2 code bytes, then dim/16 scale bytes) is assembled in LDS and written out as whole
// 32-bit words, so code and scale bytes leave as one contiguous, coalesced row.
#include "common.h"
#include "launch.h"

namespace csa2 {

constexpr int kQuantWaves = 4;
constexpr int kMaxDim = 4096;

template <bool kBf16>
__global__ __launch_bounds__(kQuantWaves * kWave) void quantize_kernel(const void* __restrict__ src,
                                                                      int64_t n_rows, int dim,
                                                                      uint8_t* __restrict__ rows) {
  // LDS stage for the packed rows of this workgroup (one per wave), 32-bit words
  __shared__ uint32_t stage[kQuantWaves][CSA2_ROW_BYTES(kMaxDim) / 4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * kQuantWaves + wave;
  const int row_bytes = CSA2_ROW_BYTES(dim);
  const int words = row_bytes / 4;
  const int chunks = dim / 8;  // 8-channel chunks
  uint32_t* st = stage[wave];
  uint8_t* st8 = reinterpret_cast<uint8_t*>(st);

  if (row < n_rows) {
    for (int c = lane; c < chunks; c += kWave) {  // c is even on even lanes: groups stay in pairs
      float x[8];
      if (kBf16) {
        const uint4 v = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + row * dim)[c];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[2 * i] = __uint_as_float(w[i] << 16);
          x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
      } else {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(src) + row * dim) + 2 * c;
        const float4 a = p[0], b = p[1];
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
      }
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
      amax = fmaxf(amax, shfl_xor_f(amax, 1));
      const uint32_t sc = e4m3_scale_code(amax);
      const float s = e4m3_mag(sc);
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t j = s > 0.0f ? e2m1_mag_code(fabsf(x[i]), s) : 0u;
        uint32_t code = ((__float_as_uint(x[i]) >> 28) & 8u) | j;
        word |= code << (4 * i);
      }
      st[c] = word;                                   // codes: bytes 4c .. 4c+3
      if ((c & 1) == 0) st8[dim / 2 + (c >> 1)] = (uint8_t)sc;  // scale of group c/2
    }
  }
  __syncthreads();
  if (row < n_rows) {
    uint32_t* dst = reinterpret_cast<uint32_t*>(rows + row * row_bytes);
    for (int w = lane; w < words; w += kWave) dst[w] = st[w];
  }
}

// Stand-alone dequantization to fp32 (the attention kernel dequantizes on its own).
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ rows, int64_t n_rows,
                                                      int dim, float* __restrict__ out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= n_rows) return;
  const int row_bytes = CSA2_ROW_BYTES(dim);
  const uint8_t* r = rows + row * row_bytes;
  for (int c = lane; c < dim / 8; c += kWave) {
    const uint32_t w = reinterpret_cast<const uint32_t*>(r)[c];
    const float s = e4m3_value(r[dim / 2 + (c >> 1)]);
    float v[8];
    e2m1x8_to_f32(w, 0.5f * s, v);
    float4* o = reinterpret_cast<float4*>(out + row * dim) + 2 * c;
    o[0] = make_float4(v[0], v[1], v[2], v[3]);
    o[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

hipError_t launch_quantize(const void* src, bool bf16, int64_t n_rows, int dim, uint8_t* rows,
                           hipStream_t s) {
  if (n_rows == 0) return hipSuccess;
  dim3 grid((unsigned)((n_rows + kQuantWaves - 1) / kQuantWaves)), block(kQuantWaves * kWave);
  if (bf16)
    hipLaunchKernelGGL(quantize_kernel<true>, grid, block, 0, s, src, n_rows, dim, rows);
  else
    hipLaunchKernelGGL(quantize_kernel<false>, grid, block, 0, s, src, n_rows, dim, rows);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* rows, int64_t n_rows, int dim, float* out, hipStream_t s) {
  if (n_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)((n_rows + 3) / 4)), dim3(256), 0, s, rows, n_rows,
                     dim, out);
  return hipGetLastError();
}

}  // namespace csa2
