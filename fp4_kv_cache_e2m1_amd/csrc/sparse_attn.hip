// Sparse attention over the selected FP4 main-KV entries.
// Source: DeepSeek-V4.1-Flash walkthrough (wkq9411.github.io), 一(四) (each query attends to its
// selected main-KV entries; one latent per entry is key and value) and 一(五)4 (the FP4 cache is
// dequantized before attention, no FP4 matmul needed).
//
// A workgroup owns one query token, up to 64 heads (16 per wave) and a contiguous slice of its
// selected entries, walked in chunks of 32:
//   1. gather: the 32 selected 288-byte rows are copied to LDS, 18 lanes x 16 B per row;
//   2. dequantize in LDS: each (2 entries x 32 channels) item is decoded once into a bf16 copy
//      X[key][ch] (operand of q.x) and an f16 transposed copy Xt[ch][key] (operand of p.x). Both
//      are exact: every E2M1 x E4M3 product has at most 6 significant bits;
//   3. S^T = X Q^T on v_mfma_f32_16x16x32_bf16 (two 16-key tiles x 16 heads per wave): each lane
//      ends up with 8 keys of one head, which is exactly the B operand layout P^T needs next;
//   4. online softmax in fp32 (exp2 domain), per head, across the 4 lanes sharing a head;
//   5. O^T += Xt P^T on v_mfma_f32_16x16x32_f16, 32 channel tiles, fp32 accumulators.
// Decode rows (few query tokens) are split over the selected entries; a second kernel merges the
// per-split (max, sum, unnormalized output) triples.
#include <math.h>

#include <algorithm>

#include "common.h"
#include "launch.h"

namespace csa2 {

constexpr int kD = 512;                  // latent channels
constexpr int kRowB = 288;               // packed bytes per entry
constexpr int kKC = 32;                  // entries per chunk
constexpr int kXbPitch = kD + 8;         // bf16 elements per X row (pad against bank conflicts)
constexpr int kXtPitch = kKC + 4;        // f16 elements per Xt row
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Dequantize channels 32 cs .. 32 cs + 31 of staged entry `key`: fp32 values to v, and their bf16
// patterns (exact, so the top half of each fp32 pattern) to X[key][32 cs ..].
CSA2_DEV void decode_slab(const uint4* raw, int key, int cs, uint16_t* xb, float* v) {
  const uint8_t* rb = reinterpret_cast<const uint8_t*>(raw) + key * kRowB;
  const uint4 codes = *reinterpret_cast<const uint4*>(rb + 16 * cs);
  const uint32_t sc2 = *reinterpret_cast<const uint16_t*>(rb + 256 + 2 * cs);
  const float h0 = 0.5f * e4m3_value(sc2 & 0xFF), h1 = 0.5f * e4m3_value(sc2 >> 8);
  e2m1x8_to_f32(codes.x, h0, v);
  e2m1x8_to_f32(codes.y, h0, v + 8);
  e2m1x8_to_f32(codes.z, h1, v + 16);
  e2m1x8_to_f32(codes.w, h1, v + 24);
  uint4* dst = reinterpret_cast<uint4*>(xb + key * kXbPitch + 32 * cs);
#pragma unroll
  for (int qd = 0; qd < 4; ++qd) {
    uint32_t w[4];
#pragma unroll
    for (int h = 0; h < 4; ++h)
      w[h] = (__float_as_uint(v[8 * qd + 2 * h]) >> 16) | (__float_as_uint(v[8 * qd + 2 * h + 1]) & 0xFFFF0000u);
    dst[qd] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ rows, int n_max,
    const int32_t* __restrict__ idx, int T, int H, int K, int keys_per_split, float sm_scale,
    float* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  constexpr int NT = NW * 64;
  __shared__ uint4 raw[kKC * (kRowB / 16)];
  __shared__ __attribute__((aligned(16))) uint16_t xb[kKC * kXbPitch];
  __shared__ __attribute__((aligned(16))) uint16_t xt[kD * kXtPitch];
  __shared__ int kvalid[kKC];

  const int qr = blockIdx.x, split = blockIdx.y, hg = blockIdx.z;
  const int n_splits = gridDim.y;
  const int b = qr / T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int head = hg * (NW * 16) + wave * 16 + l16;   // this lane's head

  // Q^T operand: lane holds q[head][32 kk + 8 g .. +8] for kk = 0..15
  bf16x8_t qv[16];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(q + ((int64_t)qr * H + head) * kD);
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) qv[kk] = __builtin_bit_cast(bf16x8_t, qp[4 * kk + g]);
  }
  f32x4_t acc[32];
#pragma unroll
  for (int mt = 0; mt < 32; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;
  const float qscale = sm_scale * kLog2e;

  const int kbeg = split * keys_per_split;
  const int kend = min(K, kbeg + keys_per_split);
  const int32_t* irow = idx + (int64_t)qr * K;
  const uint8_t* rbase = rows + (int64_t)b * n_max * kRowB;

  for (int c0 = kbeg; c0 < kend; c0 += kKC) {
    // ---- 1. gather the chunk's rows into LDS ----
    if (tid < kKC) {
      const int kslot = c0 + tid;
      const int p = kslot < kend ? irow[kslot] : -1;
      kvalid[tid] = (p >= 0 && p < n_max) ? p : -1;
    }
    __syncthreads();
    for (int it = tid; it < kKC * 18; it += NT) {
      const int kr = it / 18, part = it - kr * 18;
      const int p = kvalid[kr];
      uint4 v = make_uint4(0, 0, 0, 0);
      if (p >= 0) v = *reinterpret_cast<const uint4*>(rbase + (int64_t)p * kRowB + 16 * part);
      raw[it] = v;
    }
    __syncthreads();
    // ---- 2. dequantize: item = (key pair kp, 32-channel slab cs) ----
    for (int it = tid; it < 16 * 16; it += NT) {
      const int kp = it & 15, cs = it >> 4;
      float v0[32], v1[32];
      decode_slab(raw, 2 * kp, cs, xb, v0);
      decode_slab(raw, 2 * kp + 1, cs, xb, v1);
      // f16 transposed copy: one 32-bit word (2 keys) per channel
#pragma unroll
      for (int c = 0; c < 32; ++c) {
        const _Float16 a = (_Float16)v0[c], bb = (_Float16)v1[c];
        const uint32_t w = (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, bb) << 16);
        *reinterpret_cast<uint32_t*>(xt + (32 * cs + c) * kXtPitch + 2 * kp) = w;
      }
    }
    __syncthreads();
    // ---- 3. S^T = X Q^T for this wave's 16 heads ----
    f32x4_t s[2];
#pragma unroll
    for (int tl = 0; tl < 2; ++tl) {
      s[tl] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const uint16_t* xr = xb + (16 * tl + l16) * kXbPitch + 8 * g;
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) {
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(xr + 32 * kk));
        s[tl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qv[kk], s[tl], 0, 0, 0);
      }
    }
    // ---- 4. online softmax; lane holds keys 16 tl + 4 g + i of head l16 ----
    float t[8];
    float cmax = -INFINITY;
#pragma unroll
    for (int tl = 0; tl < 2; ++tl)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 16 * tl + 4 * g + i;
        const float x = kvalid[key] >= 0 ? s[tl][i] * qscale : -INFINITY;
        t[4 * tl + i] = x;
        cmax = fmaxf(cmax, x);
      }
    cmax = fmaxf(cmax, shfl_xor_f(cmax, 16));
    cmax = fmaxf(cmax, shfl_xor_f(cmax, 32));
    const float m_new = fmaxf(m_run, cmax);
    float psum = 0.0f;
    f16x8_t pb;
    if (m_new == -INFINITY) {
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[i] = (_Float16)0.0f;
    } else {
      const float alpha = exp2f(m_run - m_new);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const _Float16 p = (_Float16)exp2f(t[i] - m_new);
        psum += (float)p;   // normalize by the weights the f16 MFMA actually uses
        pb[i] = p;
      }
      l_run *= alpha;
#pragma unroll
      for (int mt = 0; mt < 32; ++mt) acc[mt] *= alpha;
      m_run = m_new;
    }
    psum += shfl_xor_f(psum, 16);
    psum += shfl_xor_f(psum, 32);
    l_run += psum;
    // ---- 5. O^T += Xt P^T; A rows are channels, k slots are keys {4g..4g+3, 16+4g..16+4g+3} ----
#pragma unroll
    for (int mt = 0; mt < 32; ++mt) {
      const uint16_t* xr = xt + (16 * mt + l16) * kXtPitch + 4 * g;
      const uint2 lo = *reinterpret_cast<const uint2*>(xr);
      const uint2 hi = *reinterpret_cast<const uint2*>(xr + 16);
      const f16x8_t a = __builtin_bit_cast(f16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pb, acc[mt], 0, 0, 0);
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds O^T[16 mt + 4 g + i][head] ----
  const int64_t orow = (int64_t)qr * H + head;
  if (n_splits == 1) {
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    float4* op = reinterpret_cast<float4*>(out + orow * kD);
#pragma unroll
    for (int mt = 0; mt < 32; ++mt)
      op[4 * mt + g] = make_float4(acc[mt][0] * inv, acc[mt][1] * inv, acc[mt][2] * inv, acc[mt][3] * inv);
    if (lse && g == 0) lse[orow] = l_run > 0.0f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
  } else {
    const int64_t prow = (int64_t)split * gridDim.x * H + orow;
    float4* op = reinterpret_cast<float4*>(part_o + prow * kD);
#pragma unroll
    for (int mt = 0; mt < 32; ++mt) op[4 * mt + g] = make_float4(acc[mt][0], acc[mt][1], acc[mt][2], acc[mt][3]);
    if (g == 0) {
      part_ml[2 * prow] = m_run;
      part_ml[2 * prow + 1] = l_run;
    }
  }
}

// Merge of split results: one wave per (query row, head), lane owns 8 channels.
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml,
                                                           int n_splits, int64_t n_rows_h,
                                                           float* __restrict__ out,
                                                           float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int64_t rh = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (rh >= n_rows_h) return;
  float M = -INFINITY;
  for (int sp = 0; sp < n_splits; ++sp) M = fmaxf(M, part_ml[2 * (sp * n_rows_h + rh)]);
  float o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float L = 0.0f;
  if (M != -INFINITY) {
    for (int sp = 0; sp < n_splits; ++sp) {
      const int64_t pr = sp * n_rows_h + rh;
      const float m = part_ml[2 * pr];
      if (m == -INFINITY) continue;
      const float w = exp2f(m - M);
      L += w * part_ml[2 * pr + 1];
      const float4* pp = reinterpret_cast<const float4*>(part_o + pr * kD) + 2 * lane;
      const float4 a = pp[0], c = pp[1];
      o[0] += w * a.x; o[1] += w * a.y; o[2] += w * a.z; o[3] += w * a.w;
      o[4] += w * c.x; o[5] += w * c.y; o[6] += w * c.z; o[7] += w * c.w;
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  float4* op = reinterpret_cast<float4*>(out + rh * kD) + 2 * lane;
  op[0] = make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
  op[1] = make_float4(o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv);
  if (lse && lane == 0) lse[rh] = L > 0.0f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

static int attn_splits(int B, int T, int H, int K) {
  const int hpw = H >= 64 ? 64 : H;
  const int64_t wgs = (int64_t)B * T * (H / hpw);
  if (wgs >= 256 || K <= 2 * kKC) return 1;
  int splits = (int)std::min<int64_t>((K + 2 * kKC - 1) / (2 * kKC), std::max<int64_t>(1, 512 / wgs));
  return std::max(1, splits);
}

size_t attn_workspace(int B, int T, int H, int D, int K) {
  const int sp = attn_splits(B, T, H, K);
  if (sp == 1) return 0;
  const size_t rows_h = (size_t)B * T * H;
  return sp * rows_h * (size_t)D * 4 + sp * rows_h * 8 + 256;
}

hipError_t launch_sparse_attn(const uint16_t* q, const uint8_t* rows, int n_max, const int32_t* idx,
                              int B, int T, int H, int D, int K, float sm_scale, float* out,
                              float* lse, void* ws, hipStream_t s) {
  const int64_t nq = (int64_t)B * T;
  if (nq == 0 || H == 0) return hipSuccess;
  const int sp = attn_splits(B, T, H, K);
  int kps = (K + sp - 1) / sp;
  kps = std::max(kKC, (kps + kKC - 1) / kKC * kKC);
  const int n_splits = std::max(1, (K + kps - 1) / kps);
  const int hpw = H >= 64 ? 64 : H;
  float* part_o = nullptr;
  float* part_ml = nullptr;
  if (n_splits > 1) {
    part_o = static_cast<float*>(ws);
    part_ml = part_o + (size_t)n_splits * nq * H * kD;
  }
  dim3 grid((unsigned)nq, (unsigned)n_splits, (unsigned)(H / hpw));
  switch (hpw / 16) {
    case 1: hipLaunchKernelGGL(sparse_attn_kernel<1>, grid, dim3(64), 0, s, q, rows, n_max, idx, T, H, K, kps, sm_scale, out, lse, part_o, part_ml); break;
    case 2: hipLaunchKernelGGL(sparse_attn_kernel<2>, grid, dim3(128), 0, s, q, rows, n_max, idx, T, H, K, kps, sm_scale, out, lse, part_o, part_ml); break;
    case 3: hipLaunchKernelGGL(sparse_attn_kernel<3>, grid, dim3(192), 0, s, q, rows, n_max, idx, T, H, K, kps, sm_scale, out, lse, part_o, part_ml); break;
    default: hipLaunchKernelGGL(sparse_attn_kernel<4>, grid, dim3(256), 0, s, q, rows, n_max, idx, T, H, K, kps, sm_scale, out, lse, part_o, part_ml); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_splits == 1) return e;
  const int64_t rows_h = nq * H;
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)((rows_h + 3) / 4)), dim3(256), 0, s, part_o, part_ml,
                     n_splits, rows_h, out, lse);
  return hipGetLastError();
}

}  // namespace csa2
