// Sparse attention over the selected FP4 main-KV entries.
// Source: DeepSeek-V4.1-Flash walkthrough (wkq9411.github.io), 一(四) (each query attends to its
// selected main-KV entries; one latent per entry is key and value) and 一(五)4 (the FP4 cache is
// dequantized before attention, no FP4 matmul needed).
//
// A workgroup owns one query token, up to 64 heads (16 per wave) and a contiguous slice of its
// selected entries, walked in chunks of 32:
//   1. gather: the chunk's 288-byte rows are loaded into registers one chunk ahead (18 x 16 B
//      per row) and stored to LDS, so the loads of chunk c+1 overlap the math of chunk c;
//   2. dequantize in LDS with v_cvt_scalef32_pk_f16_fp4 (two E2M1 codes -> two f16, unscaled)
//      and one packed f16 multiply by the group's E4M3 scale: both exact, since every
//      E2M1 x E4M3 product has at most 6 significant bits and lies in f16's normal range. Each
//      entry is written once as X[key][ch] (operand of q.x) and once transposed as Xt[ch][key]
//      (operand of p.x);
//   3. S^T = X Q^T on v_mfma_f32_16x16x32_f16 (two 16-key tiles x 16 heads per wave). q is
//      scaled per head by a power of two so the bf16 query converts to f16 exactly; the scale is
//      folded into the softmax scale. Each lane ends up with 8 keys of one head, exactly the B
//      operand layout P^T needs next;
//   4. online softmax in fp32 (exp2 domain), per head, across the 4 lanes sharing a head
//      (v_permlane16/32_swap exchanges);
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
constexpr int kMaxKPS = 1024;            // entries per split (indices staged in LDS)
constexpr int kXPitch = kD + 8;          // f16 elements per X row (pad against bank conflicts)
constexpr int kXtPitch = kKC + 4;        // f16 elements per Xt row
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Values of the 4 lanes that share a head (lanes l, l^16, l^32, l^48) combined.
CSA2_DEV float head_max(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
CSA2_DEV float head_sum(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Eight E2M1 codes (one word) times an E4M3 scale as four packed f16 pairs (exact).
CSA2_DEV void e2m1x8_to_f16(uint32_t w, f16x2_t s2, uint32_t* out) {
  out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2);
  out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2);
  out[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2);
  out[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2);
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ rows, int n_max,
    const int32_t* __restrict__ idx, int T, int H, int K, int keys_per_split, float sm_scale,
    float* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  constexpr int NT = NW * 64;
  constexpr int GATHER = (kKC * 18 + NT - 1) / NT;     // 16-byte row pieces per thread per chunk
  __shared__ uint4 raw[kKC * (kRowB / 16)];
  __shared__ __attribute__((aligned(16))) uint16_t xs[kKC * kXPitch];
  __shared__ __attribute__((aligned(16))) uint16_t xt[kD * kXtPitch];
  __shared__ int sidx[kMaxKPS];

  const int qr = blockIdx.x, split = blockIdx.y, hg = blockIdx.z;
  const int n_splits = gridDim.y;
  const int b = qr / T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int head = hg * (NW * 16) + wave * 16 + l16;   // this lane's head

  const int kbeg = split * keys_per_split;
  const int kend = min(K, kbeg + keys_per_split);
  const int nk = max(0, kend - kbeg);
  const int32_t* irow = idx + (int64_t)qr * K + kbeg;
  const uint8_t* rbase = rows + (int64_t)b * n_max * kRowB;

  // stage this split's indices (out-of-range -> -1)
  for (int i = tid; i < nk; i += NT) {
    const int p = irow[i];
    sidx[i] = (p >= 0 && p < n_max) ? p : -1;
  }
  __syncthreads();

  // gather of one chunk into registers
  uint4 gr[GATHER];
  auto gather = [&](int c0) {
#pragma unroll
    for (int m = 0; m < GATHER; ++m) {
      const int it = tid + m * NT;
      gr[m] = make_uint4(0, 0, 0, 0);
      if (it < kKC * 18) {
        const int kr = it / 18, part = it - kr * 18;
        const int ks = c0 + kr;
        const int p = ks < nk ? sidx[ks] : -1;
        if (p >= 0) gr[m] = *reinterpret_cast<const uint4*>(rbase + (int64_t)p * kRowB + 16 * part);
      }
    }
  };
  if (nk > 0) gather(0);

  // Q^T operand in f16: lane holds q[head][32 kk + 8 g .. +8] * 2^qe for kk = 0..15
  f16x8_t qv[16];
  float qscale;
  {
    const uint4* qp = reinterpret_cast<const uint4*>(q + ((int64_t)qr * H + head) * kD);
    uint4 raw_q[16];
    float amax = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      raw_q[kk] = qp[4 * kk + g];
      const uint32_t w[4] = {raw_q[kk].x, raw_q[kk].y, raw_q[kk].z, raw_q[kk].w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(w[e] << 16)), fabsf(__uint_as_float(w[e] & 0xFFFF0000u))));
    }
    amax = head_max(amax);
    // power of two that brings the head's largest |q| into [2^14, 2^15): f16 holds every value
    const int qe = amax > 0.0f ? 14 - ilogbf(amax) : 0;
    const float sc = ldexpf(1.0f, qe);
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const uint32_t w[4] = {raw_q[kk].x, raw_q[kk].y, raw_q[kk].z, raw_q[kk].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qv[kk][2 * e] = (_Float16)(__uint_as_float(w[e] << 16) * sc);
        qv[kk][2 * e + 1] = (_Float16)(__uint_as_float(w[e] & 0xFFFF0000u) * sc);
      }
    }
    qscale = sm_scale * kLog2e * ldexpf(1.0f, -qe);
  }

  f32x4_t acc[32];
#pragma unroll
  for (int mt = 0; mt < 32; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;

  for (int c0 = 0; c0 < nk; c0 += kKC) {
    // ---- 1. gathered rows -> LDS; prefetch the next chunk ----
#pragma unroll
    for (int m = 0; m < GATHER; ++m) {
      const int it = tid + m * NT;
      if (it < kKC * 18) raw[it] = gr[m];
    }
    __syncthreads();
    if (c0 + kKC < nk) gather(c0 + kKC);
    // ---- 2. dequantize: item = (key pair kp, 32-channel slab cs) ----
    for (int it = tid; it < 16 * 16; it += NT) {
      const int kp = it & 15, cs = it >> 4;
      uint32_t va[16], vb[16];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int key = 2 * kp + e;
        const uint8_t* rb = reinterpret_cast<const uint8_t*>(raw) + key * kRowB;
        const uint4 codes = *reinterpret_cast<const uint4*>(rb + 16 * cs);
        const uint32_t sc2 = *reinterpret_cast<const uint16_t*>(rb + 256 + 2 * cs);
        const _Float16 s0 = (_Float16)e4m3_value(sc2 & 0xFF), s1 = (_Float16)e4m3_value(sc2 >> 8);
        uint32_t* v = e ? vb : va;
        e2m1x8_to_f16(codes.x, f16x2_t{s0, s0}, v);
        e2m1x8_to_f16(codes.y, f16x2_t{s0, s0}, v + 4);
        e2m1x8_to_f16(codes.z, f16x2_t{s1, s1}, v + 8);
        e2m1x8_to_f16(codes.w, f16x2_t{s1, s1}, v + 12);
        uint4* dst = reinterpret_cast<uint4*>(xs + key * kXPitch + 32 * cs);
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) dst[qd] = make_uint4(v[4 * qd], v[4 * qd + 1], v[4 * qd + 2], v[4 * qd + 3]);
      }
      // transposed copy: one word = (key 2kp, key 2kp+1) for each channel
      uint32_t* xtp = reinterpret_cast<uint32_t*>(xt + (32 * cs) * kXtPitch + 2 * kp);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        xtp[(2 * i) * (kXtPitch / 2)] = __builtin_amdgcn_perm(vb[i], va[i], 0x05040100u);
        xtp[(2 * i + 1) * (kXtPitch / 2)] = __builtin_amdgcn_perm(vb[i], va[i], 0x07060302u);
      }
    }
    __syncthreads();
    // ---- 3. S^T = X Q^T for this wave's 16 heads ----
    f32x4_t sacc[2];
#pragma unroll
    for (int tl = 0; tl < 2; ++tl) {
      sacc[tl] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const uint16_t* xr = xs + (16 * tl + l16) * kXPitch + 8 * g;
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) {
        const f16x8_t a = __builtin_bit_cast(f16x8_t, *reinterpret_cast<const uint4*>(xr + 32 * kk));
        sacc[tl] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qv[kk], sacc[tl], 0, 0, 0);
      }
    }
    // ---- 4. online softmax; lane holds keys c0 + 16 tl + 4 g + i of head l16 ----
    float t[8];
    float cmax = -INFINITY;
#pragma unroll
    for (int tl = 0; tl < 2; ++tl)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ks = c0 + 16 * tl + 4 * g + i;
        const float x = (ks < nk && sidx[ks] >= 0) ? sacc[tl][i] * qscale : -INFINITY;
        t[4 * tl + i] = x;
        cmax = fmaxf(cmax, x);
      }
    cmax = head_max(cmax);
    const float m_new = fmaxf(m_run, cmax);
    float psum = 0.0f;
    f16x8_t pb;
    if (m_new == -INFINITY) {
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[i] = (_Float16)0.0f;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const _Float16 p = (_Float16)exp2f(t[i] - m_new);
        psum += (float)p;   // normalize by the weights the f16 MFMA actually uses
        pb[i] = p;
      }
      if (m_new != m_run) {
        const float alpha = exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int mt = 0; mt < 32; ++mt) acc[mt] *= alpha;
        m_run = m_new;
      }
    }
    l_run += head_sum(psum);
    // ---- 5. O^T += Xt P^T; A rows are channels, k slots are keys {4g..4g+3, 16+4g..16+4g+3} ----
#pragma unroll
    for (int mt = 0; mt < 32; ++mt) {
      const uint16_t* xr = xt + (16 * mt + l16) * kXtPitch + 4 * g;
      const uint2 lo = *reinterpret_cast<const uint2*>(xr);
      const uint2 hi = *reinterpret_cast<const uint2*>(xr + 16);
      const f16x8_t a = __builtin_bit_cast(f16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pb, acc[mt], 0, 0, 0);
    }
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

// ---------------------------------------------------------------------------------------------
// Decode form: few query rows. A workgroup owns (query row, 16-head group, slice of entries). Its
// NG sub-groups of 4 waves each take an equal part of the slice and walk it in chunks of KC
// entries, in lockstep (shared barriers, separate LDS buffers), so each SIMD runs NG waves that
// hide each other's latencies. Wave w of a sub-group owns channels 128w .. 128w+127 throughout:
//   - it gathers only the bytes of its channels (a lane: one entry's 64-channel slab, 32 code
//     bytes and 4 scale bytes, straight into registers) and dequantizes them into its own slab
//     of X[entry][channel] (f16, exact), which only it reads, so no barrier guards X;
//   - scores: each wave computes partial S^T = X Q^T over its own 128 channels for all KC
//     entries x 16 heads (16x16x32 f16 MFMA) and writes them to a small LDS tile (two, used in
//     turn); after the chunk's one barrier every wave adds the 4 partials, so the sub-group's
//     waves hold the same scores;
//   - every wave runs the same online softmax (identical inputs and arithmetic, so the running
//     (max, sum) agree across the sub-group), then O^T += X^T P^T for its 128 channels over the
//     chunk (16x16x32 f16 MFMA, the chunk's two 16-entry halves as one operand). The A operand
//     (8 entries of one channel per lane) comes straight from X through two transposing LDS
//     reads ds_read_b64_tr_b16; the B operand (the same 8 entries of one head per lane) is the
//     lane's own softmax output.
// At the end the sub-groups' (max, sum, output) states merge in LDS, so a query row needs no
// second kernel unless its entries are also split over workgroups. The gathers of the next PF
// chunks are in flight while a chunk is processed (the query is loaded first, so it does not
// queue behind them). Workgroups are placed so that all of a query row's run on one XCD and
// share its L2. The softmax reference max is only moved when a new score exceeds it by more
// than 2^8, so probabilities stay <= 256 (exact enough in f16) and the accumulators are rescaled
// rarely.
constexpr float kLazyRescale = 8.0f;            // log2 headroom before the reference max moves
constexpr int kDKC = 32;                        // decode entries per chunk
constexpr int kDPF = 2;                         // decode chunks gathered ahead
constexpr int kDNG = 2;                         // decode sub-groups per workgroup
constexpr int kDecodeFill = 256;                // decode workgroups wanted: one per CU

template <int KC, int NG>
struct DecodeSmem {
  static constexpr int kX = KC * kXPitch * 2;
  static constexpr int kS = 4 * KC * 16 * 4;    // the 4 waves' partial scores, KC entries x 16 heads
  static constexpr int kGroup = kX + 2 * kS;    // one sub-group's buffers (two score tiles)
  static constexpr int kOut = 4 * 8 * 64 * 16;  // one sub-group's output tiles at the merge
  static_assert(NG * kGroup >= (NG - 1) * kOut, "the merge reuses the sub-groups' buffers");
  static constexpr int kIdx = kMaxKPS * 4;
  static constexpr int kMl = (NG > 2 ? NG : 2) * 16 * 2 * 4;  // query amax, then per-group (max, sum)
  static constexpr int kQ = 16 * kXPitch * 2;   // the 16 heads' scaled f16 queries
  static constexpr int kTotal = NG * kGroup + kIdx + kMl + kQ;
};

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// The two 16-entry halves of a chunk as one K = 32 operand of v_mfma_f32_16x16x32_f16: lane
// group g (lane / 16) holds entries 4 g .. 4 g + 3 of the first half and then of the second half,
// in the A operand (transposed X, from two ds_read_b64_tr_b16) and in the B operand (P) alike, so
// the MFMA's k index pairs the same entries on both sides. One K = 32 MFMA does the work of two
// K = 16 ones at the doubled rate gfx950 gives the K = 32 form.
CSA2_DEV f16x8_t cat_halves(f16x4_t lo, f16x4_t hi) { return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7); }
CSA2_DEV f16x8_t xt_chunk(const uint16_t* p, int pitch) {
  const s16x4_t a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
  const s16x4_t a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p + 16 * pitch));
  return cat_halves(__builtin_bit_cast(f16x4_t, a0), __builtin_bit_cast(f16x4_t, a1));
}

// Two E4M3 scale bytes (low half of w) as f16 (exact: E4M3 values fit f16).
CSA2_DEV f16x2_t e4m3x2_to_f16(uint32_t w) { return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false); }

template <int KC, int PF, int NG>
__global__ __launch_bounds__(256 * NG) void sparse_attn_decode_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ rows, int n_max,
    const int32_t* __restrict__ idx, int T, int H, int K, int keys_per_split, float sm_scale,
    float* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float* __restrict__ part_ml, int n_rows, int n_splits, int final_out, int per_xcd) {
  using Sm = DecodeSmem<KC, NG>;
  constexpr int NT = 256 * NG, NS = KC / 16;    // NS entry steps of 16 per chunk
  static_assert(KC == 32, "a wave's 64 lanes gather the chunk's 32 entries x 2 slabs of 64 channels");
  static_assert(NG >= 1 && NG <= 4, "sub-groups");
  __shared__ __attribute__((aligned(16))) unsigned char smem[Sm::kTotal];
  int* sidx = reinterpret_cast<int*>(smem + NG * Sm::kGroup);
  float* ml = reinterpret_cast<float*>(smem + NG * Sm::kGroup + Sm::kIdx);
  uint16_t* qs = reinterpret_cast<uint16_t*>(smem + NG * Sm::kGroup + Sm::kIdx + Sm::kMl);

  // Workgroup i runs on XCD i mod 8; each XCD takes a contiguous range of work items ordered
  // (query row, split, head group), so all workgroups of a query row share one L2: the rows they
  // gather and the query they load are fetched from HBM about once.
  const int n_hg = H / 16;
  const int u = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (u >= n_rows * n_splits * n_hg) return;
  const int qr = u / (n_splits * n_hg), split = (u / n_hg) % n_splits, hg = u % n_hg;
  const int b = qr / T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sg = wave >> 2, w4 = wave & 3;   // sub-group and wave within it
  const int l16 = lane & 15, g = lane >> 4;
  const int head = hg * 16 + l16;

  unsigned char* gbase = smem + sg * Sm::kGroup;
  uint16_t* xs = reinterpret_cast<uint16_t*>(gbase);
  float4* sp4b = reinterpret_cast<float4*>(gbase + Sm::kX);

  const int kbeg = split * keys_per_split;
  const int nk = max(0, min(K, kbeg + keys_per_split) - kbeg);        // entries of this workgroup
  const int sub_len = ((nk + NG - 1) / NG + KC - 1) / KC * KC;          // entries per sub-group
  const int sbeg = sg * sub_len;
  const int snk = max(0, min(nk - sbeg, sub_len));                     // entries of this sub-group
  const int32_t* irow = idx + (int64_t)qr * K + kbeg;
  const uint8_t* rbase = rows + (int64_t)b * n_max * kRowB;

  // Lane: entry gkey of a chunk, channel slab gcs (64 channels) of this wave's 128. The
  // positions of its entries in the first PF chunks are loaded first, so that those gathers can
  // start without waiting for the LDS copy of the positions.
  const int gkey = lane & 31, gcs = 2 * w4 + (lane >> 5);
  int pos0[PF];
#pragma unroll
  for (int v = 0; v < PF; ++v) {
    const int ks = v * KC + gkey;
    pos0[v] = ks < snk ? irow[sbeg + ks] : -1;
  }
  // sub-group 0 loads the 16 heads' queries, wave w4 its channel blocks 4 w4 .. 4 w4 + 3
  uint4 raw_q[4];
  if (sg == 0) {
    const uint4* qp = reinterpret_cast<const uint4*>(q + ((int64_t)qr * H + head) * kD);
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) raw_q[kq] = qp[4 * (4 * w4 + kq) + g];
  }
  // the slice's entry positions: read from global once (issued together with the query loads),
  // staged in LDS for every gather
  constexpr int IPT = (kMaxKPS + NT - 1) / NT;
  int ipos[IPT];
#pragma unroll
  for (int m = 0; m < IPT; ++m) {
    const int i = tid + m * NT;
    ipos[m] = i < nk ? irow[i] : -1;
  }
  // gathers run PF chunks ahead: registers gr[v] hold chunk c0 + v KC of the current group
  struct Piece {
    uint4 c01, c23;     // the slab's 64 E2M1 codes
    uint32_t sc;        // its 4 E4M3 scales
  };
  Piece gr[PF];
  auto gather_at = [&](Piece& d, int p) {   // p: position, or anything outside [0, n_max)
    d.c01 = d.c23 = make_uint4(0, 0, 0, 0);
    d.sc = 0u;
    if (p >= 0 && p < n_max) {
      const uint8_t* rp = rbase + (int64_t)p * kRowB;
      d.c01 = *reinterpret_cast<const uint4*>(rp + 32 * gcs);
      d.c23 = *reinterpret_cast<const uint4*>(rp + 32 * gcs + 16);
      d.sc = *reinterpret_cast<const uint32_t*>(rp + 256 + 4 * gcs);
    }
  };
  auto gather = [&](Piece& d, int c0) {
    const int ks = c0 + gkey;
    gather_at(d, ks < snk ? sidx[sbeg + ks] : -1);
  };
#pragma unroll
  for (int v = 0; v < PF; ++v) gather_at(gr[v], pos0[v]);
#pragma unroll
  for (int m = 0; m < IPT; ++m) {
    const int i = tid + m * NT;
    if (i < nk) sidx[i] = (ipos[m] >= 0 && ipos[m] < n_max) ? ipos[m] : -1;
  }
  if (sg == 0) {
    float amax = 0.0f;
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
      const uint32_t w[4] = {raw_q[kq].x, raw_q[kq].y, raw_q[kq].z, raw_q[kq].w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(w[e] << 16)), fabsf(__uint_as_float(w[e] & 0xFFFF0000u))));
    }
    amax = head_max(amax);
    if (g == 0) ml[w4 * 16 + l16] = amax;
  }
  __syncthreads();
  // the queries, scaled per head by a power of two and converted to f16 (exact), into LDS
  float qscale;
  {
    const float amax = fmaxf(fmaxf(ml[l16], ml[16 + l16]), fmaxf(ml[32 + l16], ml[48 + l16]));
    const int qe = amax > 0.0f ? 14 - ilogbf(amax) : 0;
    if (sg == 0) {
      const float sc = ldexpf(1.0f, qe);
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) {
        const int kk = 4 * w4 + kq;
        const uint32_t w[4] = {raw_q[kq].x, raw_q[kq].y, raw_q[kq].z, raw_q[kq].w};
        f16x8_t h;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          h[2 * e] = (_Float16)(__uint_as_float(w[e] << 16) * sc);
          h[2 * e + 1] = (_Float16)(__uint_as_float(w[e] & 0xFFFF0000u) * sc);
        }
        *reinterpret_cast<f16x8_t*>(qs + l16 * kXPitch + 32 * kk + 8 * g) = h;
      }
    }
    qscale = sm_scale * kLog2e * ldexpf(1.0f, -qe);
  }
  __syncthreads();                                 // the scaled queries are in LDS
  f16x8_t qb[4];                                   // this wave's query fragments, kept in registers
  {
    const uint16_t* qr16 = qs + l16 * kXPitch + 128 * w4 + 8 * g;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qb[kk] = *reinterpret_cast<const f16x8_t*>(qr16 + 32 * kk);
  }

  // output tiles of this wave: channels 128 w4 + 16 j + (4 g + i), head l16
  f32x4_t acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;
  // transposing-read base for the P.V operand: entry 4 g + l16/4 (+16 s), channel 128 w4 + 4 (l16%4) (+16 j)
  const uint16_t* xtr = xs + (4 * g + (l16 >> 2)) * kXPitch + 128 * w4 + 4 * (l16 & 3);
  // partial-score tile layout: [wave][entry / 4][head][entry % 4] (a lane's 4 entries are one float4)

  // every sub-group runs the same number of chunk steps (barriers are shared); steps past its
  // entries do no work
  for (int cg = 0; cg < sub_len; cg += PF * KC)
#pragma unroll
  for (int v = 0; v < PF; ++v) {
    const int c0 = cg + v * KC;
    if (c0 >= sub_len) break;
    const bool active = c0 < snk;
    float4* sp4 = sp4b + ((c0 / KC) & 1) * (4 * (KC / 4) * 16);
    if (active) {
      // dequantize this lane's slab into X; the X slab of wave w4 is read by wave w4 only, and a
      // wave's LDS operations complete in order, so the reads below see these writes
      const Piece& pc = gr[v];
      const f16x2_t s01 = e4m3x2_to_f16(pc.sc), s23 = e4m3x2_to_f16(pc.sc >> 16);
      const f16x2_t sgm[4] = {f16x2_t{s01[0], s01[0]}, f16x2_t{s01[1], s01[1]}, f16x2_t{s23[0], s23[0]},
                              f16x2_t{s23[1], s23[1]}};
      const uint32_t cw[8] = {pc.c01.x, pc.c01.y, pc.c01.z, pc.c01.w, pc.c23.x, pc.c23.y, pc.c23.z, pc.c23.w};
      uint4* dst = reinterpret_cast<uint4*>(xs + gkey * kXPitch + 64 * gcs);
#pragma unroll
      for (int wi = 0; wi < 8; ++wi) {
        uint32_t vv[4];
        e2m1x8_to_f16(cw[wi], sgm[wi >> 1], vv);
        dst[wi] = make_uint4(vv[0], vv[1], vv[2], vv[3]);
      }
      if (c0 + PF * KC < snk) gather(gr[v], c0 + PF * KC);
      __builtin_amdgcn_wave_barrier();
      // partial S^T over this wave's channels: entry tile t, lane holds entries 16 t + 4 g + i of head l16
      const uint16_t* xr = xs + l16 * kXPitch + 128 * w4 + 8 * g;
      float4* my_sp = sp4 + w4 * (KC / 4) * 16;
#pragma unroll
      for (int t = 0; t < NS; ++t) {
        f32x4_t s0 = f32x4_t{0.f, 0.f, 0.f, 0.f}, s1 = s0;  // two chains halve the dependency latency
#pragma unroll
        for (int kk = 0; kk < 4; kk += 2) {
          const f16x8_t a0 = *reinterpret_cast<const f16x8_t*>(xr + 16 * t * kXPitch + 32 * kk);
          const f16x8_t a1 = *reinterpret_cast<const f16x8_t*>(xr + 16 * t * kXPitch + 32 * kk + 32);
          s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, qb[kk], s0, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, qb[kk + 1], s1, 0, 0, 0);
        }
        const f32x4_t sv = s0 + s1;
        my_sp[(4 * t + g) * 16 + l16] = make_float4(sv[0], sv[1], sv[2], sv[3]);
      }
    }
    __syncthreads();
    if (!active) continue;
    // complete scores and online softmax over the chunk: lane holds entries 16 s + 4 g + i of head l16
    uint64_t vmask;                  // bit e: entry c0 + e of the sub-group is a real entry
    {
      int pe = -1;
      if (lane < KC && c0 + lane < snk) pe = sidx[sbeg + c0 + lane];
      vmask = __ballot(pe >= 0);
    }
    float tv[NS][4];
    float cmax = -INFINITY;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      float4 a = sp4[(4 * s + g) * 16 + l16];
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        const float4 x = sp4[w * (KC / 4) * 16 + (4 * s + g) * 16 + l16];
        a.x += x.x; a.y += x.y; a.z += x.z; a.w += x.w;
      }
      const float sv[4] = {a.x, a.y, a.z, a.w};
      const uint32_t vb = (uint32_t)(vmask >> (16 * s + 4 * g)) & 15u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        tv[s][i] = ((vb >> i) & 1u) ? sv[i] * qscale : -INFINITY;
        cmax = fmaxf(cmax, tv[s][i]);
      }
    }
    cmax = head_max(cmax);
    if (m_run == -INFINITY) {
      m_run = cmax;                 // first entries of this head: nothing accumulated yet
    } else if (__builtin_expect(__ballot(cmax > m_run + kLazyRescale) != 0, 0)) {
      const float mn = fmaxf(m_run, cmax);
      const float alpha = exp2f(m_run - mn);
      l_run *= alpha;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] *= alpha;
      m_run = mn;
    }
    float psum = 0.0f;
    f16x4_t pb[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const _Float16 pv = m_run == -INFINITY ? (_Float16)0.0f : (_Float16)exp2f(tv[s][i] - m_run);
        psum += (float)pv;
        pb[s][i] = pv;
      }
    l_run += head_sum(psum);
    // O^T += X^T P^T: this wave's 8 channel tiles over the chunk's 32 entries, one K = 32 MFMA each
    static_assert(NS == 2, "a chunk is two 16-entry halves");
    {
      const f16x8_t p8 = cat_halves(pb[0], pb[1]);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xt_chunk(xtr + 16 * j, kXPitch), p8, acc[j], 0, 0, 0);
    }
  }

  // merge the sub-groups: groups 1.. leave (max, sum) and their tiles in LDS, group 0 combines
  float M = m_run, L = l_run;
  if (NG > 1) {
    __syncthreads();                               // every group is done with its buffers
    if (sg > 0) {
      float4* ob = reinterpret_cast<float4*>(smem + (sg - 1) * Sm::kOut);  // [w4][j][lane]
#pragma unroll
      for (int j = 0; j < 8; ++j) ob[(w4 * 8 + j) * 64 + lane] = make_float4(acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
      if (w4 == 0 && g == 0) {
        ml[(sg * 16 + l16) * 2] = m_run;
        ml[(sg * 16 + l16) * 2 + 1] = l_run;
      }
    }
    __syncthreads();
    if (sg > 0) return;
#pragma unroll
    for (int k = 1; k < NG; ++k) M = fmaxf(M, ml[(k * 16 + l16) * 2]);
    const float f0 = m_run == -INFINITY ? 0.0f : exp2f(m_run - M);
    L = l_run * f0;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= f0;
#pragma unroll
    for (int k = 1; k < NG; ++k) {
      const float mk = ml[(k * 16 + l16) * 2];
      const float fk = mk == -INFINITY ? 0.0f : exp2f(mk - M);
      L += ml[(k * 16 + l16) * 2 + 1] * fk;
      const float4* obk = reinterpret_cast<const float4*>(smem + (k - 1) * Sm::kOut);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float4 o = obk[(w4 * 8 + j) * 64 + lane];
        acc[j] += f32x4_t{o.x, o.y, o.z, o.w} * fk;
      }
    }
  }

  // every wave holds the same (M, L) and disjoint channels: write directly (final_out: the only
  // split, normalized; else an unnormalized partial of split `split` for the combine pass)
  // The 16 heads' rows leave through LDS past the merge tiles: a lane holds 16 bytes of one head
  // per store in the accumulator layout, staged each store writes two heads' 512 contiguous bytes
  const int64_t orow = (int64_t)qr * H + head;
  const float scale = final_out ? (L > 0.0f ? 1.0f / L : 0.0f) : 1.0f;
  {
    constexpr int kStRow = 132;
    static_assert((NG - 1) * Sm::kOut + 4 * 16 * kStRow * 4 <= NG * Sm::kGroup, "the output stage fits");
    if constexpr (NG == 1) __syncthreads();   // the stage overlaps the other waves' X slabs
    float* stage = reinterpret_cast<float*>(smem + (NG - 1) * Sm::kOut) + w4 * 16 * kStRow;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<f32x4_t*>(stage + l16 * kStRow + 16 * j + 4 * g) = acc[j] * scale;
    __builtin_amdgcn_wave_barrier();
    const int64_t row0 = (int64_t)qr * H + hg * 16;
    float* dst = (final_out ? out + row0 * kD : part_o + ((int64_t)split * n_rows * H + row0) * kD) +
                 (lane >> 5) * kD + 128 * w4 + 4 * (lane & 31);
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2)
      *reinterpret_cast<float4*>(dst + 2 * s2 * kD) =
          *reinterpret_cast<const float4*>(stage + (2 * s2 + (lane >> 5)) * kStRow + 4 * (lane & 31));
  }
  if (w4 == 0 && g == 0) {
    if (final_out) {
      if (lse) lse[orow] = L > 0.0f ? (M + log2f(L)) * kLn2 : -INFINITY;
    } else {
      const int64_t prow = (int64_t)split * n_rows * H + orow;
      part_ml[2 * prow] = M;
      part_ml[2 * prow + 1] = L;
    }
  }
}

// Sliding-window branch for decode (one query token per sequence): the layer's own window of
// FP8 rows ([walkthrough] 一(四): each query also attends to its own layer's sliding-window KV;
// 一(五)4: that KV stays in FP8). Same structure as the decode form above, over window rows
// wsplit * rows_per_split .. of sequence b (rows 0 .. n_win[b]-1 are valid), written as
// unnormalized partials into slots slot0 + wsplit of the decode form's split buffers, so that the
// combine pass makes one softmax of the selected entries and the window.
template <int KC, int PF, int NG>
__global__ __launch_bounds__(256 * NG) void swa_attn_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ swa_codes, const int8_t* __restrict__ swa_exp,
    const int32_t* __restrict__ n_win, int T, int prefill, int W, int H, int rows_per_split, float sm_scale,
    float* __restrict__ part_o, float* __restrict__ part_ml, int slot0, int n_rows, int n_wsplits, int per_xcd) {
  using Sm = DecodeSmem<KC, NG>;
  constexpr int NS = KC / 16;                  // NS entry steps of 16 per chunk
  static_assert(KC == 32, "a wave's 64 lanes gather the chunk's 32 entries x 2 slabs of 64 channels");
  static_assert(NG >= 1 && NG <= 4, "sub-groups");
  __shared__ __attribute__((aligned(16))) unsigned char smem[Sm::kTotal];
  float* ml = reinterpret_cast<float*>(smem + NG * Sm::kGroup + Sm::kIdx);
  uint16_t* qs = reinterpret_cast<uint16_t*>(smem + NG * Sm::kGroup + Sm::kIdx + Sm::kMl);

  // Workgroup i runs on XCD i mod 8; each XCD takes a contiguous range of work items ordered
  // (query row, split, head group), so all workgroups of a query row share one L2: the rows they
  // gather and the query they load are fetched from HBM about once.
  const int n_hg = H / 16;
  const int u = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (u >= n_rows * n_wsplits * n_hg) return;
  const int qr = u / (n_wsplits * n_hg), wsplit = (u / n_hg) % n_wsplits, hg = u % n_hg;
  const int b = qr / T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sg = wave >> 2, w4 = wave & 3;   // sub-group and wave within it
  const int l16 = lane & 15, g = lane >> 4;
  const int head = hg * 16 + l16;

  unsigned char* gbase = smem + sg * Sm::kGroup;
  uint16_t* xs = reinterpret_cast<uint16_t*>(gbase);
  float4* sp4b = reinterpret_cast<float4*>(gbase + Sm::kX);

  // decode layout (prefill == 0, T == 1): rows 0 .. n-1 of the sequence's W-row window,
  // n = n_win[b]; prefill layout (any T, including 1): the sequence's buffer holds T + W - 1 rows
  // and query t takes rows t + W - n .. t + W - 1, n = n_win[query row] (its last n tokens up to
  // its own)
  const int n_valid = max(0, min(n_win[prefill ? qr : b], W));        // window rows of this query
  const int64_t row0 = prefill ? (int64_t)b * (T + W - 1) + (qr - b * T) + (W - n_valid) : (int64_t)b * W;
  const int kbeg = wsplit * rows_per_split;
  const int nk = max(0, min(n_valid, kbeg + rows_per_split) - kbeg);  // rows of this workgroup
  const int sub_len = ((nk + NG - 1) / NG + KC - 1) / KC * KC;          // entries per sub-group
  const int sbeg = kbeg + sg * sub_len;                                 // first window row of the sub-group
  const int snk = max(0, min(nk - sg * sub_len, sub_len));             // entries of this sub-group
  const uint8_t* wbase = swa_codes + row0 * kD;                     // this query's window rows
  const int8_t* ebase = swa_exp + row0;                              // their exponents

  // Lane: entry gkey of a chunk, channel slab gcs (64 channels) of this wave's 128. The
  // positions of its entries in the first PF chunks are loaded first, so that those gathers can
  // start without waiting for the LDS copy of the positions.
  const int gkey = lane & 31, gcs = 2 * w4 + (lane >> 5);
  int pos0[PF];
#pragma unroll
  for (int v = 0; v < PF; ++v) {
    const int ks = v * KC + gkey;
    pos0[v] = ks < snk ? sbeg + ks : -1;
  }
  // sub-group 0 loads the 16 heads' queries, wave w4 its channel blocks 4 w4 .. 4 w4 + 3
  uint4 raw_q[4];
  if (sg == 0) {
    const uint4* qp = reinterpret_cast<const uint4*>(q + ((int64_t)qr * H + head) * kD);
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) raw_q[kq] = qp[4 * (4 * w4 + kq) + g];
  }

  // gathers run PF chunks ahead: registers gr[v] hold chunk c0 + v KC of the current group
  struct Piece {
    uint4 c[4];         // the slab's 64 E4M3 codes
    int e;              // the row's exponent
  };
  Piece gr[PF];
  auto gather_at = [&](Piece& d, int p) {   // p: window row, or -1
#pragma unroll
    for (int m = 0; m < 4; ++m) d.c[m] = make_uint4(0, 0, 0, 0);
    d.e = 0;
    if (p >= 0 && p < n_valid) {
      const uint4* rp = reinterpret_cast<const uint4*>(wbase + (int64_t)p * kD + 64 * gcs);
#pragma unroll
      for (int m = 0; m < 4; ++m) d.c[m] = rp[m];
      d.e = ebase[p];
    }
  };
  auto gather = [&](Piece& d, int c0) {
    const int ks = c0 + gkey;
    gather_at(d, ks < snk ? sbeg + ks : -1);
  };
#pragma unroll
  for (int v = 0; v < PF; ++v) gather_at(gr[v], pos0[v]);

  if (sg == 0) {
    float amax = 0.0f;
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
      const uint32_t w[4] = {raw_q[kq].x, raw_q[kq].y, raw_q[kq].z, raw_q[kq].w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(w[e] << 16)), fabsf(__uint_as_float(w[e] & 0xFFFF0000u))));
    }
    amax = head_max(amax);
    if (g == 0) ml[w4 * 16 + l16] = amax;
  }
  __syncthreads();
  // the queries, scaled per head by a power of two and converted to f16 (exact), into LDS
  float qscale;
  {
    const float amax = fmaxf(fmaxf(ml[l16], ml[16 + l16]), fmaxf(ml[32 + l16], ml[48 + l16]));
    const int qe = amax > 0.0f ? 14 - ilogbf(amax) : 0;
    if (sg == 0) {
      const float sc = ldexpf(1.0f, qe);
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) {
        const int kk = 4 * w4 + kq;
        const uint32_t w[4] = {raw_q[kq].x, raw_q[kq].y, raw_q[kq].z, raw_q[kq].w};
        f16x8_t h;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          h[2 * e] = (_Float16)(__uint_as_float(w[e] << 16) * sc);
          h[2 * e + 1] = (_Float16)(__uint_as_float(w[e] & 0xFFFF0000u) * sc);
        }
        *reinterpret_cast<f16x8_t*>(qs + l16 * kXPitch + 32 * kk + 8 * g) = h;
      }
    }
    qscale = sm_scale * kLog2e * ldexpf(1.0f, -qe);
  }
  __syncthreads();                                 // the scaled queries are in LDS
  f16x8_t qb[4];                                   // this wave's query fragments, kept in registers
  {
    const uint16_t* qr16 = qs + l16 * kXPitch + 128 * w4 + 8 * g;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qb[kk] = *reinterpret_cast<const f16x8_t*>(qr16 + 32 * kk);
  }

  // output tiles of this wave: channels 128 w4 + 16 j + (4 g + i), head l16
  f32x4_t acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;
  // transposing-read base for the P.V operand: entry 4 g + l16/4 (+16 s), channel 128 w4 + 4 (l16%4) (+16 j)
  const uint16_t* xtr = xs + (4 * g + (l16 >> 2)) * kXPitch + 128 * w4 + 4 * (l16 & 3);
  // partial-score tile layout: [wave][entry / 4][head][entry % 4] (a lane's 4 entries are one float4)

  // every sub-group runs the same number of chunk steps (barriers are shared); steps past its
  // entries do no work
  for (int cg = 0; cg < sub_len; cg += PF * KC)
#pragma unroll
  for (int v = 0; v < PF; ++v) {
    const int c0 = cg + v * KC;
    if (c0 >= sub_len) break;
    const bool active = c0 < snk;
    float4* sp4 = sp4b + ((c0 / KC) & 1) * (4 * (KC / 4) * 16);
    if (active) {
      // dequantize this lane's slab into X; the X slab of wave w4 is read by wave w4 only, and a
      // wave's LDS operations complete in order, so the reads below see these writes
      // E4M3 -> f16 is exact, and so is the product with the row's power of two for exponents
      // in [-15, 7] (the results stay within f16's range and precision)
      const Piece& pc = gr[v];
      const _Float16 sc = (_Float16)ldexpf(1.0f, pc.e);
      const f16x2_t s2 = f16x2_t{sc, sc};
      uint4* dst = reinterpret_cast<uint4*>(xs + gkey * kXPitch + 64 * gcs);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t cw[4] = {pc.c[m].x, pc.c[m].y, pc.c[m].z, pc.c[m].w};
        uint32_t vv[8];
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
          vv[2 * t4] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cw[t4], 1.0f, false) * s2);
          vv[2 * t4 + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cw[t4] >> 16, 1.0f, false) * s2);
        }
        dst[2 * m] = make_uint4(vv[0], vv[1], vv[2], vv[3]);
        dst[2 * m + 1] = make_uint4(vv[4], vv[5], vv[6], vv[7]);
      }
      if (c0 + PF * KC < snk) gather(gr[v], c0 + PF * KC);
      __builtin_amdgcn_wave_barrier();
      // partial S^T over this wave's channels: entry tile t, lane holds entries 16 t + 4 g + i of head l16
      const uint16_t* xr = xs + l16 * kXPitch + 128 * w4 + 8 * g;
      float4* my_sp = sp4 + w4 * (KC / 4) * 16;
#pragma unroll
      for (int t = 0; t < NS; ++t) {
        f32x4_t s0 = f32x4_t{0.f, 0.f, 0.f, 0.f}, s1 = s0;  // two chains halve the dependency latency
#pragma unroll
        for (int kk = 0; kk < 4; kk += 2) {
          const f16x8_t a0 = *reinterpret_cast<const f16x8_t*>(xr + 16 * t * kXPitch + 32 * kk);
          const f16x8_t a1 = *reinterpret_cast<const f16x8_t*>(xr + 16 * t * kXPitch + 32 * kk + 32);
          s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, qb[kk], s0, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, qb[kk + 1], s1, 0, 0, 0);
        }
        const f32x4_t sv = s0 + s1;
        my_sp[(4 * t + g) * 16 + l16] = make_float4(sv[0], sv[1], sv[2], sv[3]);
      }
    }
    __syncthreads();
    if (!active) continue;
    // complete scores and online softmax over the chunk: lane holds entries 16 s + 4 g + i of head l16
    uint64_t vmask;                  // bit e: entry c0 + e of the sub-group is a real entry
    {
      vmask = __ballot(lane < KC && c0 + lane < snk);
    }
    float tv[NS][4];
    float cmax = -INFINITY;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      float4 a = sp4[(4 * s + g) * 16 + l16];
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        const float4 x = sp4[w * (KC / 4) * 16 + (4 * s + g) * 16 + l16];
        a.x += x.x; a.y += x.y; a.z += x.z; a.w += x.w;
      }
      const float sv[4] = {a.x, a.y, a.z, a.w};
      const uint32_t vb = (uint32_t)(vmask >> (16 * s + 4 * g)) & 15u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        tv[s][i] = ((vb >> i) & 1u) ? sv[i] * qscale : -INFINITY;
        cmax = fmaxf(cmax, tv[s][i]);
      }
    }
    cmax = head_max(cmax);
    if (m_run == -INFINITY) {
      m_run = cmax;                 // first entries of this head: nothing accumulated yet
    } else if (__builtin_expect(__ballot(cmax > m_run + kLazyRescale) != 0, 0)) {
      const float mn = fmaxf(m_run, cmax);
      const float alpha = exp2f(m_run - mn);
      l_run *= alpha;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] *= alpha;
      m_run = mn;
    }
    float psum = 0.0f;
    f16x4_t pb[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const _Float16 pv = m_run == -INFINITY ? (_Float16)0.0f : (_Float16)exp2f(tv[s][i] - m_run);
        psum += (float)pv;
        pb[s][i] = pv;
      }
    l_run += head_sum(psum);
    // O^T += X^T P^T: this wave's 8 channel tiles over the chunk's 32 entries, one K = 32 MFMA each
    static_assert(NS == 2, "a chunk is two 16-entry halves");
    {
      const f16x8_t p8 = cat_halves(pb[0], pb[1]);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xt_chunk(xtr + 16 * j, kXPitch), p8, acc[j], 0, 0, 0);
    }
  }

  // merge the sub-groups: groups 1.. leave (max, sum) and their tiles in LDS, group 0 combines
  float M = m_run, L = l_run;
  if (NG > 1) {
    __syncthreads();                               // every group is done with its buffers
    if (sg > 0) {
      float4* ob = reinterpret_cast<float4*>(smem + (sg - 1) * Sm::kOut);  // [w4][j][lane]
#pragma unroll
      for (int j = 0; j < 8; ++j) ob[(w4 * 8 + j) * 64 + lane] = make_float4(acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
      if (w4 == 0 && g == 0) {
        ml[(sg * 16 + l16) * 2] = m_run;
        ml[(sg * 16 + l16) * 2 + 1] = l_run;
      }
    }
    __syncthreads();
    if (sg > 0) return;
#pragma unroll
    for (int k = 1; k < NG; ++k) M = fmaxf(M, ml[(k * 16 + l16) * 2]);
    const float f0 = m_run == -INFINITY ? 0.0f : exp2f(m_run - M);
    L = l_run * f0;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= f0;
#pragma unroll
    for (int k = 1; k < NG; ++k) {
      const float mk = ml[(k * 16 + l16) * 2];
      const float fk = mk == -INFINITY ? 0.0f : exp2f(mk - M);
      L += ml[(k * 16 + l16) * 2 + 1] * fk;
      const float4* obk = reinterpret_cast<const float4*>(smem + (k - 1) * Sm::kOut);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float4 o = obk[(w4 * 8 + j) * 64 + lane];
        acc[j] += f32x4_t{o.x, o.y, o.z, o.w} * fk;
      }
    }
  }

  // the workgroup's partial: unnormalized output and (max, sum) in the exp2 domain; the 16 heads'
  // rows leave through LDS as in the decode form (two heads' 512 contiguous bytes per store)
  const int64_t prow = (int64_t)(slot0 + wsplit) * n_rows * H + (int64_t)qr * H + head;
  {
    constexpr int kStRow = 132;
    static_assert((NG - 1) * Sm::kOut + 4 * 16 * kStRow * 4 <= NG * Sm::kGroup, "the output stage fits");
    if constexpr (NG == 1) __syncthreads();   // the stage overlaps the other waves' X slabs
    float* stage = reinterpret_cast<float*>(smem + (NG - 1) * Sm::kOut) + w4 * 16 * kStRow;
#pragma unroll
    for (int j = 0; j < 8; ++j) *reinterpret_cast<f32x4_t*>(stage + l16 * kStRow + 16 * j + 4 * g) = acc[j];
    __builtin_amdgcn_wave_barrier();
    float* dst = part_o + (prow - l16 + (lane >> 5)) * kD + 128 * w4 + 4 * (lane & 31);
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2)
      *reinterpret_cast<float4*>(dst + 2 * s2 * kD) =
          *reinterpret_cast<const float4*>(stage + (2 * s2 + (lane >> 5)) * kStRow + 4 * (lane & 31));
  }
  if (w4 == 0 && g == 0) {
    part_ml[2 * prow] = M;
    part_ml[2 * prow + 1] = L;
  }
}

// Prefill form: many query rows, so one workgroup per (query row, 64 heads) keeps the chip busy
// and each gathered entry is dequantized once for all 64 heads. Four waves; wave w owns channels
// 128w .. 128w+127 throughout, as in the decode form, but every wave serves all 64 heads:
//   - gather + dequantize: a lane fetches one entry's 64-channel slab (32 code bytes, 4 scale
//     bytes) straight into registers, PF chunks ahead, and writes it as f16 (exact) into the
//     wave's own slab of X[entry][channel], which only that wave reads (window chunks: 64 FP8
//     codes and the row's exponent of one window row, the same way);
//   - partial scores S^T = X Q^T over the wave's 128 channels for 32 entries x 64 heads
//     (16x16x32 f16 MFMA); each X fragment read from LDS feeds the four 16-head tiles;
//   - the four partials meet in LDS (the chunk's first barrier); wave w then owns head tile w:
//     it adds them, runs the online softmax of those 16 heads (fp32, exp2 domain, lazy rescale)
//     and publishes their probabilities (f16, already in the B-operand layout of P.V) and
//     rescale factors (the second barrier);
//   - O^T += X^T P^T for the wave's channels and all 64 heads (16x16x32 f16 MFMA, the A operand
//     from the transposing LDS read ds_read_b64_tr_b16), after applying the published factors.
// The selected entries' chunks come first, then (for the windowed call) the query's window rows
// as further chunks of the same softmax. At 256 registers per lane and ~77 KB of LDS two
// workgroups share a CU, so one's gathers and softmax overlap the other's matrix work.
// Workgroups of consecutive query rows, whose selections overlap, run on one XCD and share its L2.
constexpr int kPKC = 32;                         // prefill entries per chunk
constexpr int kPXPitch = kD + 24;                // f16 elements per X row of the prefill form (measured best)

template <int PF, int OCC, int XP>
__global__ __launch_bounds__(256, OCC) void sparse_attn_prefill_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ rows, int n_max,
    const int32_t* __restrict__ idx, int T, int H, int K, float sm_scale, float* __restrict__ out,
    float* __restrict__ lse, int n_rows, int per_xcd, const uint8_t* __restrict__ swa_codes,
    const int8_t* __restrict__ swa_exp, const int32_t* __restrict__ n_win, int W) {
  constexpr int KC = kPKC, NS = KC / 16;
  __shared__ __attribute__((aligned(16))) uint16_t xs[KC * XP];     // X[entry][channel], f16
  // partial S, [wave][t][ht][lane] of 4 components: one 16-byte access per lane, lane-contiguous
  __shared__ __attribute__((aligned(16))) f32x4_t spf[4 * NS * 4 * 64];
  __shared__ __attribute__((aligned(16))) f16x4_t pbuf[4 * NS * 64];     // P: [ht][s][lane]
  __shared__ __attribute__((aligned(16))) float abuf[64];                // rescale factors: [l16][head tile]
  __shared__ float amx[4 * 64];                                          // per-wave |q| max per head
  __shared__ float mlb[2 * 64];                                          // final (max, sum) per head
  __shared__ int sidx[kMaxKPS];

  const int n_hg = H / 64;
  const int u = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (u >= n_rows * n_hg) return;
  const int qr = u / n_hg, hbase = (u % n_hg) * 64;
  const int b = qr / T;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int nk = K;
  const int32_t* irow = idx + (int64_t)qr * K;
  const uint8_t* rbase = rows + (int64_t)b * n_max * kRowB;

  // gather lane: entry gkey of a chunk, 64-channel slab gcs of this wave's 128 channels
  const int gkey = lane & 31, gcs = 2 * w + (lane >> 5);
  int pos0[PF];
#pragma unroll
  for (int v = 0; v < PF; ++v) {
    const int ks = v * KC + gkey;
    pos0[v] = ks < nk ? irow[ks] : -1;
  }
  // this wave's query fragments: head 16 ht + l16, channels 128 w + 32 kk + 8 g .. +7
  uint4 rq[4][4];
  {
    const uint16_t* qrow = q + ((int64_t)qr * H + hbase) * kD + 128 * w + 8 * g;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        rq[ht][kk] = *reinterpret_cast<const uint4*>(qrow + (int64_t)(16 * ht + l16) * kD + 32 * kk);
  }
  constexpr int IPT = kMaxKPS / 256;
  int ipos[IPT];
#pragma unroll
  for (int m = 0; m < IPT; ++m) {
    const int i = tid + m * 256;
    ipos[m] = i < nk ? irow[i] : -1;
  }
  struct Piece {
    uint4 c01, c23;     // the slab's 64 E2M1 codes
    uint32_t sc;        // its 4 E4M3 scales
  };
  Piece gr[PF];
  auto gather_at = [&](Piece& d, int p) {   // p: position, or anything outside [0, n_max)
    d.c01 = d.c23 = make_uint4(0, 0, 0, 0);
    d.sc = 0u;
    if (p >= 0 && p < n_max) {
      const uint8_t* rp = rbase + (int64_t)p * kRowB;
      d.c01 = *reinterpret_cast<const uint4*>(rp + 32 * gcs);
      d.c23 = *reinterpret_cast<const uint4*>(rp + 32 * gcs + 16);
      d.sc = *reinterpret_cast<const uint32_t*>(rp + 256 + 4 * gcs);
    }
  };
#pragma unroll
  for (int v = 0; v < PF; ++v) gather_at(gr[v], pos0[v]);
#pragma unroll
  for (int m = 0; m < IPT; ++m) {
    const int i = tid + m * 256;
    if (i < nk) sidx[i] = (ipos[m] >= 0 && ipos[m] < n_max) ? ipos[m] : -1;
  }
  // per-head |q| max over this wave's channels
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) {
    float amax = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const uint32_t wq[4] = {rq[ht][kk].x, rq[ht][kk].y, rq[ht][kk].z, rq[ht][kk].w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(wq[e] << 16)), fabsf(__uint_as_float(wq[e] & 0xFFFF0000u))));
    }
    amax = head_max(amax);
    if (g == 0) amx[w * 64 + 16 * ht + l16] = amax;
  }
  __syncthreads();
  // queries scaled per head by a power of two (the head's largest |q| into [2^14, 2^15)) and
  // converted to f16 exactly; the factor is folded into the softmax scale of the owning wave
  f16x8_t qb[4][4];
  float qscale = 0.0f;
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) {
    const int hh = 16 * ht + l16;
    const float amax = fmaxf(fmaxf(amx[hh], amx[64 + hh]), fmaxf(amx[128 + hh], amx[192 + hh]));
    const int qe = amax > 0.0f ? 14 - ilogbf(amax) : 0;
    const float sc = ldexpf(1.0f, qe);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const uint32_t wq[4] = {rq[ht][kk].x, rq[ht][kk].y, rq[ht][kk].z, rq[ht][kk].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qb[ht][kk][2 * e] = (_Float16)(__uint_as_float(wq[e] << 16) * sc);
        qb[ht][kk][2 * e + 1] = (_Float16)(__uint_as_float(wq[e] & 0xFFFF0000u) * sc);
      }
    }
    if (ht == w) qscale = sm_scale * kLog2e * ldexpf(1.0f, -qe);
  }

  // output tiles: acc[ht][j] holds channels 128 w + 16 j + (4 g + i) of head 16 ht + l16
  f32x4_t acc[4][8];
#pragma unroll
  for (int ht = 0; ht < 4; ++ht)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[ht][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;    // softmax state of head 16 w + l16 (this wave owns it)
  // transposing-read base for the P.V operand: entry 4 g + l16/4 (+16 s), channel 128 w + 4 (l16%4) (+16 j)
  const uint16_t* xtr = xs + (4 * g + (l16 >> 2)) * XP + 128 * w + 4 * (l16 & 3);
  const uint16_t* xr = xs + l16 * XP + 128 * w + 8 * g;

  // The chunk's math once its 32 entries are in X (this wave's slab written by this wave):
  // partial scores, their sum and the online softmax of the owned head tile, P.V. vmask bit e:
  // entry e of the chunk is real.
  auto chunk_math = [&](uint64_t vmask) {
    // partial S^T over this wave's channels: tile (t, ht), lane holds entries 16 t + 4 g + i of head 16 ht + l16
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      f16x8_t a[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) a[kk] = *reinterpret_cast<const f16x8_t*>(xr + 16 * t * XP + 32 * kk);
      // head tiles in pairs: two independent chains interleaved step by step
#pragma unroll
      for (int hp = 0; hp < 4; hp += 2) {
        f32x4_t sv[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2)
            sv[h2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[kk], qb[hp + h2][kk], sv[h2], 0, 0, 0);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) spf[((w * NS + t) * 4 + hp + h2) * 64 + lane] = sv[h2];
      }
    }
    __syncthreads();
    // head tile w: complete scores, online softmax, publish P and the rescale factor
    {
      float tv[NS][4];
      float cmax = -INFINITY;
      // all partials are read first and masked entries get -inf added (not selected), so no read
      // is moved into a branch
#pragma unroll
      for (int t = 0; t < NS; ++t) {
        const f32x4_t* src = spf + (t * 4 + w) * 64 + lane;
        const f32x4_t sum = src[0] + src[NS * 4 * 64] + src[2 * NS * 4 * 64] + src[3 * NS * 4 * 64];
#pragma unroll
        for (int i = 0; i < 4; ++i) tv[t][i] = sum[i];
      }
#pragma unroll
      for (int t = 0; t < NS; ++t) {
        const uint32_t vb = (uint32_t)(vmask >> (16 * t + 4 * g)) & 15u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          tv[t][i] = tv[t][i] * qscale + (((vb >> i) & 1u) ? 0.0f : -INFINITY);
          cmax = fmaxf(cmax, tv[t][i]);
        }
      }
      cmax = head_max(cmax);
      float alpha = 1.0f;
      if (m_run == -INFINITY) {
        m_run = cmax;              // first entries of this head: nothing accumulated yet
      } else if (__builtin_expect(__ballot(cmax > m_run + kLazyRescale) != 0, 0)) {
        const float mn = fmaxf(m_run, cmax);
        alpha = __builtin_amdgcn_exp2f(m_run - mn);
        l_run *= alpha;
        m_run = mn;
      }
      float psum = 0.0f;
      // with no real entry yet every tv is -inf and so is m_run: exp2(-inf - 0) = 0
      const float m_use = m_run == -INFINITY ? 0.0f : m_run;
#pragma unroll
      for (int t = 0; t < NS; ++t) {
        f16x4_t pb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // exponent <= 8 (lazy rescale); v_exp_f32 directly: the result is rounded to f16 anyway
          const _Float16 pv = (_Float16)__builtin_amdgcn_exp2f(tv[t][i] - m_use);
          psum += (float)pv;       // normalize by the weights the f16 MFMA actually uses
          pb[i] = pv;
        }
        pbuf[(w * NS + t) * 64 + lane] = pb;
      }
      l_run += head_sum(psum);
      if (g == 0) abuf[4 * l16 + w] = alpha;
    }
    __syncthreads();
    // apply the owners' rescale factors, then O^T += X^T P^T over the chunk
    {
      const float4 al = *reinterpret_cast<const float4*>(&abuf[4 * l16]);  // head 16 ht + l16, ht = 0..3
      if (__ballot(al.x != 1.0f || al.y != 1.0f || al.z != 1.0f || al.w != 1.0f) != 0) {
        const float a4[4] = {al.x, al.y, al.z, al.w};
#pragma unroll
        for (int ht = 0; ht < 4; ++ht)
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[ht][j] *= a4[ht];
      }
    }
    static_assert(NS == 2, "a chunk is two 16-entry halves");
    {
      f16x8_t pb[4];
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) pb[ht] = cat_halves(pbuf[(ht * NS) * 64 + lane], pbuf[(ht * NS + 1) * 64 + lane]);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const f16x8_t a = xt_chunk(xtr + 16 * j, XP);
#pragma unroll
        for (int ht = 0; ht < 4; ++ht)
          acc[ht][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pb[ht], acc[ht][j], 0, 0, 0);
      }
    }
  };

  for (int cg = 0; cg < nk; cg += PF * KC)
#pragma unroll
  for (int v = 0; v < PF; ++v) {
    const int c0 = cg + v * KC;
    if (c0 >= nk) break;
    {
      // the next gather's position is read before this chunk's X writes, so waiting for it does
      // not wait for them
      const int ks = c0 + PF * KC + gkey;
      const int pnext = (c0 + PF * KC < nk && ks < nk) ? sidx[ks] : -1;
      // dequantize this lane's slab into X (read by this wave only; a wave's LDS operations
      // complete in order, so the reads below see these writes)
      const Piece& pc = gr[v];
      const f16x2_t s01 = e4m3x2_to_f16(pc.sc), s23 = e4m3x2_to_f16(pc.sc >> 16);
      const f16x2_t sgm[4] = {f16x2_t{s01[0], s01[0]}, f16x2_t{s01[1], s01[1]}, f16x2_t{s23[0], s23[0]},
                              f16x2_t{s23[1], s23[1]}};
      const uint32_t cw[8] = {pc.c01.x, pc.c01.y, pc.c01.z, pc.c01.w, pc.c23.x, pc.c23.y, pc.c23.z, pc.c23.w};
      uint4* dst = reinterpret_cast<uint4*>(xs + gkey * XP + 64 * gcs);
#pragma unroll
      for (int wi = 0; wi < 8; ++wi) {
        uint32_t vv[4];
        e2m1x8_to_f16(cw[wi], sgm[wi >> 1], vv);
        dst[wi] = make_uint4(vv[0], vv[1], vv[2], vv[3]);
      }
      if (c0 + PF * KC < nk) gather_at(gr[v], pnext);
    }
    __builtin_amdgcn_wave_barrier();
    uint64_t vmask;                // bit e: entry c0 + e is a real entry
    {
      int pe = -1;
      if (lane < KC && c0 + lane < nk) pe = sidx[c0 + lane];
      vmask = __ballot(pe >= 0);
    }
    chunk_math(vmask);
  }

  // The query's own sliding window ([walkthrough] 一(四)), joined to the same softmax as up to
  // W / 32 more chunks: the sequence's buffer holds T + W - 1 FP8 rows (row i = token
  // p0 - W + 1 + i) and query t takes its last n = min(n_win, W) tokens up to its own, rows
  // t + W - n .. t + W - 1. A row's value is its E4M3 codes times its power of two 2^e, exact in
  // f16 for e in [-15, 7].
  if (W > 0) {
    const int t_in = qr - b * T;
    const int n_w = max(0, min(n_win[qr], W));
    const uint8_t* wrow0 = swa_codes + ((int64_t)b * (T + W - 1) + t_in + (W - n_w)) * kD + 64 * gcs;
    const int8_t* erow0 = swa_exp + (int64_t)b * (T + W - 1) + t_in + (W - n_w);
    for (int c0 = 0; c0 < n_w; c0 += KC) {
      // a lane's 64-byte slab of window row r (zeros past the window); loading it a chunk ahead
      // measured no faster and costs registers
      const int r = c0 + gkey;
      uint4 wc[4] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
      int we = 0;
      if (r < n_w) {
        const uint4* rp = reinterpret_cast<const uint4*>(wrow0 + (int64_t)r * kD);
#pragma unroll
        for (int m = 0; m < 4; ++m) wc[m] = rp[m];
        we = erow0[r];
      }
      const _Float16 sc = (_Float16)ldexpf(1.0f, we);
      const f16x2_t s2 = f16x2_t{sc, sc};
      uint4* dst = reinterpret_cast<uint4*>(xs + gkey * XP + 64 * gcs);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t cw[4] = {wc[m].x, wc[m].y, wc[m].z, wc[m].w};
        uint32_t vv[8];
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
          vv[2 * t4] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cw[t4], 1.0f, false) * s2);
          vv[2 * t4 + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cw[t4] >> 16, 1.0f, false) * s2);
        }
        dst[2 * m] = make_uint4(vv[0], vv[1], vv[2], vv[3]);
        dst[2 * m + 1] = make_uint4(vv[4], vv[5], vv[6], vv[7]);
      }
      __builtin_amdgcn_wave_barrier();
      const int rows_here = min(KC, n_w - c0);
      chunk_math((1ull << rows_here) - 1ull);
    }
  }

  // each head's (max, sum) from its owner, then every wave writes its channels of all 64 heads
  if (g == 0) {
    mlb[2 * (16 * w + l16)] = m_run;
    mlb[2 * (16 * w + l16) + 1] = l_run;
  }
  __syncthreads();
  // The output leaves one head tile at a time through the wave's own part of X (free now): the
  // accumulator layout gives a lane 16 bytes of one head per store, so a direct store writes 16
  // pieces of 64 bytes; staged, each store writes two heads' 512 contiguous bytes. Rows of the
  // stage are 132 words apart so the 16 heads' writes fall in different banks.
  constexpr int kStRow = 132;
  static_assert(4 * 16 * kStRow * 4 <= KC * XP * 2, "the output stage fits in X");
  float* stage = reinterpret_cast<float*>(xs) + w * 16 * kStRow;
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) {
    const int hh = 16 * ht + l16;
    const float L = mlb[2 * hh + 1];
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const f32x4_t o = acc[ht][j] * inv;
      *reinterpret_cast<float4*>(stage + l16 * kStRow + 16 * j + 4 * g) = make_float4(o[0], o[1], o[2], o[3]);
    }
    __builtin_amdgcn_wave_barrier();
    float* dst = out + ((int64_t)qr * H + hbase + 16 * ht + (lane >> 5)) * kD + 128 * w + 4 * (lane & 31);
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2)
      *reinterpret_cast<float4*>(dst + 2 * s2 * kD) =
          *reinterpret_cast<const float4*>(stage + (2 * s2 + (lane >> 5)) * kStRow + 4 * (lane & 31));
    __builtin_amdgcn_wave_barrier();
  }
  if (lse && g == 0) {
    const float L = l_run;
    lse[(int64_t)qr * H + hbase + 16 * w + l16] = L > 0.0f ? (m_run + log2f(L)) * kLn2 : -INFINITY;
  }
}

// Merge of split results: one wave per (query row, head); a lane owns channels 4 lane .. +3 and
// 256 + 4 lane .. +3, so every load and store of the wave covers 1 KB contiguous. The first 8
// splits' partial rows are loaded together with all splits' (max, sum) pairs, so the common case
// waits on memory once. Workgroups are placed on the XCD whose L2 holds the partials: the
// attention kernels give each XCD a contiguous range of query rows, and so does this mapping.
constexpr int kMaxSplits = 64;

// wave-wide max / sum of one value per lane (DPP row shifts, then row broadcasts)
CSA2_DEV float wave_fmax(float v) {
  const int ninf = __float_as_int(-INFINITY);
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x111, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x112, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x114, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x118, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x142, 0xA, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x143, 0xC, 0xF, false)));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
CSA2_DEV float wave_fsum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// lse0: NULL, or slot 0 holds a normalized output whose natural log-sum-exp is lse0[row]: it
// enters as a partial with m = lse0 * log2(e) and l = 1 (l = 0 when nothing was attended).
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml,
                                                           int n_splits, int64_t n_rows_h,
                                                           float* __restrict__ out,
                                                           float* __restrict__ lse, int per_xcd,
                                                           const float* __restrict__ lse0) {
  const int lane = threadIdx.x & 63;
  const int64_t u = (int64_t)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  const int64_t rh = u * 4 + (threadIdx.x >> 6);
  if (rh >= n_rows_h) return;
  float4 a[8], c[8];
#pragma unroll
  for (int sp = 0; sp < 8; ++sp) {
    if (sp < n_splits) {
      const float4* pp = reinterpret_cast<const float4*>(part_o + (sp * n_rows_h + rh) * kD) + lane;
      a[sp] = pp[0];
      c[sp] = pp[64];
    }
  }
  // lane s < n_splits holds split s's (m, l)
  float ms = -INFINITY, ls = 0.0f;
  if (lane < n_splits) {
    if (lse0 && lane == 0) {
      const float l0 = lse0[rh];
      ms = l0 == -INFINITY ? -INFINITY : l0 * kLog2e;
      ls = l0 == -INFINITY ? 0.0f : 1.0f;
    } else {
      ms = part_ml[2 * (lane * n_rows_h + rh)];
      ls = part_ml[2 * (lane * n_rows_h + rh) + 1];
    }
  }
  const float M = wave_fmax(ms);
  const float w_lane = (ms == -INFINITY) ? 0.0f : exp2f(ms - M);
  const float L = wave_fsum(w_lane * ls);
  float o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  // empty splits (weight 0) may hold anything: they are skipped, not multiplied
  auto add = [&](float w, const float4& x, const float4& y) {
    if (w == 0.0f) return;
    o[0] += w * x.x; o[1] += w * x.y; o[2] += w * x.z; o[3] += w * x.w;
    o[4] += w * y.x; o[5] += w * y.y; o[6] += w * y.z; o[7] += w * y.w;
  };
#pragma unroll
  for (int sp = 0; sp < 8; ++sp)
    if (sp < n_splits) add(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_lane), sp)), a[sp], c[sp]);
  for (int sp = 8; sp < n_splits; ++sp) {
    const float4* pp = reinterpret_cast<const float4*>(part_o + (sp * n_rows_h + rh) * kD) + lane;
    add(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_lane), sp)), pp[0], pp[64]);
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  float4* op = reinterpret_cast<float4*>(out + rh * kD) + lane;
  op[0] = make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
  op[64] = make_float4(o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv);
  if (lse && lane == 0) lse[rh] = L > 0.0f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

// Decode form for few query rows (16 heads per workgroup), wide form otherwise (64 heads).
static bool use_decode_form(int B, int T) { return (int64_t)B * T < 512; }

// Prefill form: wide launches whose heads come in groups of 64 and whose selections fit one split.
static bool use_prefill_form(int B, int T, int H, int K) {
  return !use_decode_form(B, T) && H % 64 == 0 && K > 0 && K <= kMaxKPS;
}

static int attn_splits(int B, int T, int H, int K) {
  if (use_decode_form(B, T)) {
    const int64_t wgs = (int64_t)B * T * (H / 16);
    const int by_fill = (int)std::max<int64_t>(1, (kDecodeFill + wgs - 1) / wgs);
    // at least one chunk per sub-group
    return std::max(1, std::min((K + kDKC * kDNG - 1) / (kDKC * kDNG), by_fill));
  }
  if (use_prefill_form(B, T, H, K)) return 1;
  const int hpw = H >= 64 ? 64 : H;
  const int64_t wgs = (int64_t)B * T * (H / hpw);
  if (wgs >= 256 || K <= 2 * kKC) return 1;
  int splits = (int)std::min<int64_t>((K + 2 * kKC - 1) / (2 * kKC), std::max<int64_t>(1, 512 / wgs));
  return std::max(1, splits);
}

static int split_count(int B, int T, int H, int K, int* kps_out) {
  const int chunk = use_decode_form(B, T) ? kDKC : kKC;
  const int sp = std::max(attn_splits(B, T, H, K), (K + kMaxKPS - 1) / kMaxKPS);
  int kps = (K + sp - 1) / sp;
  kps = std::max(chunk, (kps + chunk - 1) / chunk * chunk);
  kps = std::min(kps, kMaxKPS);
  // the merge kernel reads at most kMaxSplits splits
  const int min_kps = (K + kMaxSplits - 1) / kMaxSplits;
  if (kps < min_kps) kps = (min_kps + chunk - 1) / chunk * chunk;
  if (kps_out) *kps_out = kps;
  return std::max(1, (K + kps - 1) / kps);
}

size_t attn_workspace(int B, int T, int H, int D, int K) {
  const int sp = split_count(B, T, H, K, nullptr);
  if (sp == 1) return 0;
  const size_t rows_h = (size_t)B * T * H;
  return sp * rows_h * (size_t)D * 4 + sp * rows_h * 8 + 256;
}

hipError_t launch_sparse_attn(const uint16_t* q, const uint8_t* rows, int n_max, const int32_t* idx,
                              int B, int T, int H, int D, int K, float sm_scale, float* out,
                              float* lse, void* ws, hipStream_t s) {
  const int64_t nq = (int64_t)B * T;
  if (nq == 0 || H == 0) return hipSuccess;
  int kps = 0;
  const int n_splits = split_count(B, T, H, K, &kps);
  float* part_o = nullptr;
  float* part_ml = nullptr;
  if (n_splits > 1) {
    part_o = static_cast<float*>(ws);
    part_ml = part_o + (size_t)n_splits * nq * H * kD;
  }
  if (use_prefill_form(B, T, H, K)) {
    const int64_t items = nq * (H / 64);
    const int per_xcd = (int)((items + 7) / 8);
    hipLaunchKernelGGL((sparse_attn_prefill_kernel<1, 2, kPXPitch>), dim3((unsigned)(8 * per_xcd)), dim3(256), 0, s, q, rows, n_max,
                       idx, T, H, K, sm_scale, out, lse, (int)nq, per_xcd, nullptr, nullptr, nullptr, 0);
    return hipGetLastError();
  }
  if (use_decode_form(B, T)) {
    const int64_t items = nq * n_splits * (H / 16);
    const int per_xcd = (int)((items + 7) / 8);
    hipLaunchKernelGGL((sparse_attn_decode_kernel<kDKC, kDPF, kDNG>), dim3((unsigned)(8 * per_xcd)), dim3(256 * kDNG), 0, s, q,
                       rows, n_max, idx, T, H, K, kps, sm_scale, out, lse, part_o, part_ml, (int)nq, n_splits,
                       (int)(n_splits == 1), per_xcd);
  } else {
    const int hpw = H >= 64 ? 64 : H;
    dim3 grid((unsigned)nq, (unsigned)n_splits, (unsigned)(H / hpw));
    switch (hpw / 16) {
      case 1: hipLaunchKernelGGL(sparse_attn_kernel<1>, grid, dim3(64), 0, s, q, rows, n_max, idx, T, H, K, kps, sm_scale, out, lse, part_o, part_ml); break;
      case 2: hipLaunchKernelGGL(sparse_attn_kernel<2>, grid, dim3(128), 0, s, q, rows, n_max, idx, T, H, K, kps, sm_scale, out, lse, part_o, part_ml); break;
      case 3: hipLaunchKernelGGL(sparse_attn_kernel<3>, grid, dim3(192), 0, s, q, rows, n_max, idx, T, H, K, kps, sm_scale, out, lse, part_o, part_ml); break;
      default: hipLaunchKernelGGL(sparse_attn_kernel<4>, grid, dim3(256), 0, s, q, rows, n_max, idx, T, H, K, kps, sm_scale, out, lse, part_o, part_ml); break;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_splits == 1) return e;
  const int64_t rows_h = nq * H;
  const int per_xcd = (int)(((rows_h + 3) / 4 + 7) / 8);
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)(8 * per_xcd)), dim3(256), 0, s, part_o, part_ml,
                     n_splits, rows_h, out, lse, per_xcd, nullptr);
  return hipGetLastError();
}

// The window's share of the combine pass: one slot per kDKC * kDNG window rows, or, when that
// grid would leave CUs idle (few sequences), one slot per kDKC rows for a one-sub-group form of
// the window kernel (256 lanes, half the LDS, so two workgroups share a CU).
constexpr int kSwaRowsPerSplit = kDKC * kDNG;
constexpr int kMaxSwaSplits = 4;                 // windows of up to 128 rows, 32 rows per slot

// Splits of the selected entries when the window joins them (decode form at any batch): as the
// decode form's own count, leaving kMaxSwaSplits slots of the combine pass to the window.
static int swa_sparse_splits(int B, int H, int K, int* kps_out) {
  if (K <= 0) {
    if (kps_out) *kps_out = kDKC;
    return 0;
  }
  const int64_t wgs = (int64_t)B * (H / 16);
  const int by_fill = (int)std::max<int64_t>(1, (kDecodeFill + wgs - 1) / wgs);
  int sp = std::max(1, std::min((K + kDKC * kDNG - 1) / (kDKC * kDNG), by_fill));
  sp = std::max(sp, (K + kMaxKPS - 1) / kMaxKPS);
  int kps = (K + sp - 1) / sp;
  kps = std::min(kMaxKPS, std::max(kDKC, (kps + kDKC - 1) / kDKC * kDKC));
  const int max_sp = kMaxSplits - kMaxSwaSplits;
  const int min_kps = (K + max_sp - 1) / max_sp;
  if (kps < min_kps) kps = (min_kps + kDKC - 1) / kDKC * kDKC;
  if (kps_out) *kps_out = kps;
  return (K + kps - 1) / kps;
}

size_t attn_swa_workspace(int B, int H, int D, int K) {
  const size_t slots = (size_t)swa_sparse_splits(B, H, K, nullptr) + kMaxSwaSplits;
  const size_t rows_h = (size_t)B * H;
  return slots * rows_h * (size_t)D * 4 + slots * rows_h * 8 + 256;
}

hipError_t launch_sparse_attn_swa(const uint16_t* q, const uint8_t* rows, int n_max, const int32_t* idx, int B,
                                  int H, int D, int K, const uint8_t* swa_codes, const int8_t* swa_exp,
                                  const int32_t* n_win, int W, float sm_scale, float* out, float* lse, void* ws,
                                  hipStream_t s) {
  (void)D;
  if (B == 0 || H == 0) return hipSuccess;
  int kps = kDKC;
  const int n_sp = swa_sparse_splits(B, H, K, &kps);
  const int n_ws = (W + kSwaRowsPerSplit - 1) / kSwaRowsPerSplit;     // 0 .. 2 with 64-row slots
  int n_used = 0;                                                       // window slots written
  const int64_t rows_h = (int64_t)B * H;
  float* part_o = static_cast<float*>(ws);
  float* part_ml = part_o + (size_t)(n_sp + kMaxSwaSplits) * rows_h * kD;
  const int n_hg = H / 16;
  if (n_sp > 0) {
    const int per_xcd = (int)(((int64_t)B * n_sp * n_hg + 7) / 8);
    hipLaunchKernelGGL((sparse_attn_decode_kernel<kDKC, kDPF, kDNG>), dim3((unsigned)(8 * per_xcd)), dim3(256 * kDNG), 0, s,
                       q, rows, n_max, idx, 1, H, K, kps, sm_scale, out, lse, part_o, part_ml, B, n_sp, 0, per_xcd);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (n_ws > 0) {
    // few sequences: 32-row slots and the one-sub-group kernel (19.2 -> 17.6 us per call at 4
    // sequences x 64 heads x 128 rows; at 32 sequences the two-sub-group form is faster)
    const bool small = (int64_t)B * n_ws * n_hg < 256;
    const int ws_n = small ? (W + kDKC - 1) / kDKC : n_ws;
    const int per_xcd = (int)(((int64_t)B * ws_n * n_hg + 7) / 8);
    if (small)
      hipLaunchKernelGGL((swa_attn_kernel<kDKC, kDPF, 1>), dim3((unsigned)(8 * per_xcd)), dim3(256), 0, s,
                         q, swa_codes, swa_exp, n_win, 1, 0, W, H, kDKC, sm_scale, part_o, part_ml, n_sp, B, ws_n,
                         per_xcd);
    else
      hipLaunchKernelGGL((swa_attn_kernel<kDKC, kDPF, kDNG>), dim3((unsigned)(8 * per_xcd)), dim3(256 * kDNG), 0, s,
                         q, swa_codes, swa_exp, n_win, 1, 0, W, H, kSwaRowsPerSplit, sm_scale, part_o, part_ml, n_sp, B,
                         n_ws, per_xcd);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    n_used = ws_n;
  }
  const int per_xcd = (int)(((rows_h + 3) / 4 + 7) / 8);
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)(8 * per_xcd)), dim3(256), 0, s, part_o, part_ml,
                     n_sp + n_used, rows_h, out, lse, per_xcd, nullptr);
  return hipGetLastError();
}

// Prefill with the window: slot 0 of the split buffers takes the sparse attention's normalized
// output (its log-sum-exp alongside), slot 1 the window's partials; one combine pass.
constexpr int kSwaPrefillSlots = 2;
size_t attn_swa_prefill_workspace(int B, int T, int H, int D, int K) {
  if (use_prefill_form(B, T, H, K)) return 0;       // the window joins the prefill form's own loop
  const size_t rows_h = (size_t)B * T * H;
  const size_t slots = kSwaPrefillSlots;
  const size_t parts = ((slots * rows_h * (size_t)D * 4 + slots * rows_h * 8 + rows_h * 4) + 255) & ~(size_t)255;
  return parts + (K > 0 ? attn_workspace(B, T, H, D, K) : 0) + 256;
}

hipError_t launch_sparse_attn_swa_prefill(const uint16_t* q, const uint8_t* rows, int n_max, const int32_t* idx,
                                          int B, int T, int H, int D, int K, const uint8_t* swa_codes,
                                          const int8_t* swa_exp, const int32_t* n_win, int W, float sm_scale,
                                          float* out, float* lse, void* ws, hipStream_t s) {
  if (B == 0 || T == 0 || H == 0) return hipSuccess;
  const int64_t nq = (int64_t)B * T, rows_h = nq * H;
  if (use_prefill_form(B, T, H, K)) {
    // one pass: each query's window rows run as further chunks of the same online softmax
    const int per_xcd = (int)((nq * (H / 64) + 7) / 8);
    hipLaunchKernelGGL((sparse_attn_prefill_kernel<1, 2, kPXPitch>), dim3((unsigned)(8 * per_xcd)), dim3(256), 0, s, q, rows,
                       n_max, idx, T, H, K, sm_scale, out, lse, (int)nq, per_xcd, swa_codes, swa_exp, n_win, W);
    return hipGetLastError();
  }
  const size_t slots = kSwaPrefillSlots;
  float* part_o = static_cast<float*>(ws);
  float* part_ml = part_o + slots * (size_t)rows_h * kD;
  float* lse_s = part_ml + 2 * slots * (size_t)rows_h;
  const size_t parts = ((slots * rows_h * (size_t)D * 4 + slots * rows_h * 8 + rows_h * 4) + 255) & ~(size_t)255;
  void* attn_ws = static_cast<uint8_t*>(ws) + parts;
  const int n_sp = K > 0 ? 1 : 0;
  if (n_sp) {
    const hipError_t e = launch_sparse_attn(q, rows, n_max, idx, B, T, H, D, K, sm_scale, part_o, lse_s, attn_ws, s);
    if (e != hipSuccess) return e;
  }
  // many query rows keep the chip busy: one slot holds a token's whole window (each sub-group
  // takes half of it), which halves the window workgroups and the partials the combine reads
  const int n_ws = W > 0 ? 1 : 0;
  const int rps = (W + kSwaRowsPerSplit - 1) / kSwaRowsPerSplit * kSwaRowsPerSplit;
  const int n_hg = H / 16;
  if (n_ws > 0) {
    const int per_xcd = (int)((nq * n_ws * n_hg + 7) / 8);
    hipLaunchKernelGGL((swa_attn_kernel<kDKC, kDPF, kDNG>), dim3((unsigned)(8 * per_xcd)), dim3(256 * kDNG), 0, s,
                       q, swa_codes, swa_exp, n_win, T, 1, W, H, rps, sm_scale, part_o, part_ml, n_sp,
                       (int)nq, n_ws, per_xcd);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int per_xcd = (int)(((rows_h + 3) / 4 + 7) / 8);
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)(8 * per_xcd)), dim3(256), 0, s, part_o, part_ml,
                     n_sp + n_ws, rows_h, out, lse, per_xcd, n_sp ? lse_s : nullptr);
  return hipGetLastError();
}

}  // namespace csa2
