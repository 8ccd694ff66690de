// Top-K selection and candidate-pool expansion.
// Source: DeepSeek-V4.1-Flash walkthrough (wkq9411.github.io), 一(四) (each query keeps its
// Top-K entries) and 一(四)2 (the highest-scoring blocks are chosen and the positions they
// cover become the candidate pool).
//
// One workgroup (16 waves) selects the k best of a segment of up to 32768 columns held in LDS as
// order-preserving 32-bit keys. An MSB-first radix select (8-bit digits, per-wave LDS histograms)
// finds the threshold bin; it stops early once the bin is taken whole. A wave-ordered compaction
// (ballot + popcount, no atomics) then emits the chosen columns in ascending column order, so the
// result is deterministic and ties go to the lower position. Rows longer than one segment are
// split: each segment's k best (key, position) pairs go to scratch, and the same kernel selects
// again over those candidates; the global k best always survive their segment.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace csa2 {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kSegMax = 32768;        // keys per workgroup (128 KB of LDS)
constexpr int kSegSplit = 16384;      // segment length when a row is split

struct TopkIn {
  // scores mode
  const float* scores;
  int64_t ld;                  // row stride of scores / col_to_pos
  const int32_t* n_valid;      // nullable
  int valid_div;               // columns valid per row = ceil(n_valid[r] / valid_div)
  const int32_t* col_to_pos;   // nullable
  // candidate mode
  const uint32_t* ckeys;
  const int32_t* cpos;
  int64_t cld;                 // row stride of candidate arrays
  int n_in;                    // columns per row
};

struct TopkOut {
  // final mode
  int32_t* idx;                // [rows, k * expand]
  int expand;                  // 0: plain positions; b > 0: block b expansion
  const int32_t* expand_n_vis; // nullable, positions >= n_vis[r] become -1 when expanding
  int expand_limit;            // used instead when expand_n_vis is null
  // partial mode
  uint32_t* okeys;
  int32_t* opos;
  int64_t old;                 // row stride of partial outputs (= segments * k)
};

template <bool kFromCand, bool kFinal>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkIn in, TopkOut out, int seg_len, int k) {
  extern __shared__ uint32_t lds[];
  uint32_t* keys = lds;                                    // [seg_len]
  uint32_t* whist = lds + seg_len;                         // [16][256] per-wave histograms
  __shared__ uint32_t hist[256];
  __shared__ int wcnt[kTopkWaves][2];
  __shared__ int sel_info[4];                              // digit, above, count in bin
  __shared__ int red[kTopkWaves];

  const int r = blockIdx.x, seg = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c0 = seg * seg_len;
  const int n = min(seg_len, in.n_in - c0);
  const int lim = kFromCand ? in.n_in
                            : (in.n_valid ? min((in.n_valid[r] + in.valid_div - 1) / in.valid_div, in.n_in)
                                          : in.n_in);

  // ---- load keys (0 = not a candidate) and count candidates ----
  int cnt = 0;
  for (int i = tid; i < n; i += kTopkThreads) {
    const int c = c0 + i;
    uint32_t key = 0;
    if (kFromCand) {
      if (in.cpos[r * in.cld + c] >= 0) key = in.ckeys[r * in.cld + c];
    } else if (c < lim) {
      const int p = in.col_to_pos ? in.col_to_pos[r * in.ld + c] : c;
      if (p >= 0) key = score_key(in.scores[r * in.ld + c]);
    }
    keys[i] = key;
    cnt += key != 0;
  }
  // block sum of cnt
  for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off, kWave);
  if (lane == 0) red[wave] = cnt;
  __syncthreads();
  int total = 0;
  for (int w = 0; w < kTopkWaves; ++w) total += red[w];
  const int kk = min(k, total);

  // ---- radix select: threshold range [lo, hi] and how many of it to take (krem) ----
  uint32_t lo = 1, hi = 0xFFFFFFFFu;
  int krem = kk;
  if (kk > 0 && kk < total) {
    uint32_t prefix = 0, mask = 0;
    for (int shift = 24; shift >= 0; shift -= 8) {
      uint32_t* wh = whist + wave * 256;
      for (int i = lane; i < 256; i += kWave) wh[i] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += kTopkThreads) {
        const uint32_t key = keys[i];
        if (key != 0 && (key & mask) == prefix) atomicAdd(&wh[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < 256) {
        uint32_t s = 0;
        for (int w = 0; w < kTopkWaves; ++w) s += whist[w * 256 + tid];
        hist[tid] = s;
      }
      __syncthreads();
      if (wave == 0) {
        // lane l owns bins 4l .. 4l+3; suffix sums over lanes give the count above each bin
        const int h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
        const int tot = h0 + h1 + h2 + h3;
        int suf = tot;
        for (int off = 1; off < 64; off <<= 1) {
          const int o = __shfl_down(suf, off, kWave);
          if (lane + off < 64) suf += o;
        }
        int above = suf - tot;
        const int hb[4] = {h0, h1, h2, h3};
        for (int bi = 3; bi >= 0; --bi) {
          if (above < krem && krem <= above + hb[bi]) {
            sel_info[0] = 4 * lane + bi;
            sel_info[1] = above;
            sel_info[2] = hb[bi];
          }
          above += hb[bi];
        }
      }
      __syncthreads();
      const uint32_t d = (uint32_t)sel_info[0];
      krem -= sel_info[1];
      prefix |= d << shift;
      mask |= 0xFFu << shift;
      const bool whole = sel_info[2] == krem;
      __syncthreads();  // sel_info is rewritten by the next pass
      if (whole) break;
    }
    lo = prefix;
    hi = prefix | ~mask;
  }

  // ---- wave-ordered compaction: ascending column order ----
  const int per_wave = ((n + kTopkWaves - 1) / kTopkWaves + 63) & ~63;
  const int wb = wave * per_wave, we = min(n, wb + per_wave);
  int gt = 0, eq = 0;
  if (kk > 0) {
    for (int base = wb; base < we; base += kWave) {
      const int i = base + lane;
      const uint32_t key = i < we ? keys[i] : 0u;
      const bool is_gt = key != 0 && key > hi;
      const bool is_eq = key != 0 && key >= lo && key <= hi;
      gt += __popcll(__ballot(is_gt));
      eq += __popcll(__ballot(is_eq));
    }
  }
  if (lane == 0) { wcnt[wave][0] = gt; wcnt[wave][1] = eq; }
  __syncthreads();
  int out_pos = 0, eq_before = 0;
  for (int w = 0; w < wave; ++w) {
    const int g = wcnt[w][0], e = wcnt[w][1];
    out_pos += g + max(0, min(e, krem - eq_before));
    eq_before += e;
  }
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  if (kk > 0) {
    for (int base = wb; base < we; base += kWave) {
      const int i = base + lane;
      const uint32_t key = i < we ? keys[i] : 0u;
      const bool is_gt = key != 0 && key > hi;
      const bool is_eq = key != 0 && key >= lo && key <= hi;
      const uint64_t eqm = __ballot(is_eq);
      const bool take = is_gt || (is_eq && eq_before + __popcll(eqm & lt_mask) < krem);
      const uint64_t tm = __ballot(take);
      if (take) {
        const int o = out_pos + __popcll(tm & lt_mask);
        const int c = c0 + i;
        int pos;
        if (kFromCand) pos = in.cpos[r * in.cld + c];
        else pos = in.col_to_pos ? in.col_to_pos[r * in.ld + c] : c;
        if (kFinal) {
          if (out.expand > 0) {
            const int nv = out.expand_n_vis ? out.expand_n_vis[r] : out.expand_limit;
            int32_t* dst = out.idx + ((int64_t)r * k + o) * out.expand;
            for (int u = 0; u < out.expand; ++u) {
              const int p = pos * out.expand + u;
              dst[u] = p < nv ? p : -1;
            }
          } else {
            out.idx[(int64_t)r * k + o] = pos;
          }
        } else {
          out.okeys[r * out.old + (int64_t)seg * k + o] = key;
          out.opos[r * out.old + (int64_t)seg * k + o] = pos;
        }
      }
      out_pos += __popcll(tm);
      eq_before += __popcll(eqm);
    }
  }
  // ---- padding ----
  for (int o = kk + tid; o < k; o += kTopkThreads) {
    if (kFinal) {
      const int e = out.expand > 0 ? out.expand : 1;
      for (int u = 0; u < e; ++u) out.idx[((int64_t)r * k + o) * e + u] = -1;
    } else {
      out.okeys[r * out.old + (int64_t)seg * k + o] = 0u;
      out.opos[r * out.old + (int64_t)seg * k + o] = -1;
    }
  }
}

static size_t lds_bytes(int seg_len) { return (size_t)seg_len * 4 + (size_t)kTopkWaves * 256 * 4; }

template <bool A, bool B>
static hipError_t launch_one(dim3 grid, const TopkIn& in, const TopkOut& out, int seg_len, int k,
                             hipStream_t s) {
  static bool attr_set = false;
  const size_t lds = lds_bytes(seg_len);
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)topk_kernel<A, B>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes(kSegMax));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((topk_kernel<A, B>), grid, dim3(kTopkThreads), lds, s, in, out, seg_len, k);
  return hipGetLastError();
}

// Plan of segment sizes: returns the number of stages and fills seg lengths / segment counts.
struct TopkPlan {
  int stages;
  int seg[8];
  int nseg[8];
  int n_in[8];
};

static TopkPlan make_plan(int n_cols, int k) {
  TopkPlan p{};
  int n = n_cols;
  int st = 0;
  while (true) {
    p.n_in[st] = n;
    if (n <= kSegMax || st == 7) {
      p.seg[st] = n;
      p.nseg[st] = 1;
      p.stages = st + 1;
      return p;
    }
    const int seg = min(kSegMax, max(kSegSplit, 4 * k));
    p.seg[st] = seg;
    p.nseg[st] = (n + seg - 1) / seg;
    n = p.nseg[st] * k;
    ++st;
  }
}

size_t topk_workspace(int64_t rows, int n_cols, int k) {
  const TopkPlan p = make_plan(n_cols, k);
  size_t largest = 0;
  for (int st = 0; st + 1 < p.stages; ++st)
    largest = std::max(largest, (size_t)rows * p.nseg[st] * k * 8);
  largest = (largest + 255) & ~(size_t)255;
  return 2 * largest;
}

hipError_t launch_topk(const float* scores, int64_t rows, int n_cols, const int32_t* n_valid,
                       int valid_div, const int32_t* col_to_pos, int k, int32_t* idx,
                       int expand_block, const int32_t* expand_n_vis, int expand_limit, void* ws,
                       hipStream_t s) {
  if (rows == 0 || k == 0) return hipSuccess;
  const TopkPlan p = make_plan(n_cols, k);
  size_t half = 0;
  for (int st = 0; st + 1 < p.stages; ++st) half = std::max(half, (size_t)rows * p.nseg[st] * k * 8);
  half = (half + 255) & ~(size_t)255;
  uint8_t* wsb = static_cast<uint8_t*>(ws);

  TopkOut fin{};
  fin.idx = idx;
  fin.expand = expand_block;
  fin.expand_n_vis = expand_n_vis;
  fin.expand_limit = expand_limit;
  TopkIn in{};
  in.scores = scores;
  in.ld = n_cols;
  in.n_valid = n_valid;
  in.valid_div = valid_div > 0 ? valid_div : 1;
  in.col_to_pos = col_to_pos;
  in.n_in = n_cols;
  for (int st = 0; st < p.stages; ++st) {
    const bool last = st + 1 == p.stages;
    dim3 grid((unsigned)rows, (unsigned)p.nseg[st]);
    TopkOut o = fin;
    if (!last) {
      uint8_t* buf = wsb + (st & 1) * half;
      const size_t cnt = (size_t)rows * p.nseg[st] * k;
      o.okeys = reinterpret_cast<uint32_t*>(buf);
      o.opos = reinterpret_cast<int32_t*>(buf + cnt * 4);
      o.old = (int64_t)p.nseg[st] * k;
    }
    hipError_t e;
    if (st == 0)
      e = last ? launch_one<false, true>(grid, in, o, p.seg[st], k, s)
               : launch_one<false, false>(grid, in, o, p.seg[st], k, s);
    else
      e = last ? launch_one<true, true>(grid, in, o, p.seg[st], k, s)
               : launch_one<true, false>(grid, in, o, p.seg[st], k, s);
    if (e != hipSuccess) return e;
    if (!last) {
      TopkIn next{};
      next.ckeys = o.okeys;
      next.cpos = o.opos;
      next.cld = o.old;
      next.n_in = (int)o.old;
      in = next;
    }
  }
  return hipSuccess;
}

}  // namespace csa2
