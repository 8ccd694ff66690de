// Top-K selection and candidate-pool expansion.
// Source: DeepSeek-V4.1-Flash walkthrough (wkq9411.github.io), 一(四) (each query keeps its
// Top-K entries) and 一(四)2 (the highest-scoring blocks are chosen and the positions they
// cover become the candidate pool).
//
// One workgroup (16 waves) selects the k best of a segment of up to 16384 columns. Lane l of
// wave w holds columns 64*(w*EPL + i) + l (i < EPL) in registers as order-preserving 32-bit keys
// (key 0 = not a candidate), so a wave's i-th register row is 64 consecutive columns:
//   1. pruning bound: each lane's EPL columns form a group; at least k group maxima are >= the
//      k-th largest group maximum, so the k-th best column is too. One 12-bit histogram of the
//      group maxima gives a lower edge L of that maximum's bin, and every column below L is
//      dropped (typically ~95% of them) before any further work;
//   2. MSB-first radix select over the survivors with 12, 12 and 8-bit digits (LDS histograms,
//      DPP prefix scans to locate the bin), stopping once the threshold bin is taken whole;
//   3. compaction in ascending column order with ballot + mbcnt per register row (no shuffles),
//      so the result is deterministic and ties go to the lower position.
// Rows longer than one segment are split: each segment's k best (key, position) pairs go to
// scratch, and the same kernel selects again over those candidates; the global k best always
// survive their segment.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace csa2 {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kSegMax = 16384;        // columns per workgroup: 16 per lane
constexpr int kHistBins = 4096;       // largest radix digit: 12 bits

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

// Inclusive prefix sum over the 64 lanes of a wave (DPP row shifts, then row broadcasts).
CSA2_DEV int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
  return v;
}

// Number of set bits of a wave-wide mask in lanes below this one.
CSA2_DEV int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Block-wide sum (every thread gets it). Uses red[0..kTopkWaves).
CSA2_DEV int block_sum(int v, int* red) {
  v = __builtin_amdgcn_readlane(wave_incl_scan(v), 63);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) t += red[w];
  return t;
}

// Given a filled histogram of nbins bins, find the bin d holding the krem-th largest entry:
// count above d < krem <= count above d + hist[d]. Returns (d, above, hist[d]) to every thread.
CSA2_DEV void find_bin(const uint32_t* hist, int nbins, int krem, int* red, int* info, int& d, int& above,
                       int& cnt) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bpt = nbins >= kTopkThreads ? nbins / kTopkThreads : 1;
  const bool owner = tid * bpt < nbins;
  int h[4] = {0, 0, 0, 0};
  int tot = 0;
  if (owner)
    for (int u = 0; u < bpt; ++u) { h[u] = hist[tid * bpt + u]; tot += h[u]; }
  const int pre = wave_incl_scan(tot);
  if (lane == 63) red[wave] = pre;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const int x = red[w];
    before += w < wave ? x : 0;
    all += x;
  }
  int ab = all - before - pre;    // entries in bins above this thread's bins
  if (owner && ab < krem && krem <= ab + tot) {
    for (int u = bpt - 1; u >= 0; --u) {
      if (ab < krem && krem <= ab + h[u]) {
        info[0] = tid * bpt + u;
        info[1] = ab;
        info[2] = h[u];
      }
      ab += h[u];
    }
  }
  __syncthreads();
  d = info[0];
  above = info[1];
  cnt = info[2];
  __syncthreads();
}

template <bool kFromCand, bool kFinal, int EPL>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkIn in, TopkOut out, int seg_len, int k) {
  __shared__ uint32_t hist[kHistBins];
  __shared__ int red[kTopkWaves];
  __shared__ int info[4];
  __shared__ int wcnt[kTopkWaves][2];

  const int r = blockIdx.x, seg = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c0 = seg * seg_len;
  const int n = min(seg_len, in.n_in - c0);
  const int lim = kFromCand ? in.n_in
                            : (in.n_valid ? min((in.n_valid[r] + in.valid_div - 1) / in.valid_div, in.n_in)
                                          : in.n_in);
  const int wbase = wave * 64 * EPL;       // this wave's first column (segment-relative)

  // ---- load keys into registers: register i of lane l is column wbase + 64 i + l ----
  uint32_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = wbase + 64 * i + lane, c = c0 + e;
    uint32_t kv = 0;
    if (kFromCand) {
      if (e < n) {
        const int64_t off = r * in.cld + c;
        if (in.cpos[off] >= 0) kv = in.ckeys[off];
      }
    } else if (e < n && c < lim) {
      const int p = in.col_to_pos ? in.col_to_pos[r * in.ld + c] : c;
      if (p >= 0) kv = score_key(in.scores[r * in.ld + c]);
    }
    key[i] = kv;
  }
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < EPL; ++i) cnt += key[i] != 0;
  int total = block_sum(cnt, red);
  const int kk = min(k, total);

  // ---- threshold range [lo, hi] and how many of it to take (krem) ----
  uint32_t lo = 1, hi = 0xFFFFFFFFu;
  int krem = kk;
  if (kk > 0 && kk < total) {
    // 1. pruning bound from the per-lane group maxima (needs >= k non-empty groups)
    if (EPL >= 4) {
      uint32_t gm = 0;
#pragma unroll
      for (int i = 0; i < EPL; ++i) gm = max(gm, key[i]);
      const int ng = block_sum(gm != 0, red);
      if (ng >= kk) {
        for (int i = tid; i < kHistBins; i += kTopkThreads) hist[i] = 0;
        __syncthreads();
        if (gm != 0) atomicAdd(&hist[gm >> 20], 1u);
        __syncthreads();
        int d, ab, c;
        find_bin(hist, kHistBins, kk, red, info, d, ab, c);
        const uint32_t L = (uint32_t)d << 20;
        cnt = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
          if (key[i] < L) key[i] = 0;
          cnt += key[i] != 0;
        }
        total = block_sum(cnt, red);
      }
    }
    // 2. radix select over the survivors
    if (kk < total) {
      uint32_t prefix = 0, mask = 0;
      constexpr int kShift[3] = {20, 8, 0};
      constexpr int kBits[3] = {12, 12, 8};
      for (int pass = 0; pass < 3; ++pass) {
        const int shift = kShift[pass];
        const uint32_t dmask = (1u << kBits[pass]) - 1u;
        const int nbins = 1 << kBits[pass];
        for (int i = tid; i < nbins; i += kTopkThreads) hist[i] = 0;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < EPL; ++i)
          if (key[i] != 0 && (key[i] & mask) == prefix) atomicAdd(&hist[(key[i] >> shift) & dmask], 1u);
        __syncthreads();
        int d, ab, c;
        find_bin(hist, nbins, krem, red, info, d, ab, c);
        krem -= ab;
        prefix |= (uint32_t)d << shift;
        mask |= dmask << shift;
        if (c == krem) break;
      }
      lo = prefix;
      hi = prefix | ~mask;
    }
  }

  // ---- compaction in ascending column order ----
  int gt = 0, eq = 0;
  if (kk > 0) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      gt += __popcll(__ballot(key[i] != 0 && key[i] > hi));
      eq += __popcll(__ballot(key[i] != 0 && key[i] >= lo && key[i] <= hi));
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
  if (kk > 0) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const uint32_t kv = key[i];
      const bool is_gt = kv != 0 && kv > hi;
      const bool is_eq = kv != 0 && kv >= lo && kv <= hi;
      const uint64_t be = __ballot(is_eq);
      const uint64_t bg = __ballot(is_gt);
      if ((be | bg) == 0) continue;
      const bool take = is_gt || (is_eq && eq_before + lanes_below(be) < krem);
      const uint64_t bt = __ballot(take);
      if (take) {
        const int o = out_pos + lanes_below(bt);
        const int c = c0 + wbase + 64 * i + lane;
        int pos;
        if (kFromCand) pos = in.cpos[r * in.cld + c];
        else pos = in.col_to_pos ? in.col_to_pos[r * in.ld + c] : c;
        if (kFinal) {
          if (out.expand > 0) {
            const int nv = out.expand_n_vis ? out.expand_n_vis[r] : out.expand_limit;
            int32_t* dst = out.idx + ((int64_t)r * k + o) * out.expand;
            for (int v = 0; v < out.expand; ++v) {
              const int p = pos * out.expand + v;
              dst[v] = p < nv ? p : -1;
            }
          } else {
            out.idx[(int64_t)r * k + o] = pos;
          }
        } else {
          out.okeys[r * out.old + (int64_t)seg * k + o] = kv;
          out.opos[r * out.old + (int64_t)seg * k + o] = pos;
        }
      }
      out_pos += __popcll(bt);
      eq_before += __popcll(be);
    }
  }
  // ---- padding ----
  for (int o = kk + tid; o < k; o += kTopkThreads) {
    if (kFinal) {
      const int e = out.expand > 0 ? out.expand : 1;
      for (int v = 0; v < e; ++v) out.idx[((int64_t)r * k + o) * e + v] = -1;
    } else {
      out.okeys[r * out.old + (int64_t)seg * k + o] = 0u;
      out.opos[r * out.old + (int64_t)seg * k + o] = -1;
    }
  }
}

template <bool A, bool B>
static hipError_t launch_one(dim3 grid, const TopkIn& in, const TopkOut& out, int seg_len, int k,
                             hipStream_t s) {
  const dim3 blk(kTopkThreads);
  if (seg_len <= kTopkThreads * 1)
    hipLaunchKernelGGL((topk_kernel<A, B, 1>), grid, blk, 0, s, in, out, seg_len, k);
  else if (seg_len <= kTopkThreads * 2)
    hipLaunchKernelGGL((topk_kernel<A, B, 2>), grid, blk, 0, s, in, out, seg_len, k);
  else if (seg_len <= kTopkThreads * 4)
    hipLaunchKernelGGL((topk_kernel<A, B, 4>), grid, blk, 0, s, in, out, seg_len, k);
  else if (seg_len <= kTopkThreads * 8)
    hipLaunchKernelGGL((topk_kernel<A, B, 8>), grid, blk, 0, s, in, out, seg_len, k);
  else
    hipLaunchKernelGGL((topk_kernel<A, B, 16>), grid, blk, 0, s, in, out, seg_len, k);
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
    // segments of at least 2k columns, so each stage shrinks the row
    const int seg = std::min(kSegMax, std::max(n <= 4 * kSegMax ? 4096 : kSegMax, 4 * k));
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
  if (p.seg[p.stages - 1] > kSegMax) return hipErrorInvalidValue;
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
