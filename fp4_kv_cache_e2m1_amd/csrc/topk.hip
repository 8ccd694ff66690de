// Top-K selection and candidate-pool expansion.
// Source: DeepSeek-V4.1-Flash walkthrough (wkq9411.github.io), 一(四) (each query keeps its
// Top-K entries) and 一(四)2 (the highest-scoring blocks are chosen and the positions they
// cover become the candidate pool).
//
// Order: score descending, then position ascending (so ties go to the lower position). Scores
// become order-preserving 32-bit keys (key 0 = not a candidate; -0 and +0 share a key).
//
// One workgroup (16 waves) selects the k best of a segment of up to 40960 columns. Lane l of
// wave w holds columns 64*(w*EPL + i) + l (i < EPL) in registers, so a wave's i-th register row
// is 64 consecutive columns. The selection is a short chain of barrier-separated phases, each
// a few LDS operations, because at decode sizes (a few rows) latency, not bandwidth, is the cost:
//   0. all loads of the segment are issued at once (no per-element branches); the count of
//      valid columns and of non-empty lane groups come out of one block reduction;
//   1. pruning bound: the EPL columns of a lane form a group; at least k group maxima are >= the
//      k-th largest group maximum, so the k-th best column is too. A 12-bit histogram of the
//      group maxima gives a lower edge L of that maximum's bin and every column below L is
//      dropped (typically ~95% of them);
//   2. MSB-first radix select over the survivors with 12, 12 and 8-bit digits, stopping as soon
//      as the threshold bin is taken whole. Two histogram buffers alternate, so the next one is
//      cleared while the current one fills and no phase needs an extra barrier;
//   3. compaction in ascending column order with ballot + mbcnt per register row (no shuffles),
//      so the result is deterministic.
// With many rows (prefill) one workgroup per row keeps the chip busy, so rows up to 40960 columns
// are one segment. With few rows (decode) rows longer than 16384 columns are split for
// parallelism: each segment's k best (key, position) pairs go to scratch, and the same kernel
// selects again over those candidates; the global k best always survive their segment.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace csa2 {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kSegMax = 40960;        // columns per workgroup: up to 40 per lane
constexpr int kSegSplit = 16384;      // segment length when a row is split over workgroups
constexpr int kHistBins = 4096;       // largest radix digit: 12 bits

enum TopkSrc { kSrcScores = 0, kSrcMapped = 1, kSrcCand = 2, kSrcGather = 3 };
enum TopkDst { kDstIdx = 0, kDstExpand = 1, kDstCand = 2 };

struct TopkArgs {
  const float* scores;         // [rows, ld] (kSrcScores, kSrcMapped)
  const int32_t* map;          // [rows, ld] column -> position, -1 = empty (kSrcMapped, kSrcGather)
  const float* gscores;        // kSrcGather: scores [rows, gld] indexed by position
  int64_t gld;
  const uint32_t* ckeys;       // [rows, ld] candidate keys (kSrcCand)
  const int32_t* cpos;         // [rows, ld] candidate positions, -1 = empty (kSrcCand)
  const int32_t* n_valid;      // nullable: columns valid per row = ceil(n_valid[r] / valid_div)
  int valid_div;
  int n_in;                    // columns per row
  int64_t ld;                  // row stride of the inputs
  int32_t* idx;                // [rows, k * (expand or 1)] (kDstIdx, kDstExpand)
  int expand;                  // kDstExpand: each selected block b becomes b*expand .. +expand-1
  const int32_t* exp_nvis;     // nullable, expanded positions >= n_vis[r] become -1
  int exp_limit;               // used instead of exp_nvis when it is null
  uint32_t* okeys;             // kDstCand: [rows, old]
  int32_t* opos;
  int64_t old;
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

// Block-wide sum (every thread gets it). One barrier; red[] must not be rewritten before the
// next barrier.
CSA2_DEV int block_sum(int v, int* red) {
  v = __builtin_amdgcn_readlane(wave_incl_scan(v), 63);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) t += red[w];
  return t;
}

// Given a filled histogram of nbins bins, find the bin d holding the krem-th largest entry:
// count above d < krem <= count above d + hist[d]. Returns (d, above, hist[d]) to every
// thread. Two barriers; info[] is read after the second and rewritten only after the first
// barrier of the next call.
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
}

template <int SRC, int DST, int EPL>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a, int seg_len, int k) {
  __shared__ uint32_t hist[2][kHistBins];
  __shared__ int red[kTopkWaves];
  __shared__ int info[4];
  __shared__ int wcnt[kTopkWaves][2];

  const int r = blockIdx.x, seg = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c0 = seg * seg_len;
  const int n = min(seg_len, a.n_in - c0);
  int lim = n;                              // valid columns of this segment: [0, lim)
  if (SRC != kSrcCand && a.n_valid) {
    const int nv_cols = (a.n_valid[r] + a.valid_div - 1) / a.valid_div;
    lim = max(0, min(n, nv_cols - c0));
  }
  const int wbase = wave * 64 * EPL;        // this wave's first column (segment-relative)
  const int64_t rowoff = (int64_t)r * a.ld + c0;

  // ---- 0. load: register i of lane l is column wbase + 64 i + l ----
  constexpr int NP = SRC == kSrcScores ? 1 : EPL;   // positions are kept only when not implied
  uint32_t key[EPL];
  int32_t pos[NP];
  if (lim > 0) {
    float sv[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = min(wbase + 64 * i + lane, lim - 1);  // clamped: every load is in bounds
      if (SRC == kSrcCand) {
        key[i] = a.ckeys[rowoff + e];
        pos[i % NP] = a.cpos[rowoff + e];
      } else if (SRC == kSrcGather) {
        pos[i % NP] = a.map[rowoff + e];
      } else {
        sv[i] = a.scores[rowoff + e];
        if (SRC == kSrcMapped) pos[i % NP] = a.map[rowoff + e];
      }
    }
    if (SRC == kSrcGather) {
      // scores of the listed positions (clamped into the row: every load is in bounds)
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        sv[i] = a.gscores[(int64_t)r * a.gld + min(max(pos[i % NP], 0), (int)a.gld - 1)];
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = wbase + 64 * i + lane;
      bool ok = e < lim;
      if (SRC != kSrcScores) ok = ok && pos[i % NP] >= 0;
      if (SRC == kSrcGather) ok = ok && pos[i % NP] < a.gld;
      if (SRC != kSrcCand) key[i] = score_key(sv[i]);
      key[i] = ok ? key[i] : 0u;
    }
  } else {
#pragma unroll
    for (int i = 0; i < EPL; ++i) key[i] = 0u;
  }
  int cnt = 0;
  uint32_t gm = 0;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    cnt += key[i] != 0;
    gm = max(gm, key[i]);
  }
  for (int i = tid; i < kHistBins; i += kTopkThreads) hist[0][i] = 0;
  // valid columns (<= 16384) in the low 16 bits, non-empty groups (<= 1024) above
  const int packed = block_sum(cnt | ((gm != 0) << 16), red);
  const int total = packed & 0xFFFF, ng = packed >> 16;
  const int kk = min(k, total);

  // ---- threshold range [lo, hi] and how many of it to take (krem) ----
  uint32_t lo = 1, hi = 0xFFFFFFFFu;
  int krem = kk;
  int cur = 0;                              // histogram buffer filled next
  if (kk > 0 && kk < total) {
    // 1. pruning bound from the per-lane group maxima (needs >= k non-empty groups)
    if (EPL >= 4 && ng >= kk) {
      if (gm != 0) atomicAdd(&hist[0][gm >> 20], 1u);
      for (int i = tid; i < kHistBins; i += kTopkThreads) hist[1][i] = 0;
      __syncthreads();
      int d, ab, c;
      find_bin(hist[0], kHistBins, kk, red, info, d, ab, c);
      const uint32_t L = (uint32_t)d << 20;
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (key[i] < L) key[i] = 0;
      cur = 1;
    }
    // 2. radix select over the survivors (the buffer `cur` is clear)
    uint32_t prefix = 0, mask = 0;
    constexpr int kShift[3] = {20, 8, 0};
    constexpr int kBits[3] = {12, 12, 8};
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = kShift[pass];
      const uint32_t dmask = (1u << kBits[pass]) - 1u;
      uint32_t* h = hist[cur];
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (key[i] != 0 && (key[i] & mask) == prefix) atomicAdd(&h[(key[i] >> shift) & dmask], 1u);
      for (int i = tid; i < kHistBins; i += kTopkThreads) hist[cur ^ 1][i] = 0;
      __syncthreads();
      int d, ab, c;
      find_bin(h, 1 << kBits[pass], krem, red, info, d, ab, c);
      krem -= ab;
      prefix |= (uint32_t)d << shift;
      mask |= dmask << shift;
      cur ^= 1;
      if (c == krem) break;
    }
    lo = prefix;
    hi = prefix | ~mask;
  }

  // ---- 3. compaction in ascending column order ----
  int gt = 0, eq = 0;
  if (kk > 0) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      gt += __popcll(__ballot(key[i] > hi));
      eq += __popcll(__ballot(key[i] >= lo && key[i] <= hi));
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
      const bool is_gt = kv > hi;                  // lo >= 1, so key 0 is never taken
      const bool is_eq = kv >= lo && kv <= hi;
      const uint64_t be = __ballot(is_eq);
      const bool take = is_gt || (is_eq && eq_before + lanes_below(be) < krem);
      const uint64_t bt = __ballot(take);
      if (take) {
        const int o = out_pos + lanes_below(bt);
        const int32_t p_i = SRC == kSrcScores ? c0 + wbase + 64 * i + lane : pos[i % NP];
        if (DST == kDstIdx) {
          a.idx[(int64_t)r * k + o] = p_i;
        } else if (DST == kDstExpand) {
          const int nv = a.exp_nvis ? a.exp_nvis[r] : a.exp_limit;
          int32_t* dst = a.idx + ((int64_t)r * k + o) * a.expand;
          if (a.expand == 8 && (reinterpret_cast<uintptr_t>(a.idx) & 15) == 0) {  // HSI block: two 16-byte stores
            const int p0 = p_i * 8;
            const int4 lo = make_int4(p0 < nv ? p0 : -1, p0 + 1 < nv ? p0 + 1 : -1, p0 + 2 < nv ? p0 + 2 : -1,
                                      p0 + 3 < nv ? p0 + 3 : -1);
            const int4 hi = make_int4(p0 + 4 < nv ? p0 + 4 : -1, p0 + 5 < nv ? p0 + 5 : -1, p0 + 6 < nv ? p0 + 6 : -1,
                                      p0 + 7 < nv ? p0 + 7 : -1);
            reinterpret_cast<int4*>(dst)[0] = lo;
            reinterpret_cast<int4*>(dst)[1] = hi;
          } else {
            for (int v = 0; v < a.expand; ++v) {
              const int p = p_i * a.expand + v;
              dst[v] = p < nv ? p : -1;
            }
          }
        } else {
          a.okeys[r * a.old + (int64_t)seg * k + o] = kv;
          a.opos[r * a.old + (int64_t)seg * k + o] = p_i;
        }
      }
      out_pos += __popcll(bt);
      eq_before += __popcll(be);
    }
  }
  // ---- padding ----
  for (int o = kk + tid; o < k; o += kTopkThreads) {
    if (DST == kDstIdx) {
      a.idx[(int64_t)r * k + o] = -1;
    } else if (DST == kDstExpand) {
      for (int v = 0; v < a.expand; ++v) a.idx[((int64_t)r * k + o) * a.expand + v] = -1;
    } else {
      a.okeys[r * a.old + (int64_t)seg * k + o] = 0u;
      a.opos[r * a.old + (int64_t)seg * k + o] = -1;
    }
  }
}

template <int SRC, int DST>
static hipError_t launch_one(dim3 grid, const TopkArgs& a, int seg_len, int k, hipStream_t s) {
  const dim3 blk(kTopkThreads);
  if (seg_len <= kTopkThreads * 1)
    hipLaunchKernelGGL((topk_kernel<SRC, DST, 1>), grid, blk, 0, s, a, seg_len, k);
  else if (seg_len <= kTopkThreads * 2)
    hipLaunchKernelGGL((topk_kernel<SRC, DST, 2>), grid, blk, 0, s, a, seg_len, k);
  else if (seg_len <= kTopkThreads * 4)
    hipLaunchKernelGGL((topk_kernel<SRC, DST, 4>), grid, blk, 0, s, a, seg_len, k);
  else if (seg_len <= kTopkThreads * 8)
    hipLaunchKernelGGL((topk_kernel<SRC, DST, 8>), grid, blk, 0, s, a, seg_len, k);
  else if (seg_len <= kTopkThreads * 16)
    hipLaunchKernelGGL((topk_kernel<SRC, DST, 16>), grid, blk, 0, s, a, seg_len, k);
  else if (seg_len <= kTopkThreads * 24)
    hipLaunchKernelGGL((topk_kernel<SRC, DST, 24>), grid, blk, 0, s, a, seg_len, k);
  else if (seg_len <= kTopkThreads * 32)
    hipLaunchKernelGGL((topk_kernel<SRC, DST, 32>), grid, blk, 0, s, a, seg_len, k);
  else
    hipLaunchKernelGGL((topk_kernel<SRC, DST, 40>), grid, blk, 0, s, a, seg_len, k);
  return hipGetLastError();
}

template <int SRC>
static hipError_t launch_src(dim3 grid, const TopkArgs& a, bool last, int seg_len, int k, hipStream_t s) {
  if (!last) return launch_one<SRC, kDstCand>(grid, a, seg_len, k, s);
  if (a.expand > 0) return launch_one<SRC, kDstExpand>(grid, a, seg_len, k, s);
  return launch_one<SRC, kDstIdx>(grid, a, seg_len, k, s);
}

// Plan of segment sizes: returns the number of stages and fills seg lengths / segment counts.
struct TopkPlan {
  int stages;
  int seg[8];
  int nseg[8];
  int n_in[8];
};

static TopkPlan make_plan(int64_t rows, int n_cols, int k) {
  TopkPlan p{};
  int n = n_cols;
  int st = 0;
  while (true) {
    p.n_in[st] = n;
    // many rows: one workgroup per row is enough parallelism; few rows: split long rows
    const int single = rows >= 256 ? kSegMax : kSegSplit;
    if (n <= single || st == 7) {
      p.seg[st] = n;
      p.nseg[st] = 1;
      p.stages = st + 1;
      return p;
    }
    // segments of at least 2k columns, so each stage shrinks the row
    const int seg = std::min(kSegSplit, std::max(n <= 4 * kSegSplit ? 4096 : kSegSplit, 4 * k));
    p.seg[st] = seg;
    p.nseg[st] = (n + seg - 1) / seg;
    n = p.nseg[st] * k;
    ++st;
  }
}

size_t topk_workspace(int64_t rows, int n_cols, int k) {
  const TopkPlan p = make_plan(rows, n_cols, k);
  size_t largest = 0;
  for (int st = 0; st + 1 < p.stages; ++st)
    largest = std::max(largest, (size_t)rows * p.nseg[st] * k * 8);
  largest = (largest + 255) & ~(size_t)255;
  return 2 * largest;
}

static hipError_t run_topk(const float* scores, int64_t rows, int n_cols, const int32_t* n_valid,
                           int valid_div, const int32_t* col_to_pos, int64_t gather_ld, int k, int32_t* idx,
                           int expand_block, const int32_t* expand_n_vis, int expand_limit, void* ws,
                           hipStream_t s) {
  if (rows == 0 || k == 0) return hipSuccess;
  const TopkPlan p = make_plan(rows, n_cols, k);
  if (p.seg[p.stages - 1] > kSegMax) return hipErrorInvalidValue;
  size_t half = 0;
  for (int st = 0; st + 1 < p.stages; ++st) half = std::max(half, (size_t)rows * p.nseg[st] * k * 8);
  half = (half + 255) & ~(size_t)255;
  uint8_t* wsb = static_cast<uint8_t*>(ws);

  TopkArgs a{};
  a.scores = scores;
  a.map = col_to_pos;
  a.gscores = scores;
  a.gld = gather_ld;
  a.n_valid = n_valid;
  a.valid_div = valid_div > 0 ? valid_div : 1;
  a.n_in = n_cols;
  a.ld = n_cols;
  a.idx = idx;
  a.expand = expand_block;
  a.exp_nvis = expand_n_vis;
  a.exp_limit = expand_limit;
  for (int st = 0; st < p.stages; ++st) {
    const bool last = st + 1 == p.stages;
    dim3 grid((unsigned)rows, (unsigned)p.nseg[st]);
    if (!last) {
      uint8_t* buf = wsb + (st & 1) * half;
      const size_t cnt = (size_t)rows * p.nseg[st] * k;
      a.okeys = reinterpret_cast<uint32_t*>(buf);
      a.opos = reinterpret_cast<int32_t*>(buf + cnt * 4);
      a.old = (int64_t)p.nseg[st] * k;
    }
    hipError_t e;
    if (st > 0) e = launch_src<kSrcCand>(grid, a, last, p.seg[st], k, s);
    else if (gather_ld > 0) e = launch_src<kSrcGather>(grid, a, last, p.seg[st], k, s);
    else if (col_to_pos) e = launch_src<kSrcMapped>(grid, a, last, p.seg[st], k, s);
    else e = launch_src<kSrcScores>(grid, a, last, p.seg[st], k, s);
    if (e != hipSuccess) return e;
    if (!last) {
      // the next stage reads this stage's candidates
      a.ckeys = a.okeys;
      a.cpos = a.opos;
      a.n_valid = nullptr;
      a.n_in = (int)a.old;
      a.ld = a.old;
    }
  }
  return hipSuccess;
}

hipError_t launch_topk(const float* scores, int64_t rows, int n_cols, const int32_t* n_valid,
                       int valid_div, const int32_t* col_to_pos, int k, int32_t* idx,
                       int expand_block, const int32_t* expand_n_vis, int expand_limit, void* ws,
                       hipStream_t s) {
  return run_topk(scores, rows, n_cols, n_valid, valid_div, col_to_pos, 0, k, idx, expand_block, expand_n_vis,
                  expand_limit, ws, s);
}

hipError_t launch_topk_gather(const float* scores, int n_max, int64_t rows, const int32_t* cand, int P, int k,
                              int32_t* idx, void* ws, hipStream_t s) {
  if (n_max <= 0) return hipErrorInvalidValue;
  return run_topk(scores, rows, P, nullptr, 1, cand, n_max, k, idx, 0, nullptr, 0, ws, s);
}

}  // namespace csa2
