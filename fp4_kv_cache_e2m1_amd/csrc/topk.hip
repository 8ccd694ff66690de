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
// is 64 consecutive columns. At decode sizes (a few rows) latency, not bandwidth, is the cost, so
// the selection is a short chain of phases with one barrier each:
//   0. all loads of the segment are issued at once (no per-element branches); the number of
//      valid columns and of non-empty lane groups and the key range come from one reduction;
//   1. pruning bound: the EPL columns of a lane form a group (two groups, its halves, when k
//      exceeds half the lanes); at least k group maxima are >= the k-th largest group maximum,
//      so the k-th best column is too. A histogram of the group maxima gives a lower edge L of
//      that maximum's bin and every column below L is dropped (typically ~95% of them). When
//      they fit, each wave packs its survivors in column order into 4 registers per lane;
//   2. MSB-first radix select over the survivors with digits of up to 12 bits, starting below
//      the common prefix of the candidates' key range (so that close keys still spread over the
//      bins; LDS atomics on one bin serialize), stopping once the threshold bin is taken whole.
//      Each wave locates the bin itself from a 64-bin coarse histogram and the fine bins under
//      it, and three histogram buffers rotate, so a pass needs a single barrier;
//   3. compaction in ascending column order with ballot + mbcnt per register row (no shuffles),
//      so the result is deterministic.
// With many rows (prefill) one workgroup per row keeps the chip busy, so rows up to 40960 columns
// are one segment; such whole rows run a lean form that fits two workgroups on a CU (a row's loads
// are exposed latency otherwise: every CU loads its row at the same time, then selects while HBM
// idles). With few rows (decode) rows longer than 32768 columns are split for
// parallelism: each segment's k best (key, position) pairs go to scratch, and the same kernel
// selects again over those candidates; the global k best always survive their segment.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace csa2 {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kSegMax = 40960;        // columns per workgroup: up to 40 per lane
constexpr int kSegSplit = 16384;      // segment length when a row is split over workgroups
constexpr int kSegSingle = 32768;     // few rows: longest row kept in one workgroup
constexpr int kHistBins = 4096;       // largest radix digit: 12 bits
constexpr int kCoarse = 64;           // coarse bins: the top 6 bits of a digit
constexpr int kCompact = 4 * kTopkThreads;  // pruning survivors packed 4 per lane

enum TopkSrc { kSrcScores = 0, kSrcMapped = 1, kSrcCand = 2, kSrcGather = 3, kSrcBlocks = 4 };
enum TopkDst { kDstIdx = 0, kDstExpand = 1, kDstCand = 2 };

struct TopkArgs {
  const float* scores;         // [rows, ld] (kSrcScores, kSrcMapped)
  const int32_t* map;          // [rows, ld] column -> position, -1 = empty (kSrcMapped, kSrcGather)
  const float* gscores;        // kSrcGather, kSrcBlocks: scores [rows, gld] indexed by position
  int64_t gld;
  const int32_t* blocks;       // kSrcBlocks (LDS): column c is position blocks[c / 8] * 8 + c % 8
  int32_t* sel;                // kDstExpand, nullable (LDS): the selected blocks in output order
  const uint32_t* ckeys;       // [rows, ld] candidate keys (kSrcCand)
  const int32_t* cpos;         // [rows, ld] candidate positions, -1 = empty (kSrcCand)
  const int32_t* n_valid;      // nullable: columns valid per row = ceil(n_valid[r] / valid_div)
  int valid_div;
  int n_in;                    // columns per row
  int64_t ld;                  // row stride of the inputs
  int32_t* idx;                // [rows, k * (expand or 1)] (kDstIdx, kDstExpand)
  int expand;                  // kDstExpand: each selected block b becomes b*expand .. +expand-1
  const int32_t* exp_nvis;     // nullable, expanded positions >= n_vis[r] become -1 (also kSrcBlocks)
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

// Bin of the krem-th largest entry of a histogram, found by each wave on its own (no barrier):
// lane l reads coarse bin 63 - l (the top 6 bits of the digit), a prefix scan over the lanes
// picks the coarse bin holding the krem-th entry, and the 2^fshift fine bins inside it are
// scanned the same way. Returns the digit d, the count in bins above d and the count in d.
// Every wave reads the same histograms, so every wave gets the same answer.
CSA2_DEV void find_bin(const uint32_t* fine, const uint32_t* coarse, int fshift, int krem, int& d, int& above,
                       int& cnt) {
  const int lane = threadIdx.x & 63;
  const int hc = (int)coarse[63 - lane];
  const int ic = wave_incl_scan(hc);
  const uint64_t mc = __ballot(ic >= krem);
  const int lc = mc ? (int)__builtin_ctzll(mc) : 0;
  const int cb = 63 - lc;
  const int ab = __builtin_amdgcn_readlane(ic - hc, lc);
  const int nf = 1 << fshift;
  const int hf = lane < nf ? (int)fine[cb * nf + nf - 1 - lane] : 0;
  const int inf = wave_incl_scan(hf);
  const uint64_t mf = __ballot(ab + inf >= krem);
  const int lf = mf ? (int)__builtin_ctzll(mf) : 0;
  d = cb * nf + nf - 1 - lf;
  above = ab + __builtin_amdgcn_readlane(inf - hf, lf);
  cnt = __builtin_amdgcn_readlane(hf, lf);
}

// Histograms of one selection phase: 12-bit (or 8-bit) digit counts and their 64 coarse bins.
struct alignas(16) TopkHist {
  uint32_t fine[kHistBins];
  uint32_t coarse[kCoarse];
};

CSA2_DEV void clear_hist(TopkHist& h) {
  reinterpret_cast<uint4*>(h.fine)[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
  static_assert(kHistBins == 4 * kTopkThreads, "one 16-byte clear per thread");
  if (threadIdx.x < kCoarse) h.coarse[threadIdx.x] = 0u;
}

// Called by the lanes that hold a candidate (divergent). LDS atomics on one address serialize;
// with AGG (dense candidates, whose coarse bins are few) the lanes of a wave that share the first
// such lane's coarse bin add their count in one atomic.
template <bool AGG>
CSA2_DEV void hist_add(TopkHist& h, uint32_t digit, int fshift) {
  atomicAdd(&h.fine[digit], 1u);
  const uint32_t cb = digit >> fshift;
  if (AGG) {
    const uint32_t c0 = __builtin_amdgcn_readfirstlane(cb);
    const uint64_t m = __ballot(cb == c0);
    if (cb != c0) atomicAdd(&h.coarse[cb], 1u);
    else if (lanes_below(m) == 0) atomicAdd(&h.coarse[c0], (uint32_t)__popcll(m));
  } else {
    atomicAdd(&h.coarse[cb], 1u);
  }
}

// Maximum over the 64 lanes of a wave (every lane gets it).
CSA2_DEV uint32_t wave_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Bits below the common prefix of two keys (0 when equal), and the mask of that prefix.
CSA2_DEV int low_bits(uint32_t lo, uint32_t hi) {
  const uint32_t x = lo ^ hi;
  return x ? 32 - __builtin_clz(x) : 0;
}
CSA2_DEV uint32_t prefix_mask(int rb) { return rb >= 32 ? 0u : ~0u << rb; }

// Shared memory of one selection. Three histogram buffers rotate so that each phase needs one
// barrier: a phase fills its buffer, clears the one two phases ahead, and every wave then reads
// its own copy of the answer; the buffer cleared in a phase was last read before the previous
// phase's barrier.
template <int NLIST, typename PosT = int32_t>
struct TopkSmem {
  TopkHist hist[3];
  uint32_t list_key[NLIST];      // survivors of the pruning bound, in column order
  PosT list_pos[NLIST];           // uint16_t: column within the segment
  int totals[4];                 // valid columns, non-empty lane / half / quarter groups
  uint32_t kmax, kmin;           // largest and smallest key
  uint32_t gmin[3];              // smallest non-empty group maximum (whole, half, quarter groups)
  int wcnt[kTopkWaves][2];
};

// Radix select, compaction and output over R register rows per lane. Row i of lane l in wave w is
// the (w, i, l)-th candidate in column order; key 0 marks an empty slot. Positions are pos[i] when
// EXPL, else implied as col0 + 64 i + lane. kk of the candidates are taken; `sel` says a
// threshold must be found (kk < number of candidates), and every candidate key lies in
// [lo0, hi0]. The digits start below the common prefix of lo0 and hi0: candidates that survived
// selection so far are close in value, and a digit over bits they all share would send them to
// a few bins, whose LDS atomics then serialize. DENSE: most register slots hold candidates. The
// first radix pass fills hist[1] (clear on entry) and clears hist[2].
template <int SRC, int DST, int R, bool EXPL, bool DENSE, int NPOS, int NLIST, typename PosT>
CSA2_DEV void topk_finish(const TopkArgs& a, TopkSmem<NLIST, PosT>& sm, uint32_t (&key)[R], const int32_t (&pos)[NPOS],
                          int col0, int k, int kk, bool sel, uint32_t lo0, uint32_t hi0, int r, int seg) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // loaded now so that no store of the output waits on it (loads and stores share one counter)
  const int exp_nv = DST == kDstExpand ? (a.exp_nvis ? a.exp_nvis[r] : a.exp_limit) : 0;
  // ---- threshold range [lo, hi] and how many of it to take (krem) ----
  uint32_t lo = 1, hi = 0xFFFFFFFFu;
  int krem = kk;
  if (sel) {
    // MSB-first radix select over the rb bits below the common prefix, up to 12 bits a pass;
    // pass p fills buffer (p + 1) % 3 and clears (p + 2) % 3
    int rb = low_bits(lo0, hi0);
    uint32_t mask = prefix_mask(rb);
    uint32_t prefix = hi0 & mask;
    for (int pass = 0; pass < 3 && rb > 0; ++pass) {
      const int bits = min(12, rb);
      const int shift = rb - bits;
      const int fshift = max(0, bits - 6);
      const uint32_t dmask = (1u << bits) - 1u;
      TopkHist& h = sm.hist[(pass + 1) % 3];
      if (DENSE && pass == 0) {
#pragma unroll
        for (int i = 0; i < R; ++i)
          if (key[i] != 0) hist_add<true>(h, (key[i] >> shift) & dmask, fshift);
      } else {
#pragma unroll
        for (int i = 0; i < R; ++i)
          if (key[i] != 0 && (key[i] & mask) == prefix) hist_add<false>(h, (key[i] >> shift) & dmask, fshift);
      }
      clear_hist(sm.hist[(pass + 2) % 3]);
      __syncthreads();
      int d, ab, c;
      find_bin(h.fine, h.coarse, fshift, krem, d, ab, c);
      krem -= ab;
      prefix |= (uint32_t)d << shift;
      mask |= dmask << shift;
      rb -= bits;
      if (c == krem) break;
    }
    lo = prefix;
    hi = prefix | ~mask;
  }

  // ---- compaction in ascending column order ----
  int gt = 0, eq = 0;
  if (kk > 0) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      gt += __popcll(__ballot(key[i] > hi));
      eq += __popcll(__ballot(key[i] >= lo && key[i] <= hi));
    }
  }
  if (lane == 0) { sm.wcnt[wave][0] = gt; sm.wcnt[wave][1] = eq; }
  __syncthreads();
  // output offset of this wave: the waves before it take all their keys above the threshold
  // range and, in column order, the first krem keys inside it
  int out_pos = 0, eq_before = 0;
  {
    const int g = lane < kTopkWaves ? sm.wcnt[lane][0] : 0;
    const int e = lane < kTopkWaves ? sm.wcnt[lane][1] : 0;
    const int eb = wave_incl_scan(e) - e;
    const int take = g + max(0, min(e, krem - eb));
    const int tb = wave_incl_scan(take) - take;
    out_pos = __builtin_amdgcn_readlane(tb, wave);
    eq_before = __builtin_amdgcn_readlane(eb, wave);
  }
  if (kk > 0) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const uint32_t kv = key[i];
      const bool is_gt = kv > hi;                  // lo >= 1, so key 0 is never taken
      const bool is_eq = kv >= lo && kv <= hi;
      const uint64_t be = __ballot(is_eq);
      const bool take = is_gt || (is_eq && eq_before + lanes_below(be) < krem);
      const uint64_t bt = __ballot(take);
      if (take) {
        const int o = out_pos + lanes_below(bt);
        const int32_t p_i = EXPL ? pos[i % NPOS] : col0 + 64 * i + lane;
        if (DST == kDstIdx) {
          a.idx[(int64_t)r * k + o] = p_i;
        } else if (DST == kDstExpand) {
          if (a.sel) a.sel[o] = p_i;
          const int nv = exp_nv;
          int32_t* dst = a.idx + ((int64_t)r * k + o) * a.expand;
          if (a.expand == 8 && (reinterpret_cast<uintptr_t>(a.idx) & 15) == 0) {  // HSI block: two 16-byte stores
            const int p0 = p_i * 8;
            const int4 lo4 = make_int4(p0 < nv ? p0 : -1, p0 + 1 < nv ? p0 + 1 : -1, p0 + 2 < nv ? p0 + 2 : -1,
                                       p0 + 3 < nv ? p0 + 3 : -1);
            const int4 hi4 = make_int4(p0 + 4 < nv ? p0 + 4 : -1, p0 + 5 < nv ? p0 + 5 : -1,
                                       p0 + 6 < nv ? p0 + 6 : -1, p0 + 7 < nv ? p0 + 7 : -1);
            reinterpret_cast<int4*>(dst)[0] = lo4;
            reinterpret_cast<int4*>(dst)[1] = hi4;
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
  for (int o = kk + (int)threadIdx.x; o < k; o += kTopkThreads) {
    if (DST == kDstIdx) {
      a.idx[(int64_t)r * k + o] = -1;
    } else if (DST == kDstExpand) {
      if (a.sel) a.sel[o] = -1;
      for (int v = 0; v < a.expand; ++v) a.idx[((int64_t)r * k + o) * a.expand + v] = -1;
    } else {
      a.okeys[r * a.old + (int64_t)seg * k + o] = 0u;
      a.opos[r * a.old + (int64_t)seg * k + o] = -1;
    }
  }
}

// Selection of the k best columns of segment `seg` of row r by the whole workgroup.
template <int SRC, int DST, int EPL, bool LEAN = false, int NLIST, typename PosT>
CSA2_DEV void topk_segment(const TopkArgs& a, int seg_len, int k, TopkSmem<NLIST, PosT>& sm, int r, int seg) {
  static_assert(!LEAN || SRC == kSrcScores, "lean form reloads scores");
  static_assert(sizeof(PosT) == 4 || SRC == kSrcScores, "16-bit list positions are segment columns");
  // pruning survivors are packed when there are more than 4 registers per lane to gain from it
  constexpr bool kPack = EPL > 4;
  static_assert(!kPack || NLIST >= kCompact, "room for the packed survivors");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c0 = seg * seg_len;
  const int n = min(seg_len, a.n_in - c0);
  int lim = n;                              // valid columns of this segment: [0, lim)
  if (SRC != kSrcCand && a.n_valid) {
    const int nv_cols = (a.n_valid[r] + a.valid_div - 1) / a.valid_div;
    lim = max(0, min(n, nv_cols - c0));
  }
  const int wbase = wave * 64 * EPL;        // this wave's first column (segment-relative)
  const int64_t rowoff = (int64_t)r * a.ld + c0;
  const int gnv = SRC == kSrcBlocks ? (a.exp_nvis ? a.exp_nvis[r] : a.exp_limit) : 0;

  // ---- 0. load: register i of lane l is column wbase + 64 i + l ----
  constexpr int NP = SRC == kSrcScores ? 1 : EPL;   // positions are kept only when not implied
  uint32_t key[EPL];
  int32_t pos[NP];
  float sv[EPL];
  // the segment's valid columns as a buffer: loads past lim return 0 (and are masked below)
  const uint64_t ra = SRC == kSrcScores ? reinterpret_cast<uint64_t>(a.scores + rowoff) : 0u;
  const uint32_t ra_lo = __builtin_amdgcn_readfirstlane((uint32_t)ra), ra_hi = __builtin_amdgcn_readfirstlane((uint32_t)(ra >> 32));
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void*>(((uint64_t)ra_hi << 32) | ra_lo), 0, SRC == kSrcScores ? max(lim, 0) * 4 : 0, 0x00020000);
  const int vo = (wbase + lane) * 4;
  if (SRC == kSrcScores && lim > 0) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) sv[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, vo + 256 * i, 0, 0));
  } else if (lim > 0) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = min(wbase + 64 * i + lane, lim - 1);  // clamped: every load is in bounds
      if (SRC == kSrcCand) {
        key[i] = a.ckeys[rowoff + e];
        pos[i % NP] = a.cpos[rowoff + e];
      } else if (SRC == kSrcGather) {
        pos[i % NP] = a.map[rowoff + e];
      } else if (SRC == kSrcBlocks) {
        const int blk = a.blocks[e >> 3];
        const int p = blk * 8 + (e & 7);
        pos[i % NP] = blk >= 0 && p < gnv ? p : -1;
      } else {
        sv[i] = a.scores[rowoff + e];
        if (SRC == kSrcMapped) pos[i % NP] = a.map[rowoff + e];
      }
    }
  }
  // the first two phases' buffers are cleared while the loads are in flight
  clear_hist(sm.hist[0]);
  clear_hist(sm.hist[1]);
  if (tid < 4) sm.totals[tid] = 0;
  if (tid == 0) {
    sm.kmax = 0u;
    sm.kmin = 0xFFFFFFFFu;
    sm.gmin[0] = 0xFFFFFFFFu;
    sm.gmin[1] = 0xFFFFFFFFu;
    sm.gmin[2] = 0xFFFFFFFFu;
  }
  __syncthreads();
  if (lim > 0) {
    if (SRC == kSrcGather || SRC == kSrcBlocks) {
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
      if (SRC == kSrcGather || SRC == kSrcBlocks) ok = ok && pos[i % NP] < a.gld;
      if (SRC != kSrcCand) key[i] = score_key(sv[i]);
      key[i] = ok ? key[i] : 0u;
    }
  } else {
#pragma unroll
    for (int i = 0; i < EPL; ++i) key[i] = 0u;
  }
  // group maxima: a lane's EPL columns (gm), its two halves (gh[0], gh[1]) and, for pool block
  // selections (k of the order of the lane count or more), its four quarters (gq)
  constexpr int HALF = EPL >= 8 ? EPL / 2 : EPL;
  constexpr bool kQuarters = DST == kDstExpand && EPL >= 16;
  constexpr int QTR = EPL / 4;
  int cnt = 0;
  uint32_t gh[2] = {0u, 0u}, mn = 0u;       // mn: complement of the smallest key
  uint32_t gq[kQuarters ? 4 : 1] = {};
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    cnt += key[i] != 0;
    gh[i / HALF > 0] = max(gh[i / HALF > 0], key[i]);
    if constexpr (kQuarters) gq[min(3, i / QTR)] = max(gq[min(3, i / QTR)], key[i]);
    mn = max(mn, key[i] ? ~key[i] : 0u);
  }
  const uint32_t gm = max(gh[0], gh[1]);
  // phase 0: counts and key range
  {
    const int wc = __builtin_amdgcn_readlane(wave_incl_scan(cnt), 63);
    const int wg = (int)__popcll(__ballot(gm != 0));
    const int wh = (int)(__popcll(__ballot(gh[0] != 0)) + __popcll(__ballot(gh[1] != 0)));
    const uint32_t wmax = wave_max(gm), wmn = wave_max(mn), wgmn = wave_max(gm ? ~gm : 0u);
    const uint32_t whmn = wave_max(max(gh[0] ? ~gh[0] : 0u, gh[1] ? ~gh[1] : 0u));
    if (lane == 0) {
      atomicAdd(&sm.totals[0], wc);
      atomicAdd(&sm.totals[1], wg);
      atomicAdd(&sm.totals[2], wh);
      atomicMax(&sm.kmax, wmax);
      atomicMin(&sm.kmin, ~wmn);
      atomicMin(&sm.gmin[0], ~wgmn);
      atomicMin(&sm.gmin[1], ~whmn);
    }
    if constexpr (kQuarters) {
      int wq = 0;
      uint32_t qmn = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        wq += (int)__popcll(__ballot(gq[j] != 0));
        qmn = max(qmn, gq[j] ? ~gq[j] : 0u);
      }
      const uint32_t wqmn = wave_max(qmn);
      if (lane == 0) {
        atomicAdd(&sm.totals[3], wq);
        atomicMin(&sm.gmin[2], ~wqmn);
      }
    }
  }
  __syncthreads();
  const int total = sm.totals[0];
  const uint32_t kmax = sm.kmax, kmin = sm.kmin;
  const int kk = min(k, total);
  const bool sel = kk > 0 && kk < total;
  // half groups when kk is more than half the lane groups (the kk-th largest of the lane group
  // maxima would be a weak bound), quarter groups when it is more than half the half groups too
  const bool halves = EPL >= 8 && 2 * kk > sm.totals[1];
  const bool quarters = kQuarters && halves && 2 * kk > sm.totals[2];
  const int level = quarters ? 2 : (halves ? 1 : 0);
  const int ng = sm.totals[level + 1];

  // lean form: the keys are not kept past the packing pass; the paths that need all of them read
  // the row again (floor_key: the pruning bound, or 1 for every valid column)
  auto reload = [&](uint32_t floor_key) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) sv[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, vo + 256 * i, 0, 0));
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const uint32_t kv = wbase + 64 * i + lane < lim ? score_key(sv[i]) : 0u;
      key[i] = kv >= floor_key ? kv : 0u;
    }
  };
  // 1. pruning bound: at least kk (disjoint) group maxima are >= the kk-th largest group maximum,
  //    so the kk-th best column is too; every column below that maximum's bin is dropped. The
  //    bins are up to 12 bits below the common prefix of the group maxima.
  if (EPL >= 4 && sel && ng >= kk) {
    const uint32_t gmin = sm.gmin[level];
    const int rb = low_bits(gmin, kmax);
    uint32_t L = kmax;                      // all group maxima equal
    if (rb > 0) {
      // 12-bit bins: when the group maxima span both signs, the top 6 bits alone would put
      // every positive one in a single bin
      const int bits = min(12, rb), shift = rb - bits, fshift = max(0, bits - 6);
      const uint32_t dm = (1u << bits) - 1u;
      if (quarters) {
        if constexpr (kQuarters) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (gq[j] != 0) hist_add<true>(sm.hist[0], (gq[j] >> shift) & dm, fshift);
        }
      } else if (halves) {
        if (gh[0] != 0) hist_add<true>(sm.hist[0], (gh[0] >> shift) & dm, fshift);
        if (gh[1] != 0) hist_add<true>(sm.hist[0], (gh[1] >> shift) & dm, fshift);
      } else {
        if (gm != 0) hist_add<true>(sm.hist[0], (gm >> shift) & dm, fshift);
      }
      __syncthreads();
      int d, ab, c;
      find_bin(sm.hist[0].fine, sm.hist[0].coarse, fshift, kk, d, ab, c);
      L = (kmax & prefix_mask(rb)) | ((uint32_t)d << shift);
    }
    L = max(L, 1u);
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (key[i] < L) key[i] = 0;
    // The survivors are usually a few percent of the columns. When they fit, they are packed in
    // column order into at most NLIST / 1024 rows per lane (4; block selections, whose bound is
    // the looser one of many small groups, have room for 8 and use 4 when every wave's
    // survivors fit 256 slots), so the passes below touch those registers, not EPL.
    if constexpr (kPack) {
      constexpr int kSlots = NLIST / kTopkWaves, kRP = kSlots / 64;
      // each wave packs its survivors, in column order, into its own kSlots slots; when no wave
      // overflows, every wave continues from its slots (the slot order keeps column order)
      int o = 0;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const bool live = key[i] != 0;
        const uint64_t m = __ballot(live);
        const int j = o + lanes_below(m);
        if (live && j < kSlots) {
          sm.list_key[wave * kSlots + j] = key[i];
          sm.list_pos[wave * kSlots + j] =
              (PosT)(SRC != kSrcScores ? pos[i % NP] : (sizeof(PosT) == 4 ? c0 : 0) + wbase + 64 * i + lane);
        }
        o += (int)__popcll(m);
      }
      if (lane == 0) sm.wcnt[wave][0] = o;
      __syncthreads();
      const int most = (int)wave_max((uint32_t)(lane < kTopkWaves ? sm.wcnt[lane][0] : 0));
      // the passes over the packed list cost in proportion to its registers, so a list that fits
      // half the slots takes the half-width form
      auto finish_packed = [&](auto rp) {
        constexpr int RP = decltype(rp)::value;
        uint32_t keyp[RP];
        int32_t posp[RP];
#pragma unroll
        for (int u = 0; u < RP; ++u) {
          const int j = 64 * u + lane;
          keyp[u] = j < o ? sm.list_key[wave * kSlots + j] : 0u;
          posp[u] = (int32_t)sm.list_pos[wave * kSlots + j] + (sizeof(PosT) == 4 ? 0 : c0);
        }
        topk_finish<SRC, DST, RP, true, false>(a, sm, keyp, posp, 0, k, kk, true, L, kmax, r, seg);
      };
      if constexpr (kRP > 4) {
        if (most <= kSlots / 2) {
          finish_packed(std::integral_constant<int, kRP / 2>{});
          return;
        }
      }
      if (most <= kSlots) {
        finish_packed(std::integral_constant<int, kRP>{});
        return;
      }
      // wcnt is rewritten only after the next barrier, which every wave reaches after reading it
    }
    if constexpr (LEAN) reload(L);
    topk_finish<SRC, DST, EPL, SRC != kSrcScores, true>(a, sm, key, pos, c0 + wbase, k, kk, true, L, kmax, r, seg);
    return;
  }
  if constexpr (LEAN) reload(1u);
  topk_finish<SRC, DST, EPL, SRC != kSrcScores, true>(a, sm, key, pos, c0 + wbase, k, kk, sel, kmin, kmax, r, seg);
}

template <int SRC, int DST, int EPL>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a, int seg_len, int k) {
  // block selections (pool) pack up to 512 survivors per wave
  __shared__ TopkSmem<(EPL > 4 ? (DST == kDstExpand ? 2 * kCompact : kCompact) : 1)> sm;
  topk_segment<SRC, DST, EPL>(a, seg_len, k, sm, blockIdx.x, blockIdx.y);
}

// Whole score rows (one segment per row, k best as indices): the lean form. Keys live in registers
// only until the pruning survivors are packed (the rare paths that need every key again read the
// row again), and list positions are 16-bit segment columns, so the kernel fits 64 registers per
// lane and 75 KB of LDS: two rows share a CU, and one row's loads run under the other's selection.
template <int EPL>
__global__ __launch_bounds__(kTopkThreads) __attribute__((amdgpu_waves_per_eu(8))) void topk_rows_kernel(
    TopkArgs a, int seg_len, int k) {
  __shared__ TopkSmem<kCompact, uint16_t> sm;
  topk_segment<kSrcScores, kDstIdx, EPL, true>(a, seg_len, k, sm, blockIdx.x, blockIdx.y);
}

// HSI Full layer in one workgroup per row: the pool (the k_blocks best blocks of the block
// maxima, expanded to positions) and then the layer's Top-K over the pool's positions, whose
// list stays in LDS between the two selections.
constexpr int kSelMax = kSegMax / 8;        // pool blocks: up to 40960 positions
template <int EPL_A, int EPL_B>
__global__ __launch_bounds__(kTopkThreads) void pool_topk_kernel(TopkArgs pa, TopkArgs pb, int k_blocks, int k) {
  __shared__ TopkSmem<2 * kCompact> sm;   // up to 512 pool-block survivors per wave
  __shared__ int32_t sel[kSelMax];
  pa.sel = sel;
  topk_segment<kSrcScores, kDstExpand, EPL_A>(pa, pa.n_in, k_blocks, sm, blockIdx.x, 0);
  __syncthreads();                            // the selected blocks are in LDS; sm is free again
  pb.blocks = sel;
  topk_segment<kSrcBlocks, kDstIdx, EPL_B>(pb, pb.n_in, k, sm, blockIdx.x, 0);
}

template <int SRC, int DST>
static hipError_t launch_one(dim3 grid, const TopkArgs& a, int seg_len, int k, hipStream_t s) {
  const dim3 blk(kTopkThreads);
  constexpr bool kRows = SRC == kSrcScores && DST == kDstIdx;
#define CSA2_TOPK_EPL(E)                                                                \
  if (seg_len <= kTopkThreads * (E)) {                                                   \
    if constexpr (kRows && (E) >= 8)                                                     \
      hipLaunchKernelGGL((topk_rows_kernel<E>), grid, blk, 0, s, a, seg_len, k);         \
    else                                                                                 \
      hipLaunchKernelGGL((topk_kernel<SRC, DST, E>), grid, blk, 0, s, a, seg_len, k);   \
    return hipGetLastError();                                                            \
  }
  // Whole score rows (prefill, one workgroup per row) take register counts in steps of 4 and the
  // 33 of a 33792-column row (32768 + 1024 entries): loads and per-register passes over register
  // rows that only repeat a row's last column are the selection's main waste at these lengths.
  CSA2_TOPK_EPL(1)
  CSA2_TOPK_EPL(2)
  CSA2_TOPK_EPL(4)
  CSA2_TOPK_EPL(8)
  if constexpr (kRows) { CSA2_TOPK_EPL(12) }
  CSA2_TOPK_EPL(16)
  if constexpr (kRows) { CSA2_TOPK_EPL(20) }
  CSA2_TOPK_EPL(24)
  if constexpr (kRows) { CSA2_TOPK_EPL(28) }
  CSA2_TOPK_EPL(32)
  if constexpr (kRows) { CSA2_TOPK_EPL(33) CSA2_TOPK_EPL(36) }
#undef CSA2_TOPK_EPL
  if constexpr (kRows)
    hipLaunchKernelGGL((topk_rows_kernel<40>), grid, blk, 0, s, a, seg_len, k);
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
    const int single = rows >= 256 ? kSegMax : kSegSingle;
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

template <int EPL_A>
static hipError_t launch_pool_topk_b(int epl_b, dim3 grid, const TopkArgs& pa, const TopkArgs& pb, int kb, int k,
                                     hipStream_t s) {
  const dim3 blk(kTopkThreads);
  switch (epl_b) {
    case 4: hipLaunchKernelGGL((pool_topk_kernel<EPL_A, 4>), grid, blk, 0, s, pa, pb, kb, k); break;
    case 8: hipLaunchKernelGGL((pool_topk_kernel<EPL_A, 8>), grid, blk, 0, s, pa, pb, kb, k); break;
    default: hipLaunchKernelGGL((pool_topk_kernel<EPL_A, 16>), grid, blk, 0, s, pa, pb, kb, k); break;
  }
  return hipGetLastError();
}

hipError_t launch_pool_topk(const float* block_max, int64_t rows, int n_blocks, const int32_t* n_vis,
                            int pool_blocks, int32_t* pool, const float* scores, int n_max, int k, int32_t* idx,
                            hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int P = pool_blocks * 8;
  const int epl_a = (n_blocks + kTopkThreads - 1) / kTopkThreads;
  const int epl_b = (P + kTopkThreads - 1) / kTopkThreads;
  if (epl_a <= 4 || epl_a > 40 || epl_b <= 2 || epl_b > 16 || pool_blocks > kSelMax || k > P)
    return hipErrorNotSupported;
  TopkArgs pa{};
  pa.scores = block_max;
  pa.n_valid = n_vis;
  pa.valid_div = 8;
  pa.n_in = n_blocks;
  pa.ld = n_blocks;
  pa.idx = pool;
  pa.expand = 8;
  pa.exp_nvis = n_vis;
  pa.exp_limit = n_max;
  TopkArgs pb{};
  pb.gscores = scores;
  pb.gld = n_max;
  pb.n_in = P;
  pb.ld = P;
  pb.idx = idx;
  pb.exp_nvis = n_vis;
  pb.exp_limit = n_max;
  const dim3 grid((unsigned)rows);
  if (epl_a <= 8) return launch_pool_topk_b<8>(epl_b, grid, pa, pb, pool_blocks, k, s);
  if (epl_a <= 16) return launch_pool_topk_b<16>(epl_b, grid, pa, pb, pool_blocks, k, s);
  if (epl_a <= 24) return launch_pool_topk_b<24>(epl_b, grid, pa, pb, pool_blocks, k, s);
  if (epl_a <= 32) return launch_pool_topk_b<32>(epl_b, grid, pa, pb, pool_blocks, k, s);
  return launch_pool_topk_b<40>(epl_b, grid, pa, pb, pool_blocks, k, s);
}

}  // namespace csa2
