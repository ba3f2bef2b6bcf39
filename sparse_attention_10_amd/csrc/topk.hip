// Top-k selection and page mapping on gfx950 (the "top-k + page-mapping transforms" kernel group
// of "GLM-52 Runs on RTX 4090", section "how did he do it"; the fused page-map variant is the
// README's SGLANG_NSA_FUSE_TOPK option, renning22/glm-5.2-4090, usage section).
//
// One 512-thread workgroup per query row.  The selection is exact: equal scores go to the
// lower token index, -0.0 equals +0.0, winners come out in ascending token order.  The work is
// bound by the instruction issue and LDS of the one CU, so every pass is written for few
// instructions per key.  A "key row" is one 32-bit register across a wave: 64 consecutive
// columns, one per lane.  Wave w holds RV consecutive key rows of the row's first 512*RV
// columns in registers; later columns are streamed from L2 in segments.
//   pass 1  Scores become order-preserving uint32 keys (larger score <-> larger key; key 0
//           marks a column outside the row) and are counted into an LDS histogram of 15 bits:
//           those just below the leading bits that all keys of the row share (found from the
//           keys' min and max).  A scan of per-thread bin sums, then of the chosen thread's bins, finds the
//           bin b holding the k-th largest key.  A bin holding more than kCandCap keys is
//           narrowed by 11-bit radix rounds over the keys of that bin.
//   pass 2  Per unit (one wave's key rows of the register block, or of one streamed segment)
//           the keys above the bin are counted, and the keys inside the bin (the candidates)
//           are gathered with their columns.  The exact threshold key T is then found among the
//           candidates (one key bit at a time by ballot counts when they are few), and the
//           candidates above and equal to T are added to their units' counts.
//   output  Every wave scans the units' counts (keys equal to T are taken in column order until
//           k are taken).  Each key row's winners get their output offsets from one ballot and
//           mbcnt and their columns go to an LDS list; the whole workgroup then writes the k
//           token indices and (fused page map) cache slots with coalesced stores.
#include "dsa_internal.hpp"

namespace dsa {

namespace {

#ifndef DSA_TOPK_THREADS
#define DSA_TOPK_THREADS 512
#endif
constexpr int kThreads = DSA_TOPK_THREADS;
constexpr int kWaves = kThreads / 64;
constexpr int kHistBins = 1 << 15;                       // first digit: top 15 key bits
constexpr int kBinsPerThread = kHistBins / kThreads;     // bins summed by one thread
constexpr int kBinShift = __builtin_ctz(kBinsPerThread);
constexpr int kHistStride = kBinsPerThread + 4;          // words per thread's bins (16-byte pad)
constexpr int kHistWords = kHistStride * kThreads;
constexpr int kCandCap = 4096;                           // candidates gathered into LDS
constexpr int kCandPerWave = kCandCap / kWaves;          // per-wave candidate regions
constexpr int kPtabCache = 4096;                         // page-table entries cached in LDS
constexpr int kSmallBits = 11;                           // digit of the narrowing rounds
constexpr int kSmallBins = 1 << kSmallBits;
constexpr int kTailRows = 16;                            // key rows per wave of one streamed segment
constexpr int kSegCols = 64 * kTailRows * kWaves;        // columns of one streamed segment
// units: each wave's key rows of the register block, then of each streamed segment
constexpr int kMaxUnits = kWaves * (1 + (kMaxTopkSeq + kSegCols - 1) / kSegCols);
constexpr int kUnitsPerLane = (kMaxUnits + 63) / 64;

// Word offsets in the one LDS array: the histogram in pass 1, then these regions.
constexpr int kOffCandKey = 0;                           // u32 [kCandCap]
constexpr int kOffCandCol = kOffCandKey + kCandCap;      // u32 [kCandCap]
constexpr int kOffPtab = kOffCandCol + kCandCap;         // i32 [kPtabCache]
constexpr int kOffSmall = kOffPtab + kPtabCache;         // u32 [kSmallBins]
constexpr int kOffGCnt = kOffSmall + kSmallBins;         // u32 [kMaxUnits] per-unit counts
constexpr int kOffECnt = kOffGCnt + kMaxUnits;           // u32 [kMaxUnits]
constexpr int kOffOut = kOffECnt + kMaxUnits;            // i32 [kMaxTopK] winners' columns
constexpr int kFineWords = kSmallBins + kSmallBins / 32; // second-digit histogram (padded layout)
constexpr int kOffFine = kOffOut + kMaxTopK;             // u32 [kFineWords]
// 64 lane-indexed dummy words (and, seen from the candidate columns array, 64 more kCandCap
// words further): the writes of the lanes that keep nothing go there, so that the per-key-row
// writes need no branch (and no exec-mask round trip)
constexpr int kOffDummy = kOffFine + kFineWords;
static_assert(kOffDummy + kCandCap + 64 <= kHistWords, "LDS regions must fit in the histogram's space");
static_assert(kUnitsPerLane <= 6, "unit scan layout");
static_assert(kBinsPerThread % 4 == 0 && kBinsPerThread <= 64, "histogram layout");

// Order-preserving key of a float score: larger float <-> larger unsigned key.  Adding +0.0
// turns -0.0 into +0.0 (so the two compare equal) and leaves every other value unchanged.
// Finite scores and -inf map to keys >= 0x007FFFFF, so key 0 is free to mark "no score".
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// Word of first-digit bin `bin` (15 bits) in the histogram.  Thread t's B = kBinsPerThread bins
// [Bt, Bt+B) sit at words kHistStride*t.., 16-byte aligned, so that the per-thread sums are
// read as b128 and the 16 lanes of one LDS pass start on distinct banks.  The 4 words after
// each thread's bins are never summed.
__device__ __forceinline__ uint32_t hist_word(uint32_t bin) {
  return bin + (kHistStride - kBinsPerThread) * (bin >> kBinShift);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// A compile-time flag, so that a uniform run-time choice is taken once outside a row loop.
template <bool B>
struct Flag {
  static constexpr bool value = B;
};

__device__ __forceinline__ uint32_t mbcnt(uint64_t m, uint32_t add = 0u) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, add));
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4, 8 inside each row of
// 16 lanes, then the row totals are carried into the later rows (DPP row_shr and row_bcast).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);   // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);   // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return v;
}

// Inclusive scan of one value per thread over the workgroup.  `wsum` is LDS [kWaves].
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* wsum) {
  const int wave = threadIdx.x >> 6;
  v = wave_incl_scan(v);
  if (lane_id() == 63) wsum[wave] = v;
  __syncthreads();
  uint32_t pre = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) pre += w < wave ? wsum[w] : 0u;
  __syncthreads();
  return v + pre;
}

// Finds, among `nb` bins laid out from bin 0 up, the bin holding the kr-th largest key (bins
// are scanned from the top).  Thread t owns the bins nb-1-4t .. nb-4-4t.  Returns the bin;
// *above receives the count in higher bins, *cnt the bin's own count.
__device__ __forceinline__ uint32_t select_bin(const uint32_t* hist, int nb, uint32_t kr, uint32_t* red,
                                               uint32_t* sel, uint32_t* above, uint32_t* cnt) {
  const int tid = threadIdx.x;
  if (tid == 0) sel[0] = sel[1] = sel[2] = 0u;
  uint32_t c[4], tot = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int bin = nb - 1 - 4 * tid - j;
    c[j] = bin >= 0 ? hist[bin] : 0u;
    tot += c[j];
  }
  uint32_t acc = block_incl_scan(tot, red) - tot;   // keys in bins above this thread's first
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int bin = nb - 1 - 4 * tid - j;
    if (bin >= 0 && acc < kr && acc + c[j] >= kr) {
      sel[0] = (uint32_t)bin;
      sel[1] = acc;
      sel[2] = c[j];
    }
    acc += c[j];
  }
  __syncthreads();
  const uint32_t bin = sel[0];
  *above = sel[1];
  *cnt = sel[2];
  __syncthreads();
  return bin;
}

// Padded layout of 64*M bins for wave_select: bin b at word b + b/M, so that the M bins a
// lane reads lie M+1 words (an odd stride) from its neighbours' and no two lanes share a bank.
template <int M>
__device__ __forceinline__ uint32_t pad_word(uint32_t b) { return b + b / M; }

// One wave: among the 64*M bins of h (padded layout) scanned from the top, the bin holding the
// kr-th largest key.  Lane l owns the bins 64M-1-Ml .. 64M-M-Ml.  Every lane gets the bin, the
// count of keys above it and the bin's own count.
template <int M>
__device__ __forceinline__ void wave_select(const uint32_t* h, uint32_t kr, uint32_t& bin, uint32_t& above,
                                            uint32_t& cnt) {
  const int lane = lane_id();
  uint32_t c[M], tot = 0;
#pragma unroll
  for (int j = 0; j < M; ++j) {
    c[j] = h[pad_word<M>(64 * M - 1 - M * lane - j)];
    tot += c[j];
  }
  uint32_t acc = wave_incl_scan(tot) - tot;
  int fb = -1;
  uint32_t fa = 0, fc = 0;
#pragma unroll
  for (int j = 0; j < M; ++j) {
    if (acc < kr && acc + c[j] >= kr) {
      fb = 64 * M - 1 - M * lane - j;
      fa = acc;
      fc = c[j];
    }
    acc += c[j];
  }
  const uint64_t m = __ballot(fb >= 0);
  const int src = m ? (int)__builtin_ctzll(m) : 0;
  bin = (uint32_t)__builtin_amdgcn_readlane(fb < 0 ? 0 : fb, src);
  above = (uint32_t)__builtin_amdgcn_readlane((int)fa, src);
  cnt = (uint32_t)__builtin_amdgcn_readlane((int)fc, src);
}

// One radix round over the keys matching (pmask, pval): a histogram of the D bits below the
// prefix, then select_bin.  `keys_fn(visitor)` visits every key of the set.
template <typename KeysFn>
__device__ __forceinline__ uint32_t radix_round(KeysFn&& keys_fn, uint32_t pmask, uint32_t pval, int shift, int D,
                                                uint32_t kr, uint32_t* hist, uint32_t* red, uint32_t* sel,
                                                uint32_t* above, uint32_t* cnt) {
  const int nb = 1 << D;
  for (int j = threadIdx.x; j < nb; j += kThreads) hist[j] = 0u;
  __syncthreads();
  keys_fn([&](uint32_t u) {
    if (u && (u & pmask) == pval) atomicAdd(&hist[__builtin_amdgcn_ubfe(u, shift, D)], 1u);
  });
  __syncthreads();
  return select_bin(hist, nb, kr, red, sel, above, cnt);
}

// MODE 0: one workgroup per row.  MODE 1 (first pass over long rows): one workgroup per chunk
// of p.chunk_len columns, whose winners go to the candidate list.  MODE 2 (second pass): one
// workgroup per row, over the row's candidates (position j of the list holds the column
// p.cand_col[j]; positions ascend with columns, so ties still go to the lower column).
template <int RV, int MODE>
__global__ __launch_bounds__(kThreads) void topk_kernel(TopkParams p) {
  __shared__ __attribute__((aligned(16))) uint32_t big[kHistWords];   // histogram, then the regions above
  __shared__ uint32_t tsum[kThreads + kThreads / 8];   // padded layout of wave_select<8>
  __shared__ uint32_t red[kWaves];
  __shared__ uint32_t sel[4];
  __shared__ uint32_t wave_cnt[kWaves];
  __shared__ uint32_t wave_min[kWaves], wave_max[kWaves];
  __shared__ uint32_t cand_n;

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform (kept in a scalar register)
  const int row = MODE == 1 ? (int)blockIdx.x / p.nchunks : (int)blockIdx.x;
  const int chunk = MODE == 1 ? (int)blockIdx.x - row * p.nchunks : 0;
  const int b = row / p.q_count, il = row - b * p.q_count;
  const int i = p.q_begin + il;                     // the row's query index in its sequence
  const int Lb = p.seq_lens[b];
  if (tid == 0 && il == 0 && chunk == 0) dbg_seq_len(p.dbg, Lb, p.Q, p.max_seq_len);
  int n_row = Lb - p.Q + i + 1;                    // visible tokens of this row
#ifdef DSA_DEBUG
  n_row = min(n_row, p.max_seq_len - p.Q + i + 1); // (a length past max_seq_len, flagged, is cut there)
#endif
  n_row = n_row < 0 ? 0 : n_row;
  n_row = (int64_t)n_row > p.ld ? (int)p.ld : n_row;   // guards against lengths past the scores row
  n_row = n_row > kMaxTopkSeq ? kMaxTopkSeq : n_row;
  if constexpr (MODE != 0) n_row = min(n_row, p.nchunks * p.chunk_len);   // the candidate rows' reach
  const int k = p.k;
  const int32_t* ptab = p.page_table + (int64_t)b * p.maxP;
  const int kc = min(k, p.chunk_len);              // candidates kept per full chunk
  // n: keys this workgroup ranks; srow: their scores; c0: column of the first (MODE 1)
  int n = n_row, c0 = 0;
  const float* srow = p.scores + (int64_t)row * p.ld;
  if constexpr (MODE == 1) {
    c0 = chunk * p.chunk_len;
    n = min(max(n_row - c0, 0), p.chunk_len);
    srow += c0;
  } else if constexpr (MODE == 2) {
    const int nch = (n_row + p.chunk_len - 1) / p.chunk_len;
    n = nch > 0 ? (nch - 1) * kc + min(k, n_row - (nch - 1) * p.chunk_len) : 0;
    srow = p.cand_score + (int64_t)row * p.cand_ld;
  }
  const int32_t* ccol = MODE == 2 ? p.cand_col + (int64_t)row * p.cand_ld : nullptr;
#ifdef DSA_DEBUG
  if constexpr (MODE != 2) {   // (the candidates of the second pass come from checked chunks)
    bool nan_seen = false;
    for (int j = tid; j < n; j += kThreads) nan_seen |= srow[j] != srow[j];
    if (nan_seen) dbg_flag(p.dbg, kDbgNanScore);
  }
#endif
  // MODE 1 writes its winners after those of the chunks before it (each keeps kc)
  float* cs_out = MODE == 1 ? p.cand_score + (int64_t)row * p.cand_ld + (int64_t)chunk * kc : nullptr;
  int32_t* cc_out = MODE == 1 ? p.cand_col + (int64_t)row * p.cand_ld + (int64_t)chunk * kc : nullptr;
  const int64_t out_row = (int64_t)b * p.Q + i;
  int32_t* idx_out = MODE == 1 ? nullptr : p.idx + out_row * k;
  int32_t* slot_out = MODE != 1 && p.slots ? p.slots + out_row * k : nullptr;

  // The register block is requested before the row's length arrives: the loads need only the
  // row's extent in memory, and columns past the row are masked when the keys are formed.
  constexpr int kRegRows = RV * kWaves;              // key rows held in registers
  const int64_t ext = MODE == 2 ? p.cand_ld : MODE == 1 ? min((int64_t)p.chunk_len, p.ld - c0) : p.ld;
  float x[RV];
  if (((int64_t)kRegRows << 6) <= ext) {
    const float* wrow = srow + ((wave * RV) << 6);   // uniform base, lane offset, constant row offsets
#pragma unroll
    for (int j = 0; j < RV; ++j) x[j] = wrow[(j << 6) + lane];
  } else {
#pragma unroll
    for (int j = 0; j < RV; ++j) x[j] = srow[min(((wave * RV + j) << 6) + lane, (int)ext - 1)];
  }

  if constexpr (MODE == 1) {
    if (n <= k) {   // the whole chunk is kept
      for (int j = tid; j < n; j += kThreads) {
        cs_out[j] = srow[j];
        cc_out[j] = c0 + j;
      }
      return;
    }
  } else {
    if (n_row <= k || n <= k) {   // everything visible (every candidate) is selected
      for (int j = tid; j < k; j += kThreads) {
        const int t = j < n ? (MODE == 2 ? ccol[j] : j) : -1;
        idx_out[j] = t;
        if (slot_out) slot_out[j] = t >= 0 ? dbg_page(p.dbg, ptab[t / p.P], p.num_slots, p.P) * p.P + t % p.P : -1;
      }
      return;
    }
  }

  // ---- pass 1: keys (registers), page-table row (registers), first-digit histogram
  const int nrows = (n + 63) >> 6;
  const int nseg = nrows > kRegRows ? (nrows - kRegRows + kTailRows * kWaves - 1) / (kTailRows * kWaves) : 0;
  const int npages = (n_row + p.P - 1) / p.P;       // pages of the row's visible columns
  const bool cache_pages = slot_out != nullptr && npages <= kPtabCache;
  // key row r (uniform) holds columns 64r .. 64r+63; register row j of wave w is row w*RV + j
  auto key_of = [&](float x, int r) -> uint32_t {
    return ((r + 1) << 6) <= n || (r << 6) + lane < n ? order_key(x) : 0u;
  };
  // the register block lies wholly inside the row (the common case): no per-row clamps
  const bool reg_full = (kRegRows << 6) <= n;
  uint32_t key[RV];
  {
    // the histogram is cleared while the loads are in flight
    u32x4* l4 = (u32x4*)big;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < (kHistWords / 4 + kThreads - 1) / kThreads; ++j)
      if (j * kThreads + tid < kHistWords / 4) l4[j * kThreads + tid] = z;
    if (reg_full) {
#pragma unroll
      for (int j = 0; j < RV; ++j) key[j] = order_key(x[j]);
    } else {
#pragma unroll
      for (int j = 0; j < RV; ++j) key[j] = key_of(x[j], wave * RV + j);
    }
  }
  int32_t pv[kPtabCache / kThreads];
  if (cache_pages) {
#pragma unroll
    for (int u = 0; u < kPtabCache / kThreads; ++u)
      pv[u] = dbg_page(p.dbg, ptab[min(u * kThreads + tid, npages - 1)], p.num_slots, p.P);
  }

  // The streamed key rows (from kRegRows on), in segments of kTailRows rows per wave.
  // begin(s) and end(s) bracket this wave's rows of segment s; f(key, key row) is called
  // uniformly per wave (it may hold ballots).
  // Segment s+1 is loaded while segment s is processed (two register buffers).
  auto tail_pass = [&, srow](auto&& f, auto&& begin, auto&& end) {
    auto load = [&](float (&x)[kTailRows], int s) {
      const int r0 = kRegRows + (s * kWaves + wave) * kTailRows;
      if (((r0 + kTailRows) << 6) <= n) {
        const float* wrow = srow + (r0 << 6);
#pragma unroll
        for (int u = 0; u < kTailRows; ++u) x[u] = wrow[(u << 6) + lane];
      } else {
#pragma unroll
        for (int u = 0; u < kTailRows; ++u) x[u] = srow[min(((r0 + u) << 6) + lane, n - 1)];
      }
    };
    auto run = [&](const float (&x)[kTailRows], int s) {
      const int r0 = kRegRows + (s * kWaves + wave) * kTailRows;
      begin(s);
      if (((r0 + kTailRows) << 6) <= n) {
#pragma unroll
        for (int u = 0; u < kTailRows; ++u) f(order_key(x[u]), r0 + u);
      } else {
#pragma unroll
        for (int u = 0; u < kTailRows; ++u)
          if (r0 + u < nrows) f(key_of(x[u], r0 + u), r0 + u);   // uniform
      }
      end(s);
    };
    float xa[kTailRows], xb[kTailRows];
    if (nseg > 0) load(xa, 0);
    for (int s = 0; s < nseg; s += 2) {
      if (s + 1 < nseg) load(xb, s + 1);
      run(xa, s);
      if (s + 1 < nseg) {
        if (s + 2 < nseg) load(xa, s + 2);
        run(xb, s + 1);
      }
    }
  };
  auto nop = [](int) {};
  auto all_keys = [&](auto&& visit) {
#pragma unroll
    for (int j = 0; j < RV; ++j) visit(key[j]);
    tail_pass([&](uint32_t kk, int) { visit(kk); }, nop, nop);
  };

  // ---- the first digit: the 15 key bits below the leading bits that every key of the row
  // shares (the keys' min and max agree on them), so that a row of close scores still spreads
  // over the histogram.  Rows with a streamed part (which would need a pass of its own for
  // the min and max) take the top 15 bits.
  {
    uint32_t mn = ~0u, mx = 0u;                      // key 0 (outside the row) is left out of the min
#pragma unroll
    for (int j = 0; j < RV; ++j) {
      mn = min(mn, key[j] ? key[j] : ~0u);
      mx = max(mx, key[j]);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      mn = min(mn, (uint32_t)__shfl_xor((int)mn, o));
      mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
    }
    if (lane == 0) {
      wave_min[wave] = mn;
      wave_max[wave] = mx;
    }
  }
  __syncthreads();
  uint32_t kmin = wave_min[0], kmax = wave_max[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    kmin = min(kmin, wave_min[w]);
    kmax = max(kmax, wave_max[w]);
  }
  // (n > k >= 1, so some key is in the row and kmin <= kmax)
  const int common = nseg > 0 ? 0 : (kmin ^ kmax) ? __builtin_clz(kmin ^ kmax) : 32;
  const int sh1 = common >= 17 ? 0 : 17 - common;   // the digit is key bits [sh1, sh1 + 15)
  auto bin1 = [sh1](uint32_t kk) { return (kk >> sh1) & 0x7FFFu; };
  {
    // a column outside the row counts into one of 32 words that are never summed (spread so
    // that a short row does not pile onto one LDS address)
    const uint32_t dummy = (uint32_t)(kHistStride * (lane & 31) + kBinsPerThread);
    auto count = [&](uint32_t kk, int r) {
      if (((r + 1) << 6) <= n) atomicAdd(&big[hist_word(bin1(kk))], 1u);
      else if ((r << 6) < n) atomicAdd(&big[kk ? hist_word(bin1(kk)) : dummy], 1u);
    };
    if (reg_full) {
#pragma unroll
      for (int j = 0; j < RV; ++j) atomicAdd(&big[hist_word(bin1(key[j]))], 1u);
    } else {
#pragma unroll
      for (int j = 0; j < RV; ++j) count(key[j], wave * RV + j);
    }
    tail_pass(count, nop, nop);
  }
  __syncthreads();

  // ---- the first-digit bin: sums of kBinsPerThread bins per thread, then the bins of the chosen sum
  {
    const u32x4* h4 = (const u32x4*)(big + kHistStride * tid);
    u32x4 acc = h4[0];
#pragma unroll
    for (int j = 1; j < kBinsPerThread / 4; ++j) acc += h4[j];
    tsum[pad_word<kThreads / 64>(tid)] = acc[0] + acc[1] + acc[2] + acc[3];
  }
  __syncthreads();
  // every wave finds the same bin on its own (no further barrier)
  uint32_t r1, above, cnt;
  wave_select<kThreads / 64>(tsum, (uint32_t)k, r1, above, cnt);
  uint32_t kr = (uint32_t)k - above;
  uint32_t fb, above1;
  {
    // the thread range's kBinsPerThread bins, scanned from the top by one wave
    const uint32_t* h = big + kHistStride * r1;
    const uint32_t c1 = lane < kBinsPerThread ? h[kBinsPerThread - 1 - lane] : 0u;
    const uint32_t incl = wave_incl_scan(c1);
    const uint64_t m = __ballot(lane < kBinsPerThread && incl - c1 < kr && incl >= kr);
    const int src = m ? (int)__builtin_ctzll(m) : 0;
    fb = (uint32_t)(kBinsPerThread - 1 - src);
    above1 = (uint32_t)__builtin_amdgcn_readlane((int)(incl - c1), src);
    cnt = (uint32_t)__builtin_amdgcn_readlane((int)c1, src);
  }
  const uint32_t b1 = r1 * kBinsPerThread + fb;
  kr -= above1;
  __syncthreads();                                   // every wave has read the histogram
  // the bin's keys: the shared leading bits, then b1
  int plen = 32 - sh1;
  uint32_t pmask = ~0u << sh1;
  uint32_t pval = (sh1 + 15 >= 32 ? 0u : kmin & (~0u << (sh1 + 15))) | (b1 << sh1);
  bool take_all = cnt == kr;                         // the whole bin is selected

  // ---- narrowing rounds while the bin is too large to gather (many equal or near-equal keys)
  uint32_t* shist = big + kOffSmall;
  while (!take_all && cnt > (uint32_t)kCandCap && plen < 32) {
    const int D = min(kSmallBits, 32 - plen);
    const int shift = 32 - plen - D;
    uint32_t ab;
    const uint32_t bin = radix_round(all_keys, pmask, pval, shift, D, kr, shist, red, sel, &ab, &cnt);
    kr -= ab;
    plen += D;
    pmask = plen == 32 ? ~0u : ~0u << (32 - plen);
    pval |= bin << shift;
    take_all = cnt == kr;
  }
  // Three cases: the whole bin is taken; the bin is one key value (its first kr keys in column
  // order are taken); or the bin's keys are gathered and the exact threshold found among them.
  const bool gather = !take_all && plen < 32;
  const bool count_eq = !take_all && plen == 32;
  const bool per_wave = cnt <= (uint32_t)kCandPerWave;   // no wave can overflow its region
  const uint32_t t_lo = pval, t_hi = pval | ~pmask;
  const uint32_t t_gt = take_all ? t_lo - 1u : t_hi;  // keys above t_gt are taken for sure

  // ---- pass 2: per unit, the count of keys above t_gt (and, for a one-value bin, inside it);
  // gather the bin's keys
  uint32_t* cand_key = big + kOffCandKey;
  uint32_t* cand_col = big + kOffCandCol;
  int32_t* ptab_s = (int32_t*)(big + kOffPtab);
  uint32_t* g_cnt = big + kOffGCnt;                  // per unit: keys taken as "above"
  uint32_t* e_cnt = big + kOffECnt;                  // per unit: keys equal to the threshold
  if (cache_pages) {
#pragma unroll
    for (int u = 0; u < kPtabCache / kThreads; ++u) ptab_s[u * kThreads + tid] = pv[u];
  }
  // second digit: the D2 key bits below the bin's prefix, counted over the gathered keys
  const int D2 = min(kSmallBits, 32 - plen);
  const int sh2 = 32 - plen - D2;
  uint32_t* fhist = big + kOffFine;
  for (int j = tid; j < kFineWords; j += kThreads) fhist[j] = 0u;
  if (tid == 0) cand_n = 0u;
  __syncthreads();
  uint32_t wcount = 0;                               // candidates of this wave so far (uniform)
  uint32_t ug = 0, ue = 0;                           // this lane's counts in the current unit
  // (the LDS region pointers are captured by value so that they stay in registers)
  auto unit_done = [&, g_cnt, e_cnt](int u) {
    const uint32_t gs = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(ug), 63);
    const uint32_t es = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(ue), 63);
    if (lane == 0) {
      g_cnt[u] = gs;
      e_cnt[u] = es;
    }
    ug = 0u;
    ue = 0u;
  };
  // G: gather the bin's keys; PW: into per-wave regions; CE: count the keys equal to t_lo
  auto pass2 = [&, cand_key, cand_col](auto G, auto PW, auto CE) {
    auto classify = [&](uint32_t kk, int r) {
      ug += kk > t_gt ? 1u : 0u;
      if constexpr (decltype(CE)::value) ue += kk == t_lo ? 1u : 0u;
      if constexpr (decltype(G)::value) {
        const bool in = kk - t_lo <= t_hi - t_lo;   // t_lo <= key <= t_hi (key 0 < t_lo wraps high)
        const uint64_t me = __ballot(in);
        if constexpr (decltype(PW)::value) {
          if (in) {
            const uint32_t pos = mbcnt(me, wave * kCandPerWave + wcount);
            cand_key[pos] = kk;
            cand_col[pos] = (uint32_t)((r << 6) + lane);
          }
          wcount += (uint32_t)__popcll(me);
        } else if (me) {                             // uniform
          uint32_t b0 = 0;
          if (lane == 0) b0 = atomicAdd(&cand_n, (uint32_t)__popcll(me));
          const uint32_t base = __builtin_amdgcn_readfirstlane(b0);
          if (in) {
            const uint32_t pos = base + mbcnt(me);
            cand_key[pos] = kk;
            cand_col[pos] = (uint32_t)((r << 6) + lane);
          }
        }
      }
    };
    if constexpr (decltype(G)::value && decltype(PW)::value && !decltype(CE)::value) {
      // the register block in groups of 8 key rows: counts and ballots first; a group without
      // a key in the bin (most of them) skips the gather with one uniform branch
      constexpr int kG = RV < 8 ? RV : 8;
#pragma unroll
      for (int j0 = 0; j0 < RV; j0 += kG) {
        uint64_t me[kG], any = 0;
#pragma unroll
        for (int i = 0; i < kG; ++i) {
          const uint32_t kk = key[j0 + i];
          ug += kk > t_gt ? 1u : 0u;
          me[i] = __ballot(kk - t_lo <= t_hi - t_lo);
          any |= me[i];
        }
        if (any) {
          // (lanes outside the bin write to their dummy words: cand_key + kOffDummy + lane and
          // cand_col + kOffDummy + lane lie past every other region; an arithmetic select, since
          // a conditional here compiles to exec-mask branches)
#pragma unroll
          for (int i = 0; i < kG; ++i) {
            const uint32_t kk = key[j0 + i];
            const uint32_t in = (uint32_t)-(int32_t)(kk - t_lo <= t_hi - t_lo);
            const uint32_t at = mbcnt(me[i], wave * kCandPerWave + wcount);
            const uint32_t ad = (uint32_t)(kOffDummy - kOffCandKey + lane);
            const uint32_t pos = ad ^ ((at ^ ad) & in);
            cand_key[pos] = kk;
            cand_col[pos] = (uint32_t)(((wave * RV + j0 + i) << 6) + lane);
            wcount += (uint32_t)__popcll(me[i]);
          }
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < RV; ++j) classify(key[j], wave * RV + j);
    }
    unit_done(wave);
    tail_pass(classify, nop, [&](int s) { unit_done(kWaves * (1 + s) + wave); });
  };
  if (gather) {
    if (per_wave) pass2(Flag<true>(), Flag<true>(), Flag<false>());
    else pass2(Flag<true>(), Flag<false>(), Flag<false>());
  } else if (count_eq) {
    pass2(Flag<false>(), Flag<false>(), Flag<true>());
  } else {
    pass2(Flag<false>(), Flag<false>(), Flag<false>());
  }
  if (lane == 0) wave_cnt[wave] = wcount;
  __syncthreads();

  // ---- the exact threshold among the candidates; their counts are added to their units
  uint32_t Tg = t_gt, quota = 0u;                    // taken: key > Tg, or key == Tg among the first quota
  if (count_eq) {
    Tg = t_lo;
    quota = kr;
  }
  if (gather) {
    uint32_t T;
    auto fix = [&, cand_key, cand_col](int j) {
      const uint32_t u = cand_key[j], v = cand_col[j];
      if (u >= T) {   // one LDS word offset picks the count array (no pointer select)
        const int r = (int)(v >> 6);
        const int unit = r < kRegRows ? r / RV
                                      : kWaves * (1 + (r - kRegRows) / (kTailRows * kWaves)) +
                                            ((r - kRegRows) % (kTailRows * kWaves)) / kTailRows;
        atomicAdd(&big[(u > T ? kOffGCnt : kOffECnt) + unit], 1u);
      }
    };
    if (per_wave) {
      // every wave finds T on its own from all <= kCandPerWave candidates (up to kPerLane per
      // lane), one key bit at a time with ballot counts, then counts its own region's candidates
      uint32_t rb[kWaves + 1];
      rb[0] = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) rb[w + 1] = rb[w] + wave_cnt[w];
      if (cnt <= 64u) {
        // few candidates (the usual case): each wave holds them one per lane and finds T by a
        // ballot-count bit search over all bits below the first digit's prefix, no histogram
        uint32_t c1 = 0u;                            // 0 never matches a prefix
        if ((uint32_t)lane < cnt) {
          int w = 0;
#pragma unroll
          for (int ww = 1; ww < kWaves; ++ww) w += (uint32_t)lane >= rb[ww];
          c1 = cand_key[w * kCandPerWave + ((uint32_t)lane - rb[w])];
        }
        for (int bit = 31 - plen; bit >= 0; --bit) {
          const uint32_t m = pmask | (1u << bit), v = pval | (1u << bit);
          const uint32_t cb = (uint32_t)__popcll(__ballot((c1 & m) == v));
          if (cb >= kr) pval = v;
          else kr -= cb;
          pmask = m;
        }
        T = pval;
        for (int j = lane; j < (int)wave_cnt[wave]; j += 64) fix(wave * kCandPerWave + j);
        Tg = T;
        quota = kr;
        __syncthreads();
        goto threshold_done;
      }
      // the second digit (the D2 key bits below the prefix): one candidate per thread is counted
      static_assert(kCandPerWave <= kThreads, "one candidate per thread");
      if ((uint32_t)tid < cnt) {
        int w = 0;
#pragma unroll
        for (int ww = 1; ww < kWaves; ++ww) w += (uint32_t)tid >= rb[ww];
        const uint32_t u = cand_key[w * kCandPerWave + ((uint32_t)tid - rb[w])];
        atomicAdd(&fhist[pad_word<kSmallBins / 64>(__builtin_amdgcn_ubfe(u, sh2, D2))], 1u);
      }
      constexpr int kPerLane = (kCandPerWave + 63) / 64;
      uint32_t c[kPerLane];
#pragma unroll
      for (int q = 0; q < kPerLane; ++q) {
        const uint32_t g = (uint32_t)(q * 64 + lane);
        int w = 0;
#pragma unroll
        for (int ww = 1; ww < kWaves; ++ww) w += g >= rb[ww];
        c[q] = g < cnt ? cand_key[w * kCandPerWave + (g - rb[w])] : 0u;   // 0 never matches a prefix
      }
      __syncthreads();
      // the second digit's bin (bins past 2^D2 are empty)
      {
        uint32_t bin2, ab2, c2;
        wave_select<kSmallBins / 64>(fhist, kr, bin2, ab2, c2);
        kr -= ab2;
        plen += D2;
        pmask = plen == 32 ? ~0u : ~0u << (32 - plen);
        pval |= bin2 << sh2;
      }
      // the bit search visits only the candidate rows that hold keys of the prefix
      bool live[kPerLane];
#pragma unroll
      for (int q = 0; q < kPerLane; ++q) live[q] = __ballot((c[q] & pmask) == pval) != 0ull;
      for (int bit = 31 - plen; bit >= 0; --bit) {
        const uint32_t m = pmask | (1u << bit), v = pval | (1u << bit);
        uint32_t cb = 0;
#pragma unroll
        for (int q = 0; q < kPerLane; ++q)
          if (live[q]) cb += (uint32_t)__popcll(__ballot((c[q] & m) == v));
        if (cb >= kr) pval = v;
        else kr -= cb;
        pmask = m;
      }
      T = pval;
      for (int j = lane; j < (int)wave_cnt[wave]; j += 64) fix(wave * kCandPerWave + j);
    } else {
      auto cand_keys = [&](auto&& visit) {
        const int nc = (int)cand_n;
        for (int j = tid; j < nc; j += kThreads) visit(cand_key[j]);
      };
      while (plen < 32) {
        const int D = min(kSmallBits, 32 - plen);
        const int shift = 32 - plen - D;
        uint32_t ab, cc;
        const uint32_t bin = radix_round(cand_keys, pmask, pval, shift, D, kr, shist, red, sel, &ab, &cc);
        kr -= ab;
        plen += D;
        pmask = plen == 32 ? ~0u : ~0u << (32 - plen);
        pval |= bin << shift;
      }
      T = pval;
      const int nc = (int)cand_n;
      for (int j = tid; j < nc; j += kThreads) fix(j);
    }
    Tg = T;
    quota = kr;
    __syncthreads();
  }
threshold_done:

  // ---- order-preserving output.  Every wave scans all units' counts (no barrier): a unit's
  // output offset counts the keys taken in earlier units, where the keys equal to Tg are taken
  // in column order until quota of them are.
  constexpr int U = kUnitsPerLane;
  const int nunits = kWaves * (1 + nseg);
  uint32_t u_base[U], u_eq[U], e_total;
  {
    uint32_t gc[U], ec[U], es = 0;
#pragma unroll
    for (int a = 0; a < U; ++a) {
      const int u = lane * U + a;
      gc[a] = u < nunits ? g_cnt[u] : 0u;
      ec[a] = u < nunits ? e_cnt[u] : 0u;
      es += ec[a];
    }
    uint32_t eb = wave_incl_scan(es);
    e_total = (uint32_t)__builtin_amdgcn_readlane((int)eb, 63);
    eb -= es;
    uint32_t tk[U], ts = 0;
#pragma unroll
    for (int a = 0; a < U; ++a) {
      u_eq[a] = eb;
      tk[a] = gc[a] + min(ec[a], quota - min(eb, quota));
      eb += ec[a];
      ts += tk[a];
    }
    uint32_t tb = wave_incl_scan(ts) - ts;
#pragma unroll
    for (int a = 0; a < U; ++a) {
      u_base[a] = tb;
      tb += tk[a];
    }
  }
  // (taken before, equal keys before) of unit u, uniform: read from lane u/U, then the element
  // picked among scalars (a run-time index into the per-lane arrays would move them to memory)
  auto unit_start = [&](int u, uint32_t& tb, uint32_t& eb) {
    const int l = u / U, a = u - l * U;
    tb = (uint32_t)__builtin_amdgcn_readlane((int)u_base[0], l);
    eb = (uint32_t)__builtin_amdgcn_readlane((int)u_eq[0], l);
#pragma unroll
    for (int aa = 1; aa < U; ++aa) {
      const uint32_t tv = (uint32_t)__builtin_amdgcn_readlane((int)u_base[aa], l);
      const uint32_t ev = (uint32_t)__builtin_amdgcn_readlane((int)u_eq[aa], l);
      tb = a == aa ? tv : tb;
      eb = a == aa ? ev : eb;
    }
  };
  // When every key equal to Tg is taken (no tie to break) a key is taken iff key >= t_take.
  const bool ties = quota < e_total;
  const uint32_t t_take = quota == 0u ? Tg + 1u : Tg;
  int32_t* out_s = (int32_t*)(big + kOffOut);
  auto emit_all = [&, out_s](auto TIES) {
    uint32_t obase, eqr;                             // uniform: taken so far, equal keys so far
    auto emit = [&](uint32_t kk, int r) {
      bool take;
      if constexpr (decltype(TIES)::value) {
        const bool eq = kk == Tg;
        const uint64_t me = __ballot(eq);
        take = kk > Tg || (eq && mbcnt(me, eqr) < quota);
        eqr += (uint32_t)__popcll(me);
      } else {
        take = kk >= t_take;
      }
      const uint64_t mt = __ballot(take);
      // (a lane that takes nothing writes to its dummy word)
      out_s[take ? min(mbcnt(mt, obase), (uint32_t)kMaxTopK - 1u) : (uint32_t)(kOffDummy - kOffOut + lane)] = (r << 6) + lane;
      obase += (uint32_t)__popcll(mt);
    };
    unit_start(wave, obase, eqr);
    if constexpr (!decltype(TIES)::value) {
      // the register block in groups of 8 key rows: the 8 ballots first, then the offsets and
      // writes, so that consecutive rows do not wait on each other's count
      constexpr int kG = RV < 8 ? RV : 8;
#pragma unroll
      for (int j0 = 0; j0 < RV; j0 += kG) {
        uint64_t mt[kG];
#pragma unroll
        for (int i = 0; i < kG; ++i) mt[i] = __ballot(key[j0 + i] >= t_take);
#pragma unroll
        for (int i = 0; i < kG; ++i) {
          // (an arithmetic select: a conditional expression here compiles to exec-mask branches)
          const uint32_t tk = (uint32_t)-(int32_t)(key[j0 + i] >= t_take);   // all ones if taken
          const uint32_t at = min(mbcnt(mt[i], obase), (uint32_t)kMaxTopK - 1u);
          const uint32_t ad = (uint32_t)(kOffDummy - kOffOut + lane);
          out_s[ad ^ ((at ^ ad) & tk)] = ((wave * RV + j0 + i) << 6) + lane;
          obase += (uint32_t)__popcll(mt[i]);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < RV; ++j) emit(key[j], wave * RV + j);
    }
    tail_pass(emit, [&](int s) { unit_start(kWaves * (1 + s) + wave, obase, eqr); }, nop);
  };
  if (ties) emit_all(Flag<true>());
  else emit_all(Flag<false>());
  __syncthreads();
  // the k winners, in column order, with their cache slots (fused page map); MODE 1: their
  // scores and columns as candidates
  const int P = p.P;
  const bool p_pow2 = (P & (P - 1)) == 0;
  const int p_shift = __ffs(P) - 1;
  for (int j = tid; j < k; j += kThreads) {
    const int pos = out_s[j];
    if constexpr (MODE == 1) {
      cs_out[j] = srow[pos];
      cc_out[j] = c0 + pos;
      continue;
    }
    const int t = MODE == 2 ? ccol[pos] : pos;
    idx_out[j] = t;
    if (slot_out) {
      int pg = p_pow2 ? t >> p_shift : t / P;
      pg = min(max(pg, 0), npages - 1);            // (t is always in [0, n_row); the clamp only guards the lookup)
      const int pe = cache_pages ? big[kOffPtab + pg] : dbg_page(p.dbg, ptab[pg], p.num_slots, P);
      slot_out[j] = pe * P + (t - pg * P);
    }
  }
}

__global__ __launch_bounds__(256) void page_map_kernel(const int32_t* idx, int64_t total, int k, int Q,
                                                       const int32_t* pt, int maxP, int P, int32_t* slots,
                                                       const int32_t* seq_lens, int64_t num_slots, uint32_t* dbg) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= total) return;
  const int64_t row = g / k;
  const int b = (int)(row / Q);
  int t = idx[g];
#ifdef DSA_DEBUG
  if (t < -1 || t >= min(seq_lens[b], maxP * P)) {   // (flagged; mapped to -1)
    dbg_flag(dbg, kDbgTopkIndex);
    t = -1;
  }
#else
  (void)seq_lens;
#endif
  slots[g] = t < 0 ? -1 : dbg_page(dbg, pt[(int64_t)b * maxP + t / P], num_slots, P) * P + t % P;
}

}  // namespace

namespace {

// Two-pass plan for long rows: the chunk length L (0 = one pass) and chunks per row.  Rows of
// 64K+ columns are split when they are at most 128 (half the compute units), the chunks still
// fit one workgroup per compute unit, and a chunk keeps at most a quarter of its columns as
// candidates.  (Measured on MI355X: a 128K row takes 57 us in one pass and 24 us in chunks of
// 16K; 128 rows of 64K take 38.7 us in one pass and 36.4 us in chunks of 32K.)
struct TopkPlan {
  int L, C;
};
TopkPlan topk_plan(int64_t rows, int max_seq_len, int k) {
  if (max_seq_len < 65536 || rows > 128) return {0, 0};
  for (int L = 16384; L <= 32768; L *= 2) {
    const int C = (max_seq_len + L - 1) / L;
    if (L >= 4 * k && C >= 2 && rows * C <= 256) return {L, C};
  }
  return {0, 0};
}

template <int MODE>
void launch_topk_mode(const TopkParams& p, unsigned blocks, int keys, hipStream_t s) {
  // 8, 16, 32 or 64 key rows per wave stay in registers (up to 32K keys); keys past that are
  // re-read from L2 in each pass
  const int need = (keys + 64 * kWaves - 1) / (64 * kWaves);
  const dim3 grid(blocks), block(kThreads);
  if (need <= 8) hipLaunchKernelGGL((topk_kernel<8, MODE>), grid, block, 0, s, p);
  else if (need <= 16) hipLaunchKernelGGL((topk_kernel<16, MODE>), grid, block, 0, s, p);
  else if (need <= 32) hipLaunchKernelGGL((topk_kernel<32, MODE>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((topk_kernel<64, MODE>), grid, block, 0, s, p);
}

}  // namespace

size_t topk_workspace_bytes(int64_t rows, int max_seq_len, int k) {
  const TopkPlan pl = topk_plan(rows, max_seq_len, k);
  if (pl.L == 0) return 0;
  const int64_t ld = (int64_t)pl.C * (k < pl.L ? k : pl.L);
  return (size_t)(rows * ld) * (sizeof(float) + sizeof(int32_t)) + 256;
}

hipError_t launch_topk(const TopkParams& p1, int rows, int max_seq_len, void* ws, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  TopkParams p0 = p1;
  if (p0.q_count == 0) {
    p0.q_begin = 0;
    p0.q_count = p0.Q;
  }
  const TopkPlan pl = topk_plan(rows, max_seq_len, p0.k);
  if (pl.L == 0) {
    TopkParams p = p0;
    p.chunk_len = 1 << 30;
    launch_topk_mode<0>(p, (unsigned)rows, max_seq_len, s);
    return hipGetLastError();
  }
  TopkParams p = p0;
  p.chunk_len = pl.L;
  p.nchunks = pl.C;
  p.cand_ld = (int64_t)pl.C * (p.k < pl.L ? p.k : pl.L);
  p.cand_score = (float*)ws;
  const size_t score_bytes = ((size_t)rows * p.cand_ld * sizeof(float) + 255) / 256 * 256;
  p.cand_col = (int32_t*)((char*)ws + score_bytes);
  launch_topk_mode<1>(p, (unsigned)(rows * pl.C), pl.L, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch_topk_mode<2>(p, (unsigned)rows, (int)p.cand_ld, s);
  return hipGetLastError();
}

hipError_t launch_page_map(const int32_t* idx, int64_t total, int k, int Q, const int32_t* pt, int maxP,
                           int P, int32_t* slots, const int32_t* seq_lens, int64_t num_slots, uint32_t* dbg,
                           hipStream_t s) {
  if (total == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(page_map_kernel, dim3(blocks), dim3(256), 0, s, idx, total, k, Q, pt, maxP, P, slots,
                     seq_lens, num_slots, dbg);
  return hipGetLastError();
}

}  // namespace dsa
