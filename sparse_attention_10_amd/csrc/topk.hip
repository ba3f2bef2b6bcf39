// Top-k selection and page mapping on gfx950 (the "top-k + page-mapping transforms" kernel group
// of "GLM-52 Runs on RTX 4090", section "how did he do it"; the fused page-map variant is the
// README's SGLANG_NSA_FUSE_TOPK option, renning22/glm-5.2-4090, usage section).
//
// One 512-thread workgroup per query row.  The selection is exact: equal scores go to the
// lower token index, -0.0 equals +0.0, winners come out in ascending token order.  The work is
// bound by the vector ALU of the one CU, so the kernel touches every key only twice:
//   pass 1  Scores become order-preserving uint32 keys (larger score <-> larger key; key 0
//           marks a column outside the row) and are counted into an LDS histogram of their top
//           15 bits.  Two scans (256 coarse bins of 128, then the 128 bins of the chosen coarse
//           bin) find the bin b holding the k-th largest key.  A bin holding more than
//           kCandCap keys is narrowed by 11-bit radix rounds over the keys of that bin.
//   pass 2  Every key is classified against the bin: the ballot masks "above the bin" and
//           "inside the bin" are kept per 256 columns in LDS, and the keys inside the bin (the
//           candidates) are gathered with their columns.  The exact threshold key T is then
//           selected among the candidates in LDS, and the candidates' mask bits are corrected
//           in place (above T -> "above", below T -> cleared, equal stays).
//   output  A scan of the mask popcounts in column order gives each 256-column chunk its
//           output offset; a thread walks its chunk's set bits in ascending column order,
//           taking every key above T and the lowest-column keys equal to T until k are taken,
//           and writes the token index and (fused page map) its cache slot.
// Scores are read as aligned float4: a row that starts off 16-byte alignment is read from the
// aligned address below it, as if it had 1-3 leading columns that hold no score.  The first
// 32K columns stay in registers; columns past that are re-read from L2 in each pass.
#include "dsa_internal.hpp"

namespace dsa {

namespace {

#ifndef DSA_TOPK_THREADS
#define DSA_TOPK_THREADS 512
#endif
constexpr int kThreads = DSA_TOPK_THREADS;
constexpr int kWaves = kThreads / 64;
constexpr int kChunkCols = 256;                          // columns of one (iteration, wave) chunk
constexpr int kMaxChunks = (kMaxTopkSeq + 3 + kChunkCols - 1) / kChunkCols;
constexpr int kHistBins = 1 << 15;                       // first digit: top 15 key bits
constexpr int kBinsPerThread = kHistBins / kThreads;    // bins summed by one thread
constexpr int kBinShift = __builtin_ctz(kBinsPerThread);
constexpr int kHistWords = kHistBins + kHistBins / kBinsPerThread;   // a pad word after each thread's bins
constexpr int kCandCap = 4096;                           // candidates gathered into LDS
constexpr int kCandPerWave = kCandCap / kWaves;          // per-wave candidate regions
constexpr int kPtabCache = 4096;                         // page-table entries cached in LDS
constexpr int kSmallBits = 11;                           // digit of the narrowing rounds
constexpr int kSmallBins = 1 << kSmallBits;
constexpr int kTailBatch = 8;                            // float4 loads in flight per thread

// Word offsets in the one LDS array: the histogram in pass 1, then these regions.
constexpr int kOffGt = 0;                                // u64 [4 * kMaxChunks]
constexpr int kOffEq = kOffGt + 8 * kMaxChunks;          // u64 [4 * kMaxChunks]
constexpr int kOffCandKey = kOffEq + 8 * kMaxChunks;     // u32 [kCandCap]
constexpr int kOffCandCol = kOffCandKey + kCandCap;      // u32 [kCandCap]
constexpr int kOffPtab = kOffCandCol + kCandCap;         // i32 [kPtabCache]
constexpr int kOffSmall = kOffPtab + kPtabCache;         // u32 [kSmallBins]
constexpr int kOffCnt = kOffSmall + kSmallBins;          // u32 [2 * kMaxChunks] chunk counts
static_assert(kOffCnt + 2 * kMaxChunks <= kHistWords, "LDS regions must fit in the histogram's space");
static_assert(kWaves * 256 <= kSmallBins, "one 256-bin histogram per wave fits the small region");
static_assert(2 * kMaxChunks <= kCandCap, "chunk offsets reuse the candidate region");

// Order-preserving key of a float score: larger float <-> larger unsigned key.  Adding +0.0
// turns -0.0 into +0.0 (so the two compare equal) and leaves every other value unchanged.
// Finite scores and -inf map to keys >= 0x007FFFFF (15-bit bin >= 63), so key 0 is free to
// mark "no score" and bins 0..62 of the first-digit histogram hold no score.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// Word of bin (key >> 17) in the first-digit histogram.  With B = kBinsPerThread, bin b sits at
// word b + b/B, so that thread t sums its B bins [Bt, Bt+B) at words (B+1)t.. with no two
// lanes of a wave on one LDS bank.
__device__ __forceinline__ uint32_t hist_word(uint32_t key) { return (key >> 17) + (key >> (17 + kBinShift)); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ uint32_t mbcnt(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
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

// One wave: among the 64*M bins h[0..64M) scanned from the top, the bin holding the kr-th
// largest key.  Lane l owns the bins 64M-1-Ml .. 64M-M-Ml.  Every lane gets the bin, the count
// of keys above it and the bin's own count.
template <int M>
__device__ __forceinline__ void wave_select(const uint32_t* h, uint32_t kr, uint32_t& bin, uint32_t& above,
                                            uint32_t& cnt) {
  const int lane = lane_id();
  uint32_t c[M], tot = 0;
#pragma unroll
  for (int j = 0; j < M; ++j) {
    c[j] = h[64 * M - 1 - M * lane - j];
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

// Keys of one float4 at virtual columns v0..v0+3 (real column = virtual - o).  `full`
// (uniform in the wave) says that all of the wave's columns lie inside the row.
__device__ __forceinline__ void to_keys(const f32x4& x, int v0, int o, int n, bool full, uint32_t (&key)[4]) {
  if (full) {
#pragma unroll
    for (int j = 0; j < 4; ++j) key[j] = order_key(x[j]);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) key[j] = (uint32_t)(v0 + j - o) < (uint32_t)n ? order_key(x[j]) : 0u;
  }
}

template <int V>
__global__ __launch_bounds__(kThreads) void topk_kernel(TopkParams p) {
  __shared__ __attribute__((aligned(16))) uint32_t big[kHistWords];   // histogram, then the regions above
  __shared__ uint32_t tsum[kThreads];
  __shared__ uint32_t red[kWaves];
  __shared__ uint32_t sel[4];
  __shared__ uint32_t wave_cnt[kWaves];
  __shared__ uint32_t cand_n;

  const int tid = threadIdx.x;
  const int lane = lane_id(), wave = tid >> 6;
  const int row = blockIdx.x;
  const int b = row / p.Q, i = row - b * p.Q;
  int n = p.seq_lens[b] - p.Q + i + 1;             // visible tokens of this row
  n = n < 0 ? 0 : n;
  n = (int64_t)n > p.ld ? (int)p.ld : n;           // guards against lengths past the scores row
  n = n > kMaxTopkSeq ? kMaxTopkSeq : n;
  const int k = p.k;
  int32_t* idx_out = p.idx + (int64_t)row * k;
  int32_t* slot_out = p.slots ? p.slots + (int64_t)row * k : nullptr;
  const int32_t* ptab = p.page_table + (int64_t)b * p.maxP;

  if (n <= k) {   // everything visible is selected
    for (int j = tid; j < k; j += kThreads) {
      idx_out[j] = j < n ? j : -1;
      if (slot_out) slot_out[j] = j < n ? ptab[j / p.P] * p.P + j % p.P : -1;
    }
    return;
  }

  // ---- pass 1: keys (registers), page-table row (registers), first-digit histogram
  const float* srow = p.scores + (int64_t)row * p.ld;
  const int o = (int)(((uintptr_t)srow >> 2) & 3);  // leading columns of the aligned view
  const f32x4* vrow = (const f32x4*)(srow - o);
  const int nv = n + o;                              // virtual columns
  const int nvec = (nv + 3) >> 2;
  const int npages = (n + p.P - 1) / p.P;
  const bool cache_pages = slot_out != nullptr && npages <= kPtabCache;
  // a wave's 256 columns of vector index vi lie inside the row: chunk >= 1 and not past nv
  auto full_chunk = [&](int vi) { return (vi >> 6) > 0 && ((vi >> 6) + 1) * kChunkCols <= nv; };
  uint32_t key[V][4];
  {
    f32x4 x[V];
#pragma unroll
    for (int it = 0; it < V; ++it) x[it] = vrow[min(it * kThreads + tid, nvec - 1)];
#pragma unroll
    for (int it = 0; it < V; ++it) {
      const int vi = it * kThreads + tid;
      to_keys(x[it], 4 * vi, o, n, full_chunk(vi), key[it]);
    }
  }
  int32_t pv[kPtabCache / kThreads];
  if (cache_pages) {
#pragma unroll
    for (int u = 0; u < kPtabCache / kThreads; ++u) pv[u] = ptab[min(u * kThreads + tid, npages - 1)];
  }
  {
    u32x4* l4 = (u32x4*)big;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < (kHistWords / 4 + kThreads - 1) / kThreads; ++j)
      if (j * kThreads + tid < kHistWords / 4) l4[j * kThreads + tid] = z;
  }

  // the streamed columns: f(keys of one float4, vector index) for every vector index >= V*512,
  // in batches of kTailBatch loads per thread; called uniformly (it may hold ballots)
  auto tail_pass = [&, vrow](auto&& f) {
    for (int base = V * kThreads; base < nvec; base += kTailBatch * kThreads) {
      f32x4 x[kTailBatch];
#pragma unroll
      for (int u = 0; u < kTailBatch; ++u) x[u] = vrow[min(base + u * kThreads + tid, nvec - 1)];
#pragma unroll
      for (int u = 0; u < kTailBatch; ++u) {
        if (base + u * kThreads < nvec) {          // uniform
          uint32_t kk[4];
          const int vi = base + u * kThreads + tid;
          to_keys(x[u], 4 * vi, o, n, full_chunk(vi), kk);
          f(kk, vi);
        }
      }
    }
  };
  auto all_keys = [&](auto&& visit) {
#pragma unroll
    for (int it = 0; it < V; ++it)
#pragma unroll
      for (int j = 0; j < 4; ++j) visit(key[it][j]);
    tail_pass([&](const uint32_t (&kk)[4], int) {
#pragma unroll
      for (int j = 0; j < 4; ++j) visit(kk[j]);
    });
  };

  __syncthreads();
  {
    // a column outside the row counts into one of the bins 1..32, which no score uses (spread
    // so that a short row does not pile onto one LDS address)
    const uint32_t dummy = (uint32_t)(lane & 31) + 1u;
    auto count = [&](const uint32_t (&kk)[4], int vi) {
      if (full_chunk(vi)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) atomicAdd(&big[hist_word(kk[j])], 1u);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) atomicAdd(&big[kk[j] ? hist_word(kk[j]) : dummy], 1u);
      }
    };
#pragma unroll
    for (int it = 0; it < V; ++it) count(key[it], it * kThreads + tid);
    tail_pass(count);
  }
  __syncthreads();
  if (tid < 63) big[tid] = 0u;                       // bins 0..62 (words 0..62) hold no score
  __syncthreads();

  // ---- the first-digit bin: sums of kBinsPerThread bins per thread, then the bins of the chosen sum
  {
    uint32_t s = 0;
    const uint32_t* h = big + (kBinsPerThread + 1) * tid;
#pragma unroll
    for (int j = 0; j < kBinsPerThread; ++j) s += h[j];
    tsum[tid] = s;
  }
  __syncthreads();
  // every wave finds the same bin on its own (no further barrier)
  static_assert(kThreads % 64 == 0 && kBinsPerThread <= 64, "wave selection layout");
  uint32_t r1, above, cnt;
  wave_select<kThreads / 64>(tsum, (uint32_t)k, r1, above, cnt);
  uint32_t kr = (uint32_t)k - above;
  uint32_t fb, above1;
  {
    // the thread range's kBinsPerThread bins (padded layout), scanned from the top by one wave
    const uint32_t* h = big + (kBinsPerThread + 1) * r1;
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
  int plen = 15;
  uint32_t pmask = 0xFFFE0000u;
  uint32_t pval = b1 << 17;
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
  // gather the bin's keys (<= kCandCap), unless the whole bin is taken or it is one key value
  const bool gather = !take_all && plen < 32;
  const bool per_wave = cnt <= (uint32_t)kCandPerWave;   // no wave can overflow its region
  const uint32_t t_lo = pval, t_hi = pval | ~pmask;
  // "above" threshold of pass 2: above the bin, or (whole bin taken) inside it too
  const uint32_t t_gt = take_all ? t_lo - 1u : t_hi;
  const bool store_eq = !gather && !take_all;       // the bin is one key value: store its masks

  // ---- pass 2: classify every column; gather the bin's keys
  uint64_t* m_gt = (uint64_t*)(big + kOffGt);
  uint64_t* m_eq = (uint64_t*)(big + kOffEq);
  uint32_t* cand_key = big + kOffCandKey;
  uint32_t* cand_col = big + kOffCandCol;
  int32_t* ptab_s = (int32_t*)(big + kOffPtab);
  const int nch = (nv + kChunkCols - 1) / kChunkCols;
  if (cache_pages) {
#pragma unroll
    for (int u = 0; u < kPtabCache / kThreads; ++u) ptab_s[u * kThreads + tid] = pv[u];
  }
  uint32_t* g_cnt = big + kOffCnt;                  // per chunk: keys taken as "above"
  uint32_t* e_cnt = g_cnt + kMaxChunks;              // per chunk: keys equal to the threshold
  if (!store_eq)
    for (int j = tid; j < 4 * nch; j += kThreads) m_eq[j] = 0ull;
  if (tid == 0) cand_n = 0u;
  __syncthreads();
  uint32_t wcount = 0;                               // candidates of this wave so far (uniform)
  // (the LDS region pointers are captured by value so that they stay in registers)
  auto classify = [&, m_gt, m_eq, cand_key, cand_col, g_cnt, e_cnt](const uint32_t (&kk)[4], int vi) {
    uint64_t mg[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) mg[j] = __ballot(kk[j] > t_gt);
    const int e = vi >> 6;                           // chunk of 256 columns (uniform in the wave)
    if (lane == 0) {
      g_cnt[e] = (uint32_t)(__popcll(mg[0]) + __popcll(mg[1]) + __popcll(mg[2]) + __popcll(mg[3]));
      if (!store_eq) e_cnt[e] = 0u;
      u32x4* g4 = (u32x4*)(m_gt + 4 * e);
      g4[0] = u32x4{(uint32_t)mg[0], (uint32_t)(mg[0] >> 32), (uint32_t)mg[1], (uint32_t)(mg[1] >> 32)};
      g4[1] = u32x4{(uint32_t)mg[2], (uint32_t)(mg[2] >> 32), (uint32_t)mg[3], (uint32_t)(mg[3] >> 32)};
    }
    if (gather || store_eq) {
      bool in[4];
      uint64_t me[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        in[j] = kk[j] - t_lo <= t_hi - t_lo;         // t_lo <= key <= t_hi (key 0 < t_lo wraps high)
        me[j] = __ballot(in[j]);
      }
      if (store_eq) {
        if (lane == 0) {
          e_cnt[e] = (uint32_t)(__popcll(me[0]) + __popcll(me[1]) + __popcll(me[2]) + __popcll(me[3]));
          u32x4* e4 = (u32x4*)(m_eq + 4 * e);
          e4[0] = u32x4{(uint32_t)me[0], (uint32_t)(me[0] >> 32), (uint32_t)me[1], (uint32_t)(me[1] >> 32)};
          e4[1] = u32x4{(uint32_t)me[2], (uint32_t)(me[2] >> 32), (uint32_t)me[3], (uint32_t)(me[3] >> 32)};
        }
      } else {
        const uint32_t c0 = (uint32_t)__popcll(me[0]), c1 = (uint32_t)__popcll(me[1]);
        const uint32_t c2 = (uint32_t)__popcll(me[2]), c3 = (uint32_t)__popcll(me[3]);
        const uint32_t tot = c0 + c1 + c2 + c3;
        if (tot) {                                   // uniform
          uint32_t base;
          if (per_wave) {
            base = wave * kCandPerWave + wcount;
            wcount += tot;
          } else {
            uint32_t b0 = 0;
            if (lane == 0) b0 = atomicAdd(&cand_n, tot);
            base = __builtin_amdgcn_readfirstlane(b0);
          }
          const uint32_t pre[4] = {base, base + c0, base + c0 + c1, base + c0 + c1 + c2};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (in[j]) {
              const uint32_t pos = pre[j] + mbcnt(me[j]);
              cand_key[pos] = kk[j];
              cand_col[pos] = (uint32_t)(4 * vi + j);
            }
          }
        }
      }
    }
  };
#pragma unroll
  for (int it = 0; it < V; ++it) classify(key[it], it * kThreads + tid);
  tail_pass(classify);
  if (lane == 0) wave_cnt[wave] = wcount;
  __syncthreads();

  // ---- the exact threshold among the candidates, and the candidates' mask bits and counts
  if (gather) {
    uint32_t T;
    auto fix = [&, cand_key, cand_col](int j) {
      const uint32_t u = cand_key[j], v = cand_col[j];
      const int mi = (int)(v >> 8) * 4 + (int)(v & 3);
      const uint64_t bit = 1ull << ((v >> 2) & 63);
      if (u >= T) {   // one LDS word offset picks the mask and count array (no pointer select)
        const int which = u > T ? 0 : 1;
        atomicOr((unsigned long long*)&big[kOffGt + which * (kOffEq - kOffGt) + 2 * mi], bit);
        atomicAdd(&big[kOffCnt + which * kMaxChunks + (int)(v >> 8)], 1u);
      }
    };
    if (per_wave) {
      // every wave selects T on its own from all <= kCandPerWave candidates (8 per lane at most),
      // then fixes up the candidates of its own region
      uint32_t rb[kWaves + 1];
      rb[0] = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) rb[w + 1] = rb[w] + wave_cnt[w];
      constexpr int kPerLane = (kCandPerWave + 63) / 64;
      uint32_t c[kPerLane];
#pragma unroll
      for (int r = 0; r < kPerLane; ++r) {
        const uint32_t g = (uint32_t)(r * 64 + lane);
        int w = 0;
#pragma unroll
        for (int ww = 1; ww < kWaves; ++ww) w += g >= rb[ww];
        c[r] = g < cnt ? cand_key[w * kCandPerWave + (g - rb[w])] : 0u;
      }
      if (cnt <= 64u) {
        uint32_t cgt = 0, cge = 0;
        for (int j = 0; j < (int)cnt; ++j) {         // lane j's key, read into a scalar register
          const uint32_t q = (uint32_t)__builtin_amdgcn_readlane((int)c[0], j);
          cgt += q > c[0];
          cge += q >= c[0];
        }
        const uint64_t m = __ballot(lane < (int)cnt && cgt < kr && kr <= cge);
        const int src = (int)__builtin_ctzll(m | (1ull << 63));
        T = (uint32_t)__builtin_amdgcn_readlane((int)c[0], src);
        kr -= (uint32_t)__builtin_amdgcn_readlane((int)cgt, src);
      } else {
        uint32_t* wh = shist + wave * 256;           // this wave's 256-bin histogram
        while (plen < 32) {
          const int D = min(8, 32 - plen);
          const int shift = 32 - plen - D;
          ((u32x4*)wh)[lane] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
          for (int r = 0; r < kPerLane; ++r)
            if (c[r] && (c[r] & pmask) == pval) atomicAdd(&wh[__builtin_amdgcn_ubfe(c[r], shift, D)], 1u);
          uint32_t bin, ab, bc;
          wave_select<4>(wh, kr, bin, ab, bc);       // bins past 2^D hold nothing
          kr -= ab;
          plen += D;
          pmask = plen == 32 ? ~0u : ~0u << (32 - plen);
          pval |= bin << shift;
        }
        T = pval;
      }
      for (int j = lane; j < (int)wave_cnt[wave]; j += 64) fix(wave * kCandPerWave + j);
    } else {
      auto cand_keys = [&](auto&& visit) {
        const int nc = (int)cand_n;
        for (int j = tid; j < nc; j += kThreads) visit(cand_key[j]);
      };
      while (plen < 32) {
        const int D = min(kSmallBits, 32 - plen);
        const int shift = 32 - plen - D;
        uint32_t ab, c;
        const uint32_t bin = radix_round(cand_keys, pmask, pval, shift, D, kr, shist, red, sel, &ab, &c);
        kr -= ab;
        plen += D;
        pmask = plen == 32 ? ~0u : ~0u << (32 - plen);
        pval |= bin << shift;
      }
      T = pval;
      const int nc = (int)cand_n;
      for (int j = tid; j < nc; j += kThreads) fix(j);
    }
    __syncthreads();
  }

  // ---- order-preserving output.  Chunk offsets: a scan of the chunks' counts in column
  // order.  Then 64-column groups (chunk e, lane bit j: columns e*256 + 4l + j) are walked one
  // per thread; a winner's offset in its chunk counts the chunk's set bits in lower lanes and
  // in lower j of its own lane.
  uint32_t* pre_g = big + kOffCandKey;               // the candidates are no longer needed
  uint32_t* pre_e = pre_g + kMaxChunks;
  {
    // thread t scans the chunks [t*C, t*C + C) in one block-wide pass
    constexpr int C = (kMaxChunks + kThreads - 1) / kThreads;
    uint32_t gc[C], ec[C], gs = 0, es = 0;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int e = tid * C + c;
      gc[c] = e < nch ? g_cnt[e] : 0u;
      ec[c] = e < nch ? e_cnt[e] : 0u;
      gs += gc[c];
      es += ec[c];
    }
    uint32_t gb = block_incl_scan(gs, red) - gs;
    uint32_t eb = block_incl_scan(es, red) - es;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int e = tid * C + c;
      if (e < nch) {
        pre_g[e] = gb;
        pre_e[e] = eb;
      }
      gb += gc[c];
      eb += ec[c];
    }
    __syncthreads();
  }
  const int P = p.P;
  const bool p_pow2 = (P & (P - 1)) == 0;
  const int p_shift = __ffs(P) - 1;
  // the page lookup is chosen once for the whole walk (LDS copy or global row), so that each
  // load keeps its own address space
  auto walk = [&](auto page_of) {
  for (int q = tid; q < 4 * nch; q += kThreads) {
    const int e = q >> 2, j = q & 3;
    uint64_t mg[4], me[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      mg[jj] = m_gt[4 * e + jj];
      me[jj] = m_eq[4 * e + jj];
    }
    const uint32_t G = pre_g[e], E = pre_e[e];
    const uint64_t mgj = j == 0 ? mg[0] : j == 1 ? mg[1] : j == 2 ? mg[2] : mg[3];
    const uint64_t mej = j == 0 ? me[0] : j == 1 ? me[1] : j == 2 ? me[2] : me[3];
    uint64_t bits = mgj | mej;
    while (bits) {
      const int l = __builtin_ctzll(bits);
      bits &= bits - 1;
      const uint64_t lt = (1ull << l) - 1;
      uint32_t gb = G, eb = E;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        gb += (uint32_t)__popcll(mg[jj] & lt) + (jj < j ? (uint32_t)(mg[jj] >> l) & 1u : 0u);
        eb += (uint32_t)__popcll(me[jj] & lt) + (jj < j ? (uint32_t)(me[jj] >> l) & 1u : 0u);
      }
      bool take;
      uint32_t pos;
      if ((mgj >> l) & 1) {
        take = true;
        pos = gb + min(eb, kr);
      } else {
        take = eb < kr;
        pos = gb + eb;
      }
      if (take && pos < (uint32_t)k) {
        const int t = e * kChunkCols + 4 * l + j - o;
        idx_out[pos] = t;
        if (slot_out) {
          const int pg = p_pow2 ? t >> p_shift : t / P;
          const int off = t - pg * P;
          slot_out[pos] = page_of(pg) * P + off;
        }
      }
    }
  }
  };
  if (cache_pages) walk([&](int pg) { return big[kOffPtab + pg]; });
  else walk([&](int pg) { return ptab[pg]; });
}

__global__ __launch_bounds__(256) void page_map_kernel(const int32_t* idx, int64_t total, int k, int Q,
                                                       const int32_t* pt, int maxP, int P, int32_t* slots) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= total) return;
  const int64_t row = g / k;
  const int b = (int)(row / Q);
  const int t = idx[g];
  slots[g] = t < 0 ? -1 : pt[(int64_t)b * maxP + t / P] * P + t % P;
}

}  // namespace

size_t topk_workspace_bytes(int64_t rows, int max_seq_len) {
  (void)rows;
  (void)max_seq_len;
  return 0;
}

hipError_t launch_topk(const TopkParams& p, int rows, int max_seq_len, void* ws, hipStream_t s) {
  (void)ws;
  // 4, 8 or 16 float4 per thread stay in registers (up to 32K columns, plus up to 3 leading
  // columns of the aligned view); columns past that are re-read from L2 in each pass.
  const dim3 grid((unsigned)rows), block(kThreads);
  const int nv = max_seq_len + 3;
  constexpr int kMaxV = kThreads >= 1024 ? 8 : 16;
  if (nv <= 4 * 4 * kThreads) hipLaunchKernelGGL(topk_kernel<4>, grid, block, 0, s, p);
  else if (nv <= 8 * 4 * kThreads || kMaxV == 8) hipLaunchKernelGGL(topk_kernel<8>, grid, block, 0, s, p);
  else hipLaunchKernelGGL(topk_kernel<kMaxV>, grid, block, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_page_map(const int32_t* idx, int64_t total, int k, int Q, const int32_t* pt, int maxP,
                           int P, int32_t* slots, hipStream_t s) {
  if (total == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(page_map_kernel, dim3(blocks), dim3(256), 0, s, idx, total, k, Q, pt, maxP, P, slots);
  return hipGetLastError();
}

}  // namespace dsa
