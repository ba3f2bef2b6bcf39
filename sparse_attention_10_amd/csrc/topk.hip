// Top-k selection and page mapping on gfx950 (the "top-k + page-mapping transforms" kernel group
// of "GLM-52 Runs on RTX 4090", section "how did he do it"; the fused page-map variant is the
// README's SGLANG_NSA_FUSE_TOPK option, renning22/glm-5.2-4090, usage section).
//
// One 512-thread workgroup per query row.  The selection is exact: equal scores go to the
// lower token index, -0.0 equals +0.0, winners come out in ascending token order.
//   1. Scores become order-preserving uint32 keys (larger score <-> larger key, key 0 marks a
//      column past the row).  The first ITEMS*512 keys stay in registers; the rest of a long
//      row is re-read from L2 on each pass.  The page-table row is cached in LDS.
//   2. The bits every key shares (AND/OR reduction) fix where the keys start to differ; one
//      11-bit LDS histogram of the next bits finds the bin holding the k-th largest key.
//   3. The keys of that bin are gathered into LDS (per-wave regions, no atomics).  For the
//      narrow score distributions the indexer produces the bin holds a few dozen keys and one
//      wave finds the exact threshold key T with no barrier; larger bins are radix-selected in
//      LDS, and a bin too large to gather falls back to radix rounds over the whole row.
//   4. One classification pass stores, per 64 consecutive columns, the ballot masks of keys
//      above T and equal to T.  A scan of their popcounts in column order gives each block its
//      output offset; each thread then walks the set bits of its blocks in ascending column
//      order, taking every key above T and the lowest-index keys equal to T until k are taken,
//      and writes the token index and (fused page map) its cache slot.
#include "dsa_internal.hpp"

namespace dsa {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kBits = 11;
constexpr int kBins = 1 << kBits;
constexpr int kMaxEntries = kMaxTopkSeq / 64;    // (iteration, wave) blocks of 64 columns
constexpr int kCandPerWave = 256;                // gathered keys per wave
constexpr int kCandCap = kCandPerWave * kWaves;
constexpr int kPtabCache = 4096;                 // page-table entries cached in LDS

// Order-preserving key of a float score: larger float <-> larger unsigned key.  Adding +0.0
// turns -0.0 into +0.0 (so the two compare equal) and leaves every other value unchanged.
// Finite scores and -inf map to keys >= 0x007FFFFF, so key 0 is free to mark "no score".
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ uint32_t mbcnt(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Inclusive scan of one value per thread over the workgroup.  `wsum` is LDS [kWaves].
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* wsum) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t t = __shfl_up(v, off);
    if (lane >= off) v += t;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  uint32_t pre = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) pre += w < wave ? wsum[w] : 0u;
  __syncthreads();
  return v + pre;
}

// Visit the keys of columns [start, n) in iteration order (iteration it covers columns
// it*512 .. it*512+511, this thread's column being it*512 + tid), 8 iterations per batch so
// that 8 loads are in flight at once.  f(key, it) runs for every iteration of every thread
// (uniformly, so it may hold ballots); key is 0 past column n-1.
template <typename F>
__device__ __forceinline__ void tail_pass(const float* srow, int start, int n, F&& f) {
  constexpr int kBatch = 8;
  for (int base = start; base < n; base += kBatch * kThreads) {
    float v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) v[u] = srow[min(base + u * kThreads + (int)threadIdx.x, n - 1)];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int e = base + u * kThreads + (int)threadIdx.x;
      if (base + u * kThreads < n)   // uniform: the iteration has at least one visible column
        f(e < n ? order_key(v[u]) : 0u, (base + u * kThreads) / kThreads);
    }
  }
}

// Histogram round over keys matching (pmask, pval): find the bin of the next D bits that holds
// the kr-th largest.  Returns the bin; *above receives the count in higher bins, *cnt the bin's
// own count.  `keys_fn(visitor)` visits every key of the candidate set.
template <typename KeysFn>
__device__ __forceinline__ uint32_t hist_round(KeysFn&& keys_fn, uint32_t pmask, uint32_t pval, int shift, int D,
                                               int kr, uint32_t* hist, uint32_t* red, uint32_t* sel,
                                               uint32_t* above, uint32_t* cnt) {
  const int tid = threadIdx.x;
  const int nb = 1 << D;
  for (int j = tid; j < nb; j += kThreads) hist[j] = 0u;
  __syncthreads();
  keys_fn([&](uint32_t u) {
    if (u && (u & pmask) == pval) atomicAdd(&hist[__builtin_amdgcn_ubfe(u, shift, D)], 1u);
  });
  __syncthreads();
  // thread t owns the 4 bins nb-1-4t .. nb-4-4t, scanning from the top bin down
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
    if (bin >= 0 && acc < (uint32_t)kr && acc + c[j] >= (uint32_t)kr) {
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

template <int ITEMS>
__global__ __launch_bounds__(kThreads) void topk_kernel(TopkParams p) {
  __shared__ uint64_t m_gt[kMaxEntries];          // per 64 columns: keys above the threshold
  __shared__ uint64_t m_eq[kMaxEntries];          // ... and keys equal to it (or in the final bin)
  __shared__ uint32_t cand[kCandCap];
  __shared__ uint32_t hist[kBins];
  __shared__ int32_t ptab_s[kPtabCache];
  __shared__ uint32_t red[2 * kWaves];
  __shared__ uint32_t sel[4];
  __shared__ uint32_t wave_cnt[kWaves];

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

  // ---- load: register-resident keys, the page-table row, the common bits
  const float* srow = p.scores + (int64_t)row * p.ld;
  const int npages = (n + p.P - 1) / p.P;
  const bool cache_pages = slot_out != nullptr && npages <= kPtabCache;
  uint32_t key[ITEMS];
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) key[it] = __float_as_uint(srow[min(it * kThreads + tid, n - 1)]);
  int32_t pv[kPtabCache / kThreads];
  if (cache_pages) {
#pragma unroll
    for (int u = 0; u < kPtabCache / kThreads; ++u) pv[u] = ptab[min(u * kThreads + tid, npages - 1)];
  }
  uint32_t a_acc = ~0u, o_acc = 0u;
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    key[it] = it * kThreads + tid < n ? order_key(__uint_as_float(key[it])) : 0u;
    a_acc &= key[it] ? key[it] : ~0u;
    o_acc |= key[it];
  }
  tail_pass(srow, ITEMS * kThreads, n, [&](uint32_t u, int) {
    a_acc &= u ? u : ~0u;
    o_acc |= u;
  });
  if (cache_pages) {
#pragma unroll
    for (int u = 0; u < kPtabCache / kThreads; ++u) ptab_s[u * kThreads + tid] = pv[u];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    a_acc &= __shfl_xor(a_acc, off);
    o_acc |= __shfl_xor(o_acc, off);
  }
  if (lane == 0) {
    red[wave] = a_acc;
    red[kWaves + wave] = o_acc;
  }
  __syncthreads();
  uint32_t AND = ~0u, OR = 0u;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    AND &= red[w];
    OR |= red[kWaves + w];
  }
  __syncthreads();

  auto all_keys = [&](auto&& visit) {
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) visit(key[it]);
    tail_pass(srow, ITEMS * kThreads, n, [&](uint32_t u, int) { visit(u); });
  };

  // Final selection: keys > t_hi are taken, keys in [t_lo, t_hi] are taken lowest column
  // first until kr of them are (all of them when take_all).
  int plen = (AND ^ OR) ? __clz(AND ^ OR) : 32;     // leading bits shared by every key
  uint32_t pmask = plen == 0 ? 0u : (plen == 32 ? ~0u : ~0u << (32 - plen));
  uint32_t pval = AND & pmask;
  int kr = k;
  bool take_all = false;
  bool gathered = false;                            // the final bin's keys sit in cand[]

  // ---- radix rounds over the whole row until the bin holding the k-th key is small enough
  while (plen < 32) {
    const int D = min(kBits, 32 - plen);
    const int shift = 32 - plen - D;
    uint32_t above, cnt;
    const uint32_t bin = hist_round(all_keys, pmask, pval, shift, D, kr, hist, red, sel, &above, &cnt);
    kr -= (int)above;
    plen += D;
    pmask = plen == 32 ? ~0u : ~0u << (32 - plen);
    pval |= bin << shift;
    if ((int)cnt == kr) {                           // the whole bin is selected
      take_all = true;
      break;
    }
    if (plen < 32 && cnt <= (uint32_t)kCandCap) {
      // ---- gather the bin's keys into per-wave LDS regions (offsets kept per wave, no atomics)
      uint32_t wcount = 0;
      all_keys([&](uint32_t u) {
        const bool c = u && (u & pmask) == pval;
        const uint64_t m = __ballot(c);
        const uint32_t at = wcount + mbcnt(m);
        if (c && at < (uint32_t)kCandPerWave) cand[wave * kCandPerWave + at] = u;
        wcount += (uint32_t)__popcll(m);
      });
      if (lane == 0) wave_cnt[wave] = wcount;
      __syncthreads();
      bool fits = true;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) fits = fits && wave_cnt[w] <= (uint32_t)kCandPerWave;
      if (fits) {
        gathered = true;
        break;
      }
      __syncthreads();
    }
  }

  if (gathered) {
    // candidates: cand[w*kCandPerWave + j] for j < wave_cnt[w]; all share the bin's prefix
    int ntot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) ntot += (int)wave_cnt[w];
    if (ntot <= 64) {
      // ---- one wave: the exact threshold among <= 64 keys, no barrier
      if (wave == 0) {
        int src_w = 0, src_j = lane;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {       // lane -> (wave region, position)
          const int c = (int)wave_cnt[w];
          if (src_w == w && src_j >= c) {
            src_j -= c;
            ++src_w;
          }
        }
        const bool have = lane < ntot;
        const uint32_t mine = have ? cand[src_w * kCandPerWave + src_j] : 0u;
        int cgt = 0, cge = 0;
        for (int j = 0; j < ntot; ++j) {
          const uint32_t o = __shfl(mine, j);
          cgt += o > mine;
          cge += o >= mine;
        }
        if (have && cgt < kr && kr <= cge) {
          sel[0] = mine;
          sel[1] = (uint32_t)(kr - cgt);
        }
      }
      __syncthreads();
      pval = sel[0];
      kr = (int)sel[1];
      pmask = ~0u;
      __syncthreads();
    } else {
      // ---- radix rounds over the gathered keys in LDS
      auto cand_keys = [&](auto&& visit) {
        for (int j = lane; j < kCandPerWave; j += 64) visit(j < (int)wave_cnt[wave] ? cand[wave * kCandPerWave + j] : 0u);
      };
      while (plen < 32) {
        const int D = min(kBits, 32 - plen);
        const int shift = 32 - plen - D;
        uint32_t above, cnt;
        const uint32_t bin = hist_round(cand_keys, pmask, pval, shift, D, kr, hist, red, sel, &above, &cnt);
        kr -= (int)above;
        plen += D;
        pmask = plen == 32 ? ~0u : ~0u << (32 - plen);
        pval |= bin << shift;
      }
    }
  }
  const uint32_t t_lo = pval, t_hi = pval | ~pmask;

  // ---- classify every column once; keep the ballots per 64 columns in LDS
  const int nit = (n + kThreads - 1) / kThreads;
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    if (it < nit) {
      const uint64_t gm = __ballot(key[it] > t_hi);
      const uint64_t em = __ballot(key[it] && key[it] >= t_lo && key[it] <= t_hi);
      if (lane == 0) {
        m_gt[it * kWaves + wave] = gm;
        m_eq[it * kWaves + wave] = em;
      }
    }
  }
  tail_pass(srow, ITEMS * kThreads, n, [&](uint32_t u, int it) {
    const uint64_t gm = __ballot(u > t_hi);
    const uint64_t em = __ballot(u && u >= t_lo && u <= t_hi);
    if (lane == 0) {
      m_gt[it * kWaves + wave] = gm;
      m_eq[it * kWaves + wave] = em;
    }
  });
  __syncthreads();

  // ---- order-preserving compaction: in rounds of 512 blocks (block = 64 columns), thread t
  // takes block r*512 + t; a scan of the blocks' counts (plus the carry of earlier rounds)
  // gives its output offsets, then it walks the block's set bits in ascending column order
  const int ne = nit * kWaves;
  const int P = p.P;
  const bool p_pow2 = (P & (P - 1)) == 0;
  const int p_shift = __ffs(P) - 1;
  uint32_t g_carry = 0, e_carry = 0;
  for (int r0 = 0; r0 < ne; r0 += kThreads) {
    const int e = r0 + tid;
    const uint64_t mg = e < ne ? m_gt[e] : 0ull, me = e < ne ? m_eq[e] : 0ull;
    const uint32_t g_cnt = (uint32_t)__popcll(mg), e_cnt = (uint32_t)__popcll(me);
    const uint32_t g_incl = block_incl_scan(g_cnt, red);
    uint32_t g_before = g_carry + g_incl - g_cnt;
    const uint32_t e_incl = block_incl_scan(e_cnt, red);
    uint32_t e_before = e_carry + e_incl - e_cnt;
    // round totals: the last thread's inclusive sums, shared through LDS
    if (tid == kThreads - 1) {
      sel[2] = g_incl;
      sel[3] = e_incl;
    }
    uint64_t any = mg | me;
    const int col0 = (e / kWaves) * kThreads + (e % kWaves) * 64;
    while (any) {
      const int bit = __builtin_ctzll(any);
      any &= any - 1;
      const uint64_t bm = 1ull << bit;
      uint32_t pos;
      bool take;
      if (mg & bm) {
        pos = g_before + (take_all ? e_before : min(e_before, (uint32_t)kr));
        take = true;
        ++g_before;
      } else {
        take = take_all || e_before < (uint32_t)kr;
        pos = g_before + e_before;
        ++e_before;
      }
      if (take && pos < (uint32_t)k) {
        const int t = col0 + bit;
        idx_out[pos] = t;
        if (slot_out) {
          const int pg = p_pow2 ? t >> p_shift : t / P;
          const int off = t - pg * P;
          slot_out[pos] = (cache_pages ? ptab_s[pg] : ptab[pg]) * P + off;
        }
      }
    }
    __syncthreads();
    g_carry += sel[2];
    e_carry += sel[3];
    __syncthreads();
  }
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

hipError_t launch_topk(const TopkParams& p, int rows, int max_seq_len, hipStream_t s) {
  // At most 64 keys per thread stay in registers (32K columns); keys past that are re-read
  // from L2 on each pass, so no variant needs scratch memory.
  const dim3 grid((unsigned)rows), block(kThreads);
  if (max_seq_len <= 16 * kThreads) hipLaunchKernelGGL(topk_kernel<16>, grid, block, 0, s, p);
  else if (max_seq_len <= 32 * kThreads) hipLaunchKernelGGL(topk_kernel<32>, grid, block, 0, s, p);
  else hipLaunchKernelGGL(topk_kernel<64>, grid, block, 0, s, p);
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
