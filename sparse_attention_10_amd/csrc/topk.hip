// Top-k selection and page mapping on gfx950 (the "top-k + page-mapping transforms" kernel group
// of "GLM-52 Runs on RTX 4090", section "how did he do it"; the fused page-map variant is the
// README's SGLANG_NSA_FUSE_TOPK option, renning22/glm-5.2-4090, usage section).
//
// One 1024-thread workgroup per query row:
//   1. scores -> order-preserving uint32 keys (-0.0 folded onto +0.0, so equal floats give
//      equal keys); the first ITEMS*1024 keys of the row (ITEMS <= 32) stay in registers, any
//      rest is re-read from L2 on each pass.
//   2. AND/OR reduction gives the bits all visible keys share; radix select then resolves
//      the k-th largest key 11 bits at a time from the first bit that differs, with an LDS
//      histogram per round.  If a round's winning bin holds exactly the missing count, the
//      selection is complete without resolving lower bits.
//   3. Order-preserving compaction: every (iteration, wave) block of 64 consecutive tokens
//      counts its "greater" and "equal" members with ballots; one scan over that table gives
//      each token its output position, so winners come out in ascending token order and equal
//      keys are taken lowest index first.  The page map is applied on the same store.
#include "dsa_internal.hpp"

namespace dsa {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBits = 11;
constexpr int kBins = 1 << kBits;
constexpr int kMaxIt = kMaxTopkSeq / kThreads;    // 256 iterations of 1024 tokens

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  u = (u == 0x80000000u) ? 0u : u;                 // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ uint32_t mbcnt(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Inclusive scan of one value per thread over the 1024-thread block.  `wsum` is LDS [kWaves].
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t t = __shfl_up(v, off);
    if (lane >= off) v += t;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  if (wave == 0) {
    uint32_t x = lane < kWaves ? wsum[lane] : 0u;
#pragma unroll
    for (int off = 1; off < kWaves; off <<= 1) {
      uint32_t t = __shfl_up(x, off);
      if (lane >= off) x += t;
    }
    if (lane < kWaves) wsum[lane] = x;
  }
  __syncthreads();
  const uint32_t pre = wave ? wsum[wave - 1] : 0u;
  if (total) *total = wsum[kWaves - 1];
  __syncthreads();
  return v + pre;
}

__device__ __forceinline__ uint32_t block_and_or(uint32_t a, uint32_t o, uint32_t* red, uint32_t* or_out) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    a &= __shfl_xor(a, off);
    o |= __shfl_xor(o, off);
  }
  if (lane == 0) {
    red[wave] = a;
    red[kWaves + wave] = o;
  }
  __syncthreads();
  uint32_t A = ~0u, O = 0u;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    A &= red[w];
    O |= red[kWaves + w];
  }
  __syncthreads();
  *or_out = O;
  return A;
}

// high `plen` bits of u (0 when plen == 0)
__device__ __forceinline__ uint32_t hi_bits(uint32_t u, int plen) {
  return (uint32_t)((uint64_t)u >> (32 - plen));
}

template <int ITEMS>
__global__ __launch_bounds__(kThreads) void topk_kernel(TopkParams p) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t tbl_gt[kMaxIt * kWaves];
  __shared__ uint32_t tbl_eq[kMaxIt * kWaves];
  __shared__ uint32_t red[2 * kWaves];
  __shared__ uint32_t sel_bin, sel_above;

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

  const float* srow = p.scores + (int64_t)row * p.ld;
  const int n_reg = min(n, ITEMS * kThreads);
  uint32_t key[ITEMS];
  uint32_t a_acc = ~0u, o_acc = 0u;
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const int e = it * kThreads + tid;
    key[it] = 0u;
    if (e < n_reg) {
      key[it] = order_key(srow[e]);
      a_acc &= key[it];
      o_acc |= key[it];
    }
  }
  for (int e = ITEMS * kThreads + tid; e < n; e += kThreads) {
    const uint32_t u = order_key(srow[e]);
    a_acc &= u;
    o_acc |= u;
  }
  uint32_t OR;
  const uint32_t AND = block_and_or(a_acc, o_acc, red, &OR);
  const uint32_t diff = AND ^ OR;
  int plen = diff ? __clz(diff) : 32;               // leading bits shared by every key
  uint32_t prefix = hi_bits(AND, plen);
  int kr = k;                                      // rank still to resolve among the candidates
  bool take_all = false;

  while (plen < 32) {
    const int D = min(kBits, 32 - plen);
    const int shift = 32 - plen - D;
    const int nb = 1 << D;
    const uint32_t mask = (uint32_t)nb - 1u;
    for (int j = tid; j < nb; j += kThreads) hist[j] = 0u;
    __syncthreads();
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int e = it * kThreads + tid;
      if (e < n_reg && hi_bits(key[it], plen) == prefix) atomicAdd(&hist[(key[it] >> shift) & mask], 1u);
    }
    for (int e = ITEMS * kThreads + tid; e < n; e += kThreads) {
      const uint32_t u = order_key(srow[e]);
      if (hi_bits(u, plen) == prefix) atomicAdd(&hist[(u >> shift) & mask], 1u);
    }
    __syncthreads();
    // thread t looks at bins hb = nb-1-2t and hb-1, scanning from the top bin down
    const int hb = nb - 1 - 2 * tid;
    const uint32_t c0 = hb >= 0 ? hist[hb] : 0u;
    const uint32_t c1 = hb - 1 >= 0 ? hist[hb - 1] : 0u;
    const uint32_t incl = block_incl_scan(c0 + c1, red, nullptr);
    const uint32_t above = incl - c0 - c1;          // candidates in bins above hb
    if (hb >= 0 && above < (uint32_t)kr && above + c0 >= (uint32_t)kr) {
      sel_bin = (uint32_t)hb;
      sel_above = above;
    } else if (hb - 1 >= 0 && above + c0 < (uint32_t)kr && above + c0 + c1 >= (uint32_t)kr) {
      sel_bin = (uint32_t)(hb - 1);
      sel_above = above + c0;
    }
    __syncthreads();
    const uint32_t d = sel_bin;
    const uint32_t cnt = hist[d];
    prefix = (prefix << D) | d;
    plen += D;
    kr -= (int)sel_above;
    __syncthreads();
    if ((int)cnt == kr) {                           // the whole bin is selected
      take_all = true;
      break;
    }
  }

  // ---- order-preserving compaction
  const int nit = (n + kThreads - 1) / kThreads;
  auto classify = [&](uint32_t u, bool valid, uint64_t* gm, uint64_t* em) {
    const uint32_t h = hi_bits(u, plen);
    *gm = __ballot(valid && h > prefix);
    *em = __ballot(valid && h == prefix);
  };
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    if (it < nit) {
      uint64_t gm, em;
      classify(key[it], it * kThreads + tid < n_reg, &gm, &em);
      if (lane == 0) {
        tbl_gt[it * kWaves + wave] = __popcll(gm);
        tbl_eq[it * kWaves + wave] = __popcll(em);
      }
    }
  }
  for (int it = ITEMS; it < nit; ++it) {
    const int e = it * kThreads + tid;
    const uint32_t u = e < n ? order_key(srow[e]) : 0u;
    uint64_t gm, em;
    classify(u, e < n, &gm, &em);
    if (lane == 0) {
      tbl_gt[it * kWaves + wave] = __popcll(gm);
      tbl_eq[it * kWaves + wave] = __popcll(em);
    }
  }
  __syncthreads();
  // exclusive scan of the table in token order; each thread owns up to 4 consecutive entries
  {
    const int ne = nit * kWaves;
    const int per = (ne + kThreads - 1) / kThreads;   // <= 4
    uint32_t g[4], q[4], sg = 0, sq = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = tid * per + c;
      g[c] = (c < per && e < ne) ? tbl_gt[e] : 0u;
      q[c] = (c < per && e < ne) ? tbl_eq[e] : 0u;
      sg += g[c];
      sq += q[c];
    }
    uint32_t xg = block_incl_scan(sg, red, nullptr) - sg;
    uint32_t xq = block_incl_scan(sq, red, nullptr) - sq;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = tid * per + c;
      if (c < per && e < ne) {
        tbl_gt[e] = xg;
        tbl_eq[e] = xq;
      }
      xg += g[c];
      xq += q[c];
    }
  }
  __syncthreads();
  auto emit = [&](int it, uint32_t u, bool valid) {
    uint64_t gm, em;
    classify(u, valid, &gm, &em);
    const uint32_t h = hi_bits(u, plen);
    const bool gt = valid && h > prefix, eq = valid && h == prefix;
    const uint32_t gb = tbl_gt[it * kWaves + wave] + mbcnt(gm);
    const uint32_t eb = tbl_eq[it * kWaves + wave] + mbcnt(em);
    if (gt || (eq && (take_all || eb < (uint32_t)kr))) {
      const uint32_t pos = gb + (take_all ? eb : min(eb, (uint32_t)kr));
      const int t = it * kThreads + tid;
      if (pos < (uint32_t)k) {
        idx_out[pos] = t;
        if (slot_out) slot_out[pos] = ptab[t / p.P] * p.P + t % p.P;
      }
    }
  };
#pragma unroll
  for (int it = 0; it < ITEMS; ++it)
    if (it < nit) emit(it, key[it], it * kThreads + tid < n_reg);
  for (int it = ITEMS; it < nit; ++it) {
    const int e = it * kThreads + tid;
    emit(it, e < n ? order_key(srow[e]) : 0u, e < n);
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
  const dim3 grid((unsigned)rows), block(kThreads);
  // At most 32 keys per thread stay in registers (the 32-key variant already fills the 128
  // VGPRs a 1024-thread workgroup allows); keys past 32K are re-read from L2 on each pass, so no
  // variant needs scratch memory.
  if (max_seq_len <= 8 * kThreads) hipLaunchKernelGGL(topk_kernel<8>, grid, block, 0, s, p);
  else if (max_seq_len <= 16 * kThreads) hipLaunchKernelGGL(topk_kernel<16>, grid, block, 0, s, p);
  else hipLaunchKernelGGL(topk_kernel<32>, grid, block, 0, s, p);
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
