// Lightning indexer on gfx950: s[b,i,t] = sum_h w[b,i,h] * ReLU(q[b,i,h,:] . k[slot(b,t),:]).
//
// The pages name this stage the "lightning-indexer GEMM" ("GLM-52 Runs on RTX 4090", section
// "how did he do it"; renning22/glm-5.2-4090 README, section "how it works").  Three kernels:
//
//  * indexer_reg_kernel (decode: 64 heads x 128 dims, bf16 q, bf16 or fp8 keys, one or two query
//    rows of a sequence per workgroup; more rows in groups of two whose workgroups share an XCD,
//    so the repeated key reads come from L2).  v_mfma_f32_16x16x32_bf16 with 16 heads as M and 16
//    tokens as N; keys stream HBM -> registers with 1 KB coalesced loads, turn around in a
//    per-wave LDS area into the operand layout, and every key is read once for all the rows of
//    its workgroup.  ReLU, head weights and the head sum stay in registers.
//  * indexer_prefill_kernel (many query rows per sequence, bf16 keys): 16 rows per workgroup
//    over a shared LDS ring of key stages, so each key byte feeds 16 rows and the matrix cores
//    bound the kernel.
//  * indexer_valu_kernel: any head count / dim / dtype pair, one token per thread, f32 math.
// fp8 keys are widened to bf16 exactly and their per-token scale multiplies the head sum (it is
// positive, so it commutes with the ReLU).
#include <algorithm>

#include "dsa_internal.hpp"

namespace dsa {

namespace {

template <typename T> struct Elt;
template <> struct Elt<float> {
  static __device__ __forceinline__ float get(const void* p, int64_t i) { return ((const float*)p)[i]; }
};
template <> struct Elt<__bf16> {
  static __device__ __forceinline__ float get(const void* p, int64_t i) {
    return bf16_bits_to_f32(((const uint16_t*)p)[i]);
  }
};
struct Fp8Tag {};
template <> struct Elt<Fp8Tag> {
  static __device__ __forceinline__ float get(const void* p, int64_t i) {
    return fp8_to_f32(((const uint8_t*)p)[i]);
  }
};

// ---------------------------------------------------------------------------------------------
// vector path

template <typename QT, typename KT>
__global__ __launch_bounds__(256) void indexer_valu_kernel(IndexerParams p) {
  extern __shared__ float sm[];   // q [Hi*Di] as f32, then w [Hi]
  const int b = blockIdx.z, i = blockIdx.y;
  const int Lb = p.seq_lens[b];
  if (threadIdx.x == 0 && blockIdx.x == 0 && i == 0) dbg_seq_len(p.dbg, Lb, p.Q, p.max_seq_len);
  const int L = min(Lb, p.max_seq_len);              // never write past the scores row
  const int pos = L - p.Q + i;
  const int t0 = blockIdx.x * 256;
  if (t0 >= L) return;   // whole block past the sequence (uniform)
  const int HD = p.Hi * p.Di;
  const int64_t row = (int64_t)b * p.Q + i;
  for (int e = threadIdx.x; e < HD; e += 256) sm[e] = Elt<QT>::get(p.q, row * HD + e);
  for (int e = threadIdx.x; e < p.Hi; e += 256) sm[HD + e] = p.w[row * p.Hi + e];
  __syncthreads();
  const int t = t0 + threadIdx.x;
  if (t >= L) return;
  float* out = p.scores + row * p.ld;
  if (t > pos) {
    out[t] = -INFINITY;
    return;
  }
  const int pe = dbg_page(p.dbg, p.page_table[(int64_t)b * p.maxP + t / p.P], p.num_slots, p.P);
  const int64_t slot = (int64_t)pe * p.P + t % p.P;
  const int64_t kbase = slot * p.Di;
  float acc = 0.f;
  for (int h = 0; h < p.Hi; ++h) {
    float dot = 0.f;
    for (int d = 0; d < p.Di; ++d) dot = fmaf(sm[h * p.Di + d], Elt<KT>::get(p.k_cache, kbase + d), dot);
    acc = fmaf(sm[HD + h], fmaxf(dot, 0.f), acc);
  }
  if (p.k_scale) acc *= p.k_scale[slot];
  out[t] = acc;
}

// ---------------------------------------------------------------------------------------------
// shared by the matrix-core kernels (Hi = 64, Di = 128)

constexpr int kHi = 64, kDi = 128;
constexpr int kSub = 32;                  // tokens per sub-tile of the prefill kernel (its MFMA N)

// 16-byte piece slot swizzle of a key row staged in LDS (bank-conflict-free operand reads)
template <bool FP8>
__device__ __forceinline__ int swz(int r) { return FP8 ? ((r >> 1) & 7) : (r & 15); }

// Inclusive prefix sum of one int per lane over a wave.
__device__ __forceinline__ int wave_incl_scan_i(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o);
    v += lane >= o ? u : 0;
  }
  return v;
}

// ---------------------------------------------------------------------------------------------
// matrix-core path for many query rows per sequence (a chunked prefill): Hi = 64, Di = 128, bf16
// q and keys, pages of a multiple of 32 tokens
//
// One workgroup = 16 query rows x one key range, 8 waves (two per SIMD): wave w scores the rows
// 2w and 2w+1 (q of 2 rows x 64 heads in registers, 4 M-blocks of 32 heads) against every key
// of the range.  Keys go HBM -> LDS by direct copies into a ring of 32-token stages (the decode
// kernel's swizzled row layout) and each is read once per workgroup for all 16 rows: a key byte
// feeds 16 x 64 flops, so the matrix cores bound the kernel, not the key stream (the keys of a
// chunk are shared by all its workgroups and come from L2 or the Infinity Cache).  Per 32-token
// sub-tile a wave reads its B fragments once and runs the 16 MFMAs of each of its rows; the two
// waves of a SIMD cover each other's head reductions, copies and barrier waits.

constexpr int kPfQB = 16;                        // query rows per workgroup
constexpr int kPfWaves = 8;
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kPfQW = kPfQB / kPfWaves;          // rows per wave
constexpr int kPfST = 32;                        // tokens per stage (one sub-tile: the registers of
                                                 // two would not fit beside two rows of q)
constexpr int kPfSPB = 4;                        // stages computed per barrier
constexpr int kPfNB = 3 * kPfSPB;                // ring stages
constexpr int kPfSB = kPfST * 2 * kDi;           // stage bytes (8 KB)
constexpr int kPfND = kPfSB / (kPfThreads * 16); // 16-byte copies per thread per stage
constexpr int kPfMaxPages = 2048;                // page-table entries of one key range

struct PfSmem {
  uint8_t ring[kPfNB][kPfSB];
  float w[kPfQB][kHi];
  int32_t pt[kPfMaxPages];
};

__global__ __launch_bounds__(kPfThreads) void indexer_prefill_kernel(IndexerParams p) {
  __shared__ __attribute__((aligned(16))) PfSmem sm;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // id = (b * ranges + range) * query blocks + query block; the blocks cover the rows
  // q_begin .. q_begin + q_count - 1 of each sequence
  const int nqb = (p.q_count + kPfQB - 1) / kPfQB;
  const int qb = (int)blockIdx.x % nqb;
  const int rest = (int)blockIdx.x / nqb;
  const int kr = rest % p.groups, b = rest / p.groups;
  const int Lb = p.seq_lens[b];
  if (threadIdx.x == 0 && kr == 0 && qb == 0) dbg_seq_len(p.dbg, Lb, p.Q, p.max_seq_len);
  const int L = min(Lb, p.max_seq_len);
  const int q_end = p.q_begin + p.q_count;
  const int q0 = p.q_begin + qb * kPfQB;
  const int nq = min(kPfQB, q_end - q0);           // rows of this block
  const int t_begin = kr * p.tiles_per_wg * kPfST;
  const int t_end = min(L, t_begin + p.tiles_per_wg * kPfST);
  if (t_begin >= t_end) return;                    // uniform
  const int pos_last = L - p.Q + q0 + nq - 1;      // the block's largest position
  const int t_stop = min(t_end, pos_last + 1);     // tokens at or past this are never scored
  const int nstage = t_stop > t_begin ? (t_stop - t_begin + kPfST - 1) / kPfST : 0;
  const int P = p.P;
  const int page0 = t_begin / P;
  const int npg = t_stop > t_begin ? (t_stop - 1) / P - page0 + 1 : 0;
  const int32_t* ptab_g = p.page_table + (int64_t)b * p.maxP;
  const __amdgpu_buffer_rsrc_t k_rs = rows_rsrc(p.k_cache, 2 * kDi, p.num_slots);
  const int n_in_sub = lane & 31, half = lane >> 5;

  // copy c of this thread fills LDS bytes ((c*8 + wave)*64 + lane)*16 of the stage: row r, slot
  // q, from piece q ^ swz(r) of the row; a copy's 4 rows lie in one 32-token run of one page
  int lane_row[kPfND], lane_boff[kPfND];
#pragma unroll
  for (int c = 0; c < kPfND; ++c) {
    const int off = ((c * kPfWaves + wave) * 64 + lane) * 16;
    const int r = off / (2 * kDi), q = (off % (2 * kDi)) / 16;
    lane_row[c] = r;
    lane_boff[c] = 16 * (q ^ swz<false>(r));
  }
  // page and in-page offset of copy c's run in the next stage to request, stepped by kPfST
  // tokens per stage (P is a multiple of 32: at most two page steps)
  int lk_pg[kPfND], lk_of[kPfND];
#pragma unroll
  for (int c = 0; c < kPfND; ++c) {
    const int ts = t_begin + (lane_row[c] & ~(kSub - 1));
    lk_pg[c] = ts / P;
    lk_of[c] = ts - lk_pg[c] * P;
  }
  int lk_t0 = t_begin;                             // first token of the next stage to request
  // copies of the next stage into `dst` (cache rows through pt_of), in stage order
  auto issue = [&](uint8_t* __restrict__ dst, auto&& pt_of) {
#pragma unroll
    for (int c = 0; c < kPfND; ++c) {
      const int ts = lk_t0 + (lane_row[c] & ~(kSub - 1));
      // (runs past the scored tokens read row 0: valid, never scored)
      const int s0 = ts < t_stop ? __builtin_amdgcn_readfirstlane(pt_of(lk_pg[c]) * P + lk_of[c]) : 0;
      lds_dma16_row(k_rs, s0 + (lane_row[c] & (kSub - 1)), lane_boff[c],
                    dst + ((c * kPfWaves + wave) * 64) * 16);
      lk_of[c] += kPfST;
#pragma unroll
      for (int u = 0; u < 2; ++u)
        if (lk_of[c] >= P) {
          lk_of[c] -= P;
          ++lk_pg[c];
        }
    }
    lk_t0 += kPfST;
  };
  auto pt_global = [&](int pg) { return dbg_page(p.dbg, ptab_g[pg], p.num_slots, P); };
#pragma unroll
  for (int v = 0; v < kPfNB - kPfSPB; ++v)
    if (v < nstage) issue(sm.ring[v], pt_global);

  // q of this wave's rows (clamped into the chunk; rows past it are computed, never stored):
  // lane (head m of M-block mb, half h) holds dims h*64 + s*8 .. +8 for step s
  bf16x8 afrag[kPfQW][2][8];
#pragma unroll
  for (int qi = 0; qi < kPfQW; ++qi) {
    const int row = min(q0 + wave * kPfQW + qi, q_end - 1);
    const __bf16* qrow = (const __bf16*)p.q + ((int64_t)b * p.Q + row) * kHi * kDi;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int s = 0; s < 8; ++s)
        afrag[qi][mb][s] = *(const bf16x8*)(qrow + (mb * 32 + n_in_sub) * kDi + half * 64 + s * 8);
  }
  for (int e = threadIdx.x; e < kPfQB * kHi; e += kPfThreads) {
    const int row = min(q0 + e / kHi, q_end - 1);
    (&sm.w[0][0])[e] = p.w[((int64_t)b * p.Q + row) * kHi + e % kHi];
  }
  for (int e = threadIdx.x; e < npg; e += kPfThreads) sm.pt[e] = dbg_page(p.dbg, ptab_g[page0 + e], p.num_slots, P);
  __syncthreads();

  float* out_b = p.scores + ((int64_t)b * p.q_count + (q0 - p.q_begin)) * p.ld;
  // head reduction of row qi's 32 tokens (acc) at token t; weights from LDS
  auto finish = [&](const PfSmem* __restrict__ rd, const f32x16 (&acc)[2], int qi, int t) {
    const float* wrow = rd->w[wave * kPfQW + qi];
    float part = 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 wv = *(const f32x4*)&wrow[mb * 32 + g * 8 + half * 4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)   // ReLU as one integer max on the bits (negatives -> +0)
          part = fmaf(wv[jj], __int_as_float(max(__float_as_int(acc[mb][4 * g + jj]), 0)), part);
      }
    // add the other lane half's partial sum (lanes l and l ^ 32 hold the same token)
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
    part = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    const int ri = wave * kPfQW + qi;
    const int pos = L - p.Q + q0 + ri;
    if (half == 0 && ri < nq && t < t_end) out_b[(int64_t)ri * p.ld + t] = t <= pos ? part : -INFINITY;
  };
  // stage v: B fragments once, then each row's 16 MFMAs and reduction
  auto compute = [&](const PfSmem* __restrict__ rd, int v) {
    const uint8_t* stg = rd->ring[v % kPfNB];
#pragma unroll
    for (int j = 0; j < kPfST / kSub; ++j) {
      const uint8_t* rows = stg + j * kSub * 2 * kDi;
      bf16x8 kf[8];
#pragma unroll
      for (int s = 0; s < 8; ++s)               // dims h*64 + 8s .. +8 = piece 8h + s
        kf[s] = *(const bf16x8*)(rows + n_in_sub * 2 * kDi + 16 * ((8 * half + s) ^ swz<false>(n_in_sub)));
      const int t = t_begin + v * kPfST + j * kSub + n_in_sub;
#pragma unroll
      for (int qi = 0; qi < kPfQW; ++qi) {
        f32x16 acc[2] = {f32x16{}, f32x16{}};
        // raised priority while issuing the row's MFMAs; the other wave of the SIMD runs its
        // head reduction meanwhile (c4 indexer 3755 -> 3485 us)
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int s = 0; s < 8; ++s)
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
            acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag[qi][mb][s], kf[s], acc[mb], 0, 0, 0);
        __builtin_amdgcn_s_setprio(0);
        finish(rd, acc, qi, t);
      }
    }
  };
  auto pt_lds = [&](const PfSmem* __restrict__ rd) { return [rd, page0](int pg) { return rd->pt[pg - page0]; }; };
  // kPfSPB stages per barrier, computed while the next 2 kPfSPB are in flight
  for (int v = 0; v < nstage; v += kPfSPB) {
    // stages v .. v+SPB-1 must have landed: the copies of the later stages requested so far
    // may still be outstanding (vector-memory operations complete in order)
    wait_vmcnt_later<kPfND, kPfNB - 2 * kPfSPB>(min(v + kPfNB - kPfSPB, nstage) - min(v + kPfSPB, nstage));
    lds_barrier();   // those stages landed for every wave; the previous ones are no longer read
#pragma unroll
    for (int u = kPfNB - kPfSPB; u < kPfNB; ++u)
      if (v + u < nstage) issue(sm.ring[(v + u) % kPfNB], pt_lds(&sm));
#pragma unroll
    for (int u = 0; u < kPfSPB; ++u) {
      if (v + u < nstage) compute(&sm, v + u);
      __builtin_amdgcn_sched_barrier(0);   // (keeps the stages' registers apart)
    }
  }
  // tokens of [t_begin, t_end) past the block's last position: -inf (their stages are not
  // computed)
  const int t_tail = max(t_stop, t_begin), n_tail = t_end - t_tail;
  for (int e = threadIdx.x; e < nq * n_tail; e += kPfThreads)
    out_b[(int64_t)(e / n_tail) * p.ld + t_tail + e % n_tail] = -INFINITY;
}

// ---------------------------------------------------------------------------------------------
// matrix-core decode path, keys through registers (Hi = 64, Di = 128, bf16 q, bf16 or fp8 keys;
// QB query rows of one sequence per workgroup)
//
// The contraction runs on v_mfma_f32_16x16x32_bf16 with 16 heads as M and a block of 16
// consecutive tokens as N, so each lane ends with 4 heads of one token per M-block: ReLU, the
// head weights and the sum over the lane's 16 heads of a row stay in registers, and the four
// lane groups add up with two row swaps.  The fp8 per-token scale multiplies the head sum (it is
// positive, so it commutes with the ReLU).
//
// Keys: a workgroup owns QB query rows and a range of 16-token blocks of one sequence; its waves
// take the blocks in turn (wave w: blocks w, w + NW, ...), each keeping the loads of D blocks in
// flight in a register ring.  Every load instruction reads 1 KB of whole key rows (lane i: 16
// bytes at 16i), the access pattern that streams fastest from HBM.  Each wave then turns its
// block around in a private 2-4 KB LDS area (written in load order, read in the MFMA operand
// layout, 16-byte pieces XOR-swizzled per row): a wave's LDS accesses complete in order, so this
// needs no barrier, and the waves never wait for each other after the initial staging of q
// (rows padded so the A-fragment reads are free of bank conflicts), w and the range's
// page-table entries.  The contraction index is permuted to the layout: in k-step s, lane group
// g holds dims 32g + 8s .. +8 (q the same way); fp8 keys are widened to bf16 exactly.

constexpr int kRB = 16;                 // tokens per block (the MFMA N)
constexpr int kQPitch = kDi + 8;        // bf16 per staged q row
constexpr int kRegMaxPages = 1024;      // page-table entries staged per workgroup

template <bool FP8, int QB, int NW>
struct RSmem {
  uint8_t tr[NW][kRB * (FP8 ? kDi : 2 * kDi)];   // per-wave turnaround of one key block
  __bf16 q[QB][kHi][kQPitch];
  float w[QB][kHi];
  int32_t pt[kRegMaxPages];
  int32_t part[24];
};

// Sum / inclusive prefix sum of one int per thread over an NW-wave workgroup (red: >= NW ints).
template <int NW>
__device__ __forceinline__ int wg_incl_scan(int v, int32_t* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int w = wave_incl_scan_i(v);
  if (lane == 63) red[wave] = w;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int k = 0; k < NW; ++k) before += k < wave ? red[k] : 0;
  __syncthreads();
  return w + before;
}
template <int NW>
__device__ __forceinline__ int wg_sum(int v, int32_t* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int w = wave_incl_scan_i(v);
  if (lane == 63) red[wave] = w;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int k = 0; k < NW; ++k) t += red[k];
  __syncthreads();
  return t;
}

template <bool FP8, bool CT, int QB, int NW, int D>
__global__ __launch_bounds__(NW * 64) void indexer_reg_kernel(IndexerParams p) {
  constexpr int NT = NW * 64;
  constexpr int RBY = FP8 ? kDi : 2 * kDi;        // key row bytes
  constexpr int PPR = RBY / 16;                   // 16-byte pieces per row: 8 or 16
  constexpr int NLD = kRB * RBY / 1024;           // 1 KB loads per block: 2 or 4
  constexpr int TPL = 1024 / RBY;                 // rows per load: 8 or 4
  constexpr int MB = 4 * QB;                      // 16-head M-blocks
  using Smem = RSmem<FP8, QB, NW>;
  __shared__ __attribute__((aligned(16))) Smem sm;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;

  // workgroup -> (key range kr, row group): the row groups of one key range get ids 8 apart, so
  // they run on one XCD and the later ones read the keys from its L2
  const int ng = (p.Q + QB - 1) / QB;
  const int blk = (int)blockIdx.x / (8 * ng);
  const int rem = (int)blockIdx.x - blk * 8 * ng;
  const int kr = 8 * blk + (rem & 7);
  const int q0 = (rem >> 3) * QB;
  int b, blk0, nblk;                              // sequence, first block of the range, its blocks
  if (p.balanced == 0) {
    if (kr >= p.B * p.groups) return;             // grid padding (uniform)
    b = kr / p.groups;
    blk0 = (kr - b * p.groups) * p.tiles_per_wg;
    nblk = p.tiles_per_wg;
  } else {
    // Ranges of T blocks over each sequence's own length: sequence b gets ceil(blocks_b / T)
    // ranges, numbered in sequence order, at most R = balanced + B in all.  T is the smallest of
    // a few tries upwards from total / R whose ranges fit; T = ceil(total / balanced) always
    // does.  Every workgroup derives the same partition from seq_lens (thread i: sequence i).
    const int i = threadIdx.x;
    const int Li = i < p.B ? min(p.seq_lens[i], p.max_seq_len) : 0;
    const int ti = (max(Li, 0) + kRB - 1) / kRB;
    const int total = wg_sum<NW>(ti, sm.part);
    const int R = p.balanced + p.B;
    int T = max(1, (total + R - 1) / R);
    const int T_safe = max(1, (total + p.balanced - 1) / p.balanced);
    for (int it = 0; it < 4 && T < T_safe; ++it) {
      const int cnt = wg_sum<NW>((ti + T - 1) / T, sm.part);
      if (cnt <= R) break;
      T = min(T_safe, max(T + 1, (int)(((int64_t)T * cnt + R - 1) / R)));
    }
    if (T < T_safe && wg_sum<NW>((ti + T - 1) / T, sm.part) > R) T = T_safe;
    const int gi = (ti + T - 1) / T;
    const int incl = wg_incl_scan<NW>(gi, sm.part);
    if (i < p.B && kr >= incl - gi && kr < incl) {
      sm.part[16] = i;
      sm.part[17] = incl - gi;
    }
    if (i == NT - 1) sm.part[18] = incl;          // ranges in all
    __syncthreads();
    if (kr >= sm.part[18]) return;                // (uniform)
    b = sm.part[16];
    blk0 = (kr - sm.part[17]) * T;
    nblk = T;
  }
  // With one partition per sequence (the sequence known from the block index alone) the
  // page-table entries of this wave's first D blocks are requested together with the sequence
  // length, not after it: entries are read up to the end of the table row and those at or past
  // the sequence's last scored token are never used.
  constexpr int NPE = NLD + (FP8 ? 1 : 0);
  int32_t pe_pre[D][NPE];
  if (p.balanced == 0) {
    const int32_t* prow = p.page_table + (int64_t)b * p.maxP;
#pragma unroll
    for (int u = 0; u < D; ++u)
#pragma unroll
      for (int c = 0; c < NPE; ++c) {
        const int t = (blk0 + wave + u * NW) * kRB + (c < NLD ? TPL * c + lane / PPR : n);
        const int pg = p.p_shift >= 0 ? (t >> p.p_shift) : t / p.P;
        pe_pre[u][c] = prow[min(pg, p.maxP - 1)];
      }
  }
  const int Lb = p.seq_lens[b];
  if (threadIdx.x == 0 && blk0 == 0 && q0 == 0) dbg_seq_len(p.dbg, Lb, p.Q, p.max_seq_len);
  const int L = min(Lb, p.max_seq_len);
  const int t_begin = blk0 * kRB;
  if (t_begin >= L) return;                       // uniform early exit
  const int t_end = min(L, (blk0 + nblk) * kRB);
  const int nq = min(QB, p.Q - q0);               // live rows of this group
  const int pos_last = L - p.Q + q0 + nq - 1;     // the group's largest position
  const int t_stop = min(t_end, pos_last + 1);    // tokens at or past this are never scored
  const int nb = t_stop > t_begin ? (t_stop - t_begin + kRB - 1) / kRB : 0;
  const int nbw = nb > wave ? (nb - wave + NW - 1) / NW : 0;   // this wave's blocks
  const int P = p.P;
  const int page0 = t_begin / P;
  const int npg = nb > 0 ? (t_stop - 1) / P - page0 + 1 : 0;
  const int32_t* ptab_g = p.page_table + (int64_t)b * p.maxP;
  const uint8_t* kc = (const uint8_t*)p.k_cache;

  // cache row of token t (row 0 at or past t_stop: read, never scored)
  auto slot_of = [&](int t, int c, auto&& pt_of) -> int64_t {
    int pg, of;
    if (p.p_shift >= 0) {
      pg = t >> p.p_shift;
      of = t & (P - 1);
    } else {
      pg = t / P;
      of = t - pg * P;
    }
    return t < t_stop ? (int64_t)pt_of(pg, c) * P + of : 0;
  };
  // loads of this wave's block jj: load c, lane i -> row TPL*c + i / PPR of the block, piece
  // i % PPR; fp8: the scale of token n.  Blocks past the wave's last one read row 0 (their
  // results are never stored), so every ring slot is refilled on every iteration.
  // CT (16 divides P): a block is 16 consecutive rows of one page, so one page lookup per block
  // gives a wave-uniform first row and every lane a fixed offset (load c, lane i: bytes
  // 1024c + 16i of the block).  Otherwise every lane looks up its own row.
  auto blk_tok = [&](int jj) { return t_begin + (wave + jj * NW) * kRB; };
  auto blk_row = [&](int jj, int32_t pe) -> int64_t {   // pe: page-table entry of the block's page
    const int tb = blk_tok(jj);
    if (tb >= t_stop) return 0;
    const int pg = p.p_shift >= 0 ? (tb >> p.p_shift) : tb / P;
    return (int64_t)__builtin_amdgcn_readfirstlane(pe) * P + (tb - pg * P);
  };
  auto keys_ct = [&](u32x4 (&dst)[NLD], int64_t row0) {
    const uint8_t* base = kc + row0 * RBY;
#pragma unroll
    for (int c = 0; c < NLD; ++c) dst[c] = __builtin_nontemporal_load((const u32x4*)(base + 1024 * c + 16 * lane));
  };
  auto keys_any = [&](u32x4 (&dst)[NLD], int jj, auto&& pt_of) {
    const int tb = blk_tok(jj);
#pragma unroll
    for (int c = 0; c < NLD; ++c) {
      const int64_t slot = slot_of(tb + TPL * c + lane / PPR, c, pt_of);
      dst[c] = __builtin_nontemporal_load((const u32x4*)(kc + slot * RBY + 16 * (lane % PPR)));
    }
  };

  // prologue: the page-table entries of the first D blocks, q, w and the range's page-table
  // entries are requested together; once they are in, the first D blocks' keys and scales
  int32_t pe[D][NPE];
#pragma unroll
  for (int u = 0; u < D; ++u)
#pragma unroll
    for (int c = 0; c < NPE; ++c) {
      const int t = blk_tok(u) + (c < NLD ? TPL * c + lane / PPR : n);
      int pg = p.p_shift >= 0 ? (t >> p.p_shift) : t / P;
      pe[u][c] = t < t_stop ? dbg_page(p.dbg, p.balanced == 0 ? pe_pre[u][c] : ptab_g[pg], p.num_slots, P) : 0;
    }
  constexpr int kQPer = (QB * kHi * kDi / 8 + NT - 1) / NT;
  u32x4 qv[kQPer];
  const int64_t row0 = (int64_t)b * p.Q + q0;
  {
    const u32x4* qsrc = (const u32x4*)((const __bf16*)p.q + row0 * kHi * kDi);
#pragma unroll
    for (int c = 0; c < kQPer; ++c) {
      const int e = c * NT + threadIdx.x;
      qv[c] = (e < QB * kHi * kDi / 8 && e / (kHi * kDi / 8) < nq) ? qsrc[e] : u32x4{0u, 0u, 0u, 0u};
    }
  }
  const float wv0 = threadIdx.x < QB * kHi && (int)threadIdx.x < nq * kHi ? p.w[row0 * kHi + threadIdx.x] : 0.f;
  constexpr int kPtPer = (kRegMaxPages + NT - 1) / NT;
  int32_t pv[kPtPer];
#pragma unroll
  for (int c = 0; c < kPtPer; ++c)
    pv[c] = c * NT < npg ? ptab_g[page0 + min(c * NT + (int)threadIdx.x, max(npg - 1, 0))] : 0;
  u32x4 ring[D][NLD];
  float ring_sc[D];
#pragma unroll
  for (int u = 0; u < D; ++u) {
    auto pt_pro = [&](int, int c) { return pe[u][c]; };
    if constexpr (CT) {
      const int64_t r0 = blk_row(u, pe[u][0]);
      keys_ct(ring[u], r0);
      if constexpr (FP8) ring_sc[u] = (p.k_scale + r0)[n];
    } else {
      keys_any(ring[u], u, pt_pro);
      if constexpr (FP8) ring_sc[u] = p.k_scale[slot_of(blk_tok(u) + n, NLD, pt_pro)];
    }
  }
#pragma unroll
  for (int c = 0; c < kQPer; ++c) {
    const int e = c * NT + threadIdx.x;
    if (e < QB * kHi * kDi / 8) {
      const int r = e / (kHi * kDi / 8), rest = e - r * (kHi * kDi / 8);
      const int h = rest / (kDi / 8), d8 = rest - h * (kDi / 8);
      *(u32x4*)&sm.q[r][h][8 * d8] = qv[c];
    }
  }
  if (threadIdx.x < QB * kHi) (&sm.w[0][0])[threadIdx.x] = wv0;
#pragma unroll
  for (int c = 0; c < kPtPer; ++c)
    if (c * NT + (int)threadIdx.x < npg) sm.pt[c * NT + threadIdx.x] = dbg_page(p.dbg, pv[c], p.num_slots, P);
  __syncthreads();

  // A fragments: M-block mb = (row mb/4, heads 16(mb%4) .. +16), lane: head n, dims 32g + 8s
  bf16x8 af[MB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int s = 0; s < 4; ++s) af[mb][s] = *(const bf16x8*)&sm.q[mb >> 2][16 * (mb & 3) + n][32 * g + 8 * s];
  Smem* __restrict__ rd = &sm;
  auto pt_lds = [&](int pg, int) { return rd->pt[pg - page0]; };
  // page-table entry of block jj's page from the staged table (0 past the scored tokens)
  auto blk_pe = [&](int jj) -> int32_t {
    const int tb = blk_tok(jj);
    if (tb >= t_stop) return 0;
    return rd->pt[(p.p_shift >= 0 ? (tb >> p.p_shift) : tb / P) - page0];
  };
  float* out = p.scores + row0 * p.ld;
  const int pos0 = L - p.Q + q0;                  // position of the group's first row
  uint8_t* tw = rd->tr[wave];
  // turnaround layout: row r at r * RBY, piece c at slot c ^ (r % PPR)
  int wr_off[NLD];
#pragma unroll
  for (int c = 0; c < NLD; ++c) {
    const int r = TPL * c + lane / PPR, pc = lane % PPR;
    wr_off[c] = r * RBY + 16 * (pc ^ (r % PPR));
  }

  // Per iteration jj (ring slot u = jj % D): block jj goes through the turnaround, block jj + D
  // is requested into its ring slot, block jj's MFMAs and head reduction run, then the scale of
  // block jj + D is requested into the slot block jj's scale has left.  CT: the page entry of
  // block jj + 2D is read into the slot that held block jj + D's (a D-iteration lead, so the
  // read is long done when it is used).
  int32_t pgr[D];
#pragma unroll
  for (int u = 0; u < D; ++u) pgr[u] = CT ? blk_pe(u + D) : 0;
  const int nbw_pad = (nbw + D - 1) / D * D;
  // the lane's head weights (its 16 heads of each row) stay in registers where they fit (two
  // bf16 rows need those registers for their keys and are read from LDS per block)
  constexpr bool WREG = FP8 || QB == 1;
  f32x4 wr[WREG ? QB : 1][4];
#pragma unroll
  for (int qi = 0; qi < (WREG ? QB : 1); ++qi)
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) wr[qi][hb] = *(const f32x4*)&rd->w[qi][16 * hb + 4 * g];
  for (int j0 = 0; j0 < nbw_pad; j0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int jj = j0 + u;
#pragma unroll
      for (int c = 0; c < NLD; ++c) *(u32x4*)(tw + wr_off[c]) = ring[u][c];
      int64_t row_next = 0;
      if constexpr (CT) {
        row_next = blk_row(jj + D, pgr[u]);
        keys_ct(ring[u], row_next);
        pgr[u] = blk_pe(jj + 2 * D);
      } else {
        keys_any(ring[u], jj + D, pt_lds);
      }
      // B fragments of token n: dims 32g + 8s .. +8 = bytes [32g, 32g + 32) (fp8: two pieces)
      // or [64g, 64g + 64) (bf16: four pieces) of its row
      bf16x8 kb[4];
      if constexpr (FP8) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 raw = *(const u32x4*)(tw + n * RBY + 16 * ((2 * g + h) ^ (n % PPR)));
          kb[2 * h] = fp8x8_to_bf16x8(raw[0], raw[1]);
          kb[2 * h + 1] = fp8x8_to_bf16x8(raw[2], raw[3]);
        }
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) kb[s] = *(const bf16x8*)(tw + n * RBY + 16 * ((4 * g + s) ^ (n % PPR)));
      }
      f32x4 acc[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
      // a raised priority while this wave issues its MFMAs, so that the other wave of the SIMD
      // runs its vector work (head reduction, conversions) meanwhile (c5: 147 -> 143 us)
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mb][s], kb[s], acc[mb], 0, 0, 0);
      __builtin_amdgcn_s_setprio(0);
      const float ks = FP8 ? ring_sc[u] : 1.f;
      const int tb = blk_tok(jj), t = tb + n;
#pragma unroll
      for (int qi = 0; qi < QB; ++qi) {
        float s_ = 0.f;
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) {
          const f32x4 wv = WREG ? wr[WREG ? qi : 0][hb] : *(const f32x4*)&rd->w[qi][16 * hb + 4 * g];
#pragma unroll
          for (int jx = 0; jx < 4; ++jx)   // ReLU as one integer max on the bits (negatives -> +0)
            s_ = fmaf(wv[jx], __int_as_float(max(__float_as_int(acc[4 * qi + hb][jx]), 0)), s_);
        }
        s_ = lanes4_sum(s_);
        if (g == 0 && qi < nq && jj < nbw && t < t_end) (out + (int64_t)qi * p.ld + tb)[n] = t <= pos0 + qi ? s_ * ks : -INFINITY;
      }
      // the scale of block jj + D goes into the slot this block's scale has just left
      if constexpr (FP8) {
        if constexpr (CT) ring_sc[u] = (p.k_scale + row_next)[n];
        else ring_sc[u] = p.k_scale[slot_of(blk_tok(jj + D) + n, NLD, pt_lds)];
      }
    }
  }
  // tokens of the range past the group's last position: -inf (their blocks are not computed)
  for (int t = t_begin + nb * kRB + (int)threadIdx.x; t < t_end; t += NT)
#pragma unroll
    for (int qi = 0; qi < QB; ++qi)
      if (qi < nq) out[(int64_t)qi * p.ld + t] = -INFINITY;
}
}  // namespace

bool indexer_uses_mfma(int Hi, int Di, dsa_dtype_t q_dtype, dsa_dtype_t k_dtype) {
  return Hi == kHi && Di == kDi && q_dtype == DSA_BF16 && (k_dtype == DSA_BF16 || k_dtype == DSA_FP8_E4M3FN);
}

bool indexer_uses_prefill(int Hi, int Di, int Q, int P, dsa_dtype_t q_dtype, dsa_dtype_t k_dtype) {
  return indexer_uses_mfma(Hi, Di, q_dtype, k_dtype) && k_dtype == DSA_BF16 && Q >= kPfQB && P % kSub == 0;
}

hipError_t launch_indexer(const IndexerParams& p0, dsa_dtype_t q_dtype, dsa_dtype_t k_dtype, hipStream_t s) {
  IndexerParams p = p0;
  if (p.q_count == 0) {
    p.q_begin = 0;
    p.q_count = p.Q;
  }
  if (indexer_uses_prefill(p.Hi, p.Di, p.Q, p.P, q_dtype, k_dtype)) {
    // many rows per sequence: blocks of 16 rows, key ranges so that about 256 workgroups run
    // (and one range's page-table entries fit the LDS copy)
    const int64_t nqb = (p.q_count + kPfQB - 1) / kPfQB;
    const int64_t stages = ((int64_t)p.max_seq_len + kPfST - 1) / kPfST;
    int64_t ranges = (256 + nqb * p.B - 1) / (nqb * p.B);
    const int64_t max_stages = (int64_t)(kPfMaxPages - 2) * p.P / kPfST;
    if ((stages + ranges - 1) / ranges > max_stages) ranges = (stages + max_stages - 1) / max_stages;
    if (ranges > stages) ranges = stages;
    p.groups = (int32_t)ranges;
    p.tiles_per_wg = (int32_t)((stages + ranges - 1) / ranges);
    p.p_shift = (p.P & (p.P - 1)) == 0 ? __builtin_ctz((unsigned)p.P) : -1;
    hipLaunchKernelGGL(indexer_prefill_kernel, dim3((unsigned)(nqb * ranges * p.B)), dim3(kPfThreads), 0, s, p);
    return hipGetLastError();
  }
  if (p.q_begin != 0 || p.q_count != p.Q) return hipErrorInvalidValue;   // row windows: many-rows kernel only
  if (indexer_uses_mfma(p.Hi, p.Di, q_dtype, k_dtype)) {
    // Keys straight into registers: QB rows per workgroup (one row group for Q <= 4), about one
    // round of 256 workgroups (one per compute unit) per row group.
    // At most two rows per workgroup: q of four rows fills all 256 registers of the only wave a
    // SIMD could then hold, and without a second wave to cover its latencies that was slower
    // than two groups of two rows whose repeated key reads come from L2 (64 sequences x 4 fp8
    // rows at 64K: 508 against 311 us; one sequence x 3 bf16 rows at 32K: 11.0 against 9.6 us)
    const int QB = p.Q <= 2 ? p.Q : 2;
    const int NW = 8;
    const int64_t ng = (p.Q + QB - 1) / QB;
    const int64_t blocks = ((int64_t)p.max_seq_len + kRB - 1) / kRB;
    const int64_t tb_max = std::max<int64_t>(1, (int64_t)(kRegMaxPages - 2) * p.P / kRB);
    const int64_t R = std::max<int64_t>(1, 256 / ng);
    int64_t tb = (blocks * p.B + R - 1) / R;
    tb = std::min<int64_t>(std::max<int64_t>(tb, 1), tb_max);
    int64_t groups = (blocks + tb - 1) / tb;
    p.tiles_per_wg = (int32_t)tb;
    p.groups = (int32_t)groups;
    p.p_shift = (p.P & (p.P - 1)) == 0 ? __builtin_ctz((unsigned)p.P) : -1;
    p.balanced = 0;
    int64_t ranges = p.B * groups;
    // several sequences of possibly different lengths: ranges sized from the actual lengths
    if (p.B >= 2 && 2 * p.B <= R && p.B <= NW * 64 && (p.B * blocks + (R - p.B) - 1) / (R - p.B) <= tb_max) {
      p.balanced = (int32_t)(R - p.B);
      ranges = R;
    }
    const dim3 grid((unsigned)((ranges + 7) / 8 * 8 * ng));
    const bool f8 = k_dtype == DSA_FP8_E4M3FN;
    const bool ct = p.P % kRB == 0;
#define DSA_IDX_REG2(F8, QBV, NWV, DV)                                                                          \
  do {                                                                                                       \
    if (ct) hipLaunchKernelGGL((indexer_reg_kernel<F8, true, QBV, NWV, DV>), grid, dim3(NWV * 64), 0, s, p);  \
    else hipLaunchKernelGGL((indexer_reg_kernel<F8, false, QBV, NWV, DV>), grid, dim3(NWV * 64), 0, s, p);    \
  } while (0)
    // one row: the ring depth follows this wave's block count when it is small, so that the
    // loop runs no iteration on dummy blocks (c2 at 32K: one block per wave)
    const int64_t bpw = (tb + NW - 1) / NW;
    if (QB == 1) {
      if (p.balanced) { if (f8) DSA_IDX_REG2(true, 1, 8, 4); else DSA_IDX_REG2(false, 1, 8, 3); }
      else if (bpw <= 1) { if (f8) DSA_IDX_REG2(true, 1, 8, 1); else DSA_IDX_REG2(false, 1, 8, 1); }
      else if (bpw == 2) { if (f8) DSA_IDX_REG2(true, 1, 8, 2); else DSA_IDX_REG2(false, 1, 8, 2); }
      else if (f8) DSA_IDX_REG2(true, 1, 8, 4);
      else if (bpw % 4 == 0) DSA_IDX_REG2(false, 1, 8, 4);
      else DSA_IDX_REG2(false, 1, 8, 3);
    }
    else if (QB == 2) { if (f8) DSA_IDX_REG2(true, 2, 8, 3); else DSA_IDX_REG2(false, 2, 8, 2); }
#undef DSA_IDX_REG2
    return hipGetLastError();
  }
  dim3 grid((unsigned)((p.max_seq_len + 255) / 256), (unsigned)p.Q, (unsigned)p.B);
  const size_t shm = ((size_t)p.Hi * p.Di + p.Hi) * sizeof(float);
  const bool qf = q_dtype == DSA_F32;
#define DSA_IDX_LAUNCH(QT, KT) hipLaunchKernelGGL((indexer_valu_kernel<QT, KT>), grid, dim3(256), shm, s, p)
  if (qf) {
    if (k_dtype == DSA_F32) DSA_IDX_LAUNCH(float, float);
    else if (k_dtype == DSA_BF16) DSA_IDX_LAUNCH(float, __bf16);
    else DSA_IDX_LAUNCH(float, Fp8Tag);
  } else {
    if (k_dtype == DSA_F32) DSA_IDX_LAUNCH(__bf16, float);
    else if (k_dtype == DSA_BF16) DSA_IDX_LAUNCH(__bf16, __bf16);
    else DSA_IDX_LAUNCH(__bf16, Fp8Tag);
  }
#undef DSA_IDX_LAUNCH
  return hipGetLastError();
}

}  // namespace dsa
