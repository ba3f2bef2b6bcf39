// Lightning indexer on gfx950: s[b,i,t] = sum_h w[b,i,h] * ReLU(q[b,i,h,:] . k[slot(b,t),:]).
//
// The pages name this stage the "lightning-indexer GEMM" ("GLM-52 Runs on RTX 4090", section
// "how did he do it"; renning22/glm-5.2-4090 README, section "how it works").  Two kernels:
//
//  * indexer_mfma_kernel (64 heads x 128 dims, bf16 q, bf16 or fp8 keys).  The contraction
//    runs on v_mfma_f32_32x32x16_bf16 with the indexer heads as M and tokens as N, so one
//    wave's accumulator holds, for each of its 32 tokens, 32 heads per lane half: the ReLU, the
//    head weights and the head sum stay in registers plus one exchange between lane halves.
//    Keys are read straight from HBM into the B operand: lane (token n, half h) loads bytes
//    [h*128, h*128+128) of its key row, i.e. the contraction index is permuted so that each
//    lane streams one contiguous run of its row; q is permuted the same way when it is staged.
//    fp8 keys are widened to bf16 in registers (exact) and the per-token scale is applied after
//    the head sum (it is positive, so it commutes with the ReLU).
//  * indexer_valu_kernel: any head count / dim / dtype pair, one token per thread, f32 math.
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
  const int L = min(p.seq_lens[b], p.max_seq_len);   // never write past the scores row
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
  const int64_t slot = (int64_t)p.page_table[(int64_t)b * p.maxP + t / p.P] * p.P + t % p.P;
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
// matrix-core path: Hi = 64, Di = 128, QB = 1 or 2 query rows per workgroup
//
// 8 waves (two per SIMD) stream the keys of one token range through an LDS ring of NB stages.
// A stage holds ST = 32 * 8 / QB tokens; it is filled by direct-to-LDS copies (through a
// buffer resource over the key rows) in which consecutive lanes fetch consecutive 16-byte
// pieces of key rows, so each copy moves 1 KB in few cache lines, and piece p of row r is
// stored at slot p ^ swz(r) of its LDS row so that the MFMA operand reads are free of bank
// conflicts.  Every key is read from memory once per workgroup: with QB = 2 the waves 0-3 score
// row 0 and the waves 4-7 row 1 on the same 32-token sub-tiles.  One barrier per stage (waiting
// only for LDS operations): after it the stage has landed for every wave and the stage read
// before it is free to be refilled.  The loop body reads LDS only through a restrict pointer
// and writes it only through another (the copies), so the compiler's waits for its LDS reads
// never cover the copies in flight.

constexpr int kHi = 64, kDi = 128;
constexpr int kSub = 32;                  // tokens per sub-tile (the MFMA N)
constexpr int kWaves = 8;
constexpr int kThreadsI = 64 * kWaves;
constexpr int kTile = 256;                // grid granularity: tokens per tile (128 for one-row blocks)
constexpr int kMaxTpwAny = 8;             // tiles per workgroup, any page size
constexpr int kMaxTpwContig = 128;        // tiles per workgroup when 32 | P (pages of >= 32 tokens)
constexpr int kMaxWgPages = kMaxTpwAny * kTile + 1;   // page-table entries a workgroup can span
static_assert(kMaxTpwContig * kTile / 32 + 1 <= kMaxWgPages, "page-table staging covers both layouts");

template <bool FP8, int QB>
struct Geo {
  static constexpr int RB = FP8 ? kDi : 2 * kDi;       // key row bytes
  static constexpr int WPR = kWaves / QB;              // waves per query row
  // one row: the two waves of a sub-tile take 32 heads each (HS = 2) and add their head sums
  // through LDS, so a stage is 128 tokens and the ring holds four; two rows: a wave takes all
  // 64 heads of its sub-tiles
  static constexpr int HS = QB == 1 ? 2 : 1;           // waves per sub-tile (head halves)
  static constexpr int MBW = 2 / HS;                   // 32-head M-blocks per wave
  static constexpr int SPS = WPR / HS;                 // sub-tile slots per stage
  // sub-tiles per wave and stage: two for fp8 keys and two rows, so that a stage (and the
  // barrier that closes it) covers 256 tokens
  static constexpr int SPW = (FP8 && QB == 2) ? 2 : 1;
  static constexpr int ST = kSub * SPS * SPW;          // tokens per stage
  static constexpr int SB = ST * RB;                   // stage bytes
  static constexpr int ND = SB / (kThreadsI * 16);     // 16-byte loads per thread per stage
  static constexpr int NB = QB == 1 ? 4 : 3;           // ring depth (stages of 16 / 32 KB)
  static constexpr int NSW = FP8 ? ST / 64 : 0;        // waves that also load the stage's scales
  static_assert(HS == 1 || SPW == 1, "a head-split wave keeps one pending head sum per stage");
};
template <bool FP8>
__device__ __forceinline__ int swz(int r) { return FP8 ? ((r >> 1) & 7) : (r & 15); }

// Sum and inclusive prefix sum of one int per thread over the 512-thread workgroup (wave
// shuffles, then the 8 wave totals through LDS; `red` holds at least 8 ints).
__device__ __forceinline__ int wave_incl_scan_i(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o);
    v += lane >= o ? u : 0;
  }
  return v;
}
__device__ __forceinline__ int block_incl_scan(int v, int32_t* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int w = wave_incl_scan_i(v);
  if (lane == 63) red[wave] = w;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int k = 0; k < kThreadsI / 64; ++k) before += k < wave ? red[k] : 0;
  __syncthreads();
  return w + before;
}
__device__ __forceinline__ int block_sum(int v, int32_t* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int w = wave_incl_scan_i(v);
  if (lane == 63) red[wave] = w;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int k = 0; k < kThreadsI / 64; ++k) t += red[k];
  __syncthreads();
  return t;
}

// Shared memory of indexer_mfma_kernel: ring stage = keys, then (fp8) their per-token scales.
template <bool FP8, int QB>
struct ISmem {
  uint8_t ring[Geo<FP8, QB>::NB][Geo<FP8, QB>::SB + (FP8 ? Geo<FP8, QB>::ST * 4 : 0)];
  __bf16 q[QB][kHi][kDi];
  float w[QB][kHi];
  int32_t pt[kMaxWgPages];
  float xs[2][4][kSub];    // one row: head sums of heads 32..63, by stage parity and sub-tile
  int32_t part[20];        // the balanced partition: wave partial sums, then (b, first range, ranges)
};


// CONTIG (32 divides P): a sub-tile's 32 tokens are one 32-aligned run inside one page, so its
// key rows are contiguous in the cache and one page lookup per sub-tile gives every address.
template <bool FP8, bool CONTIG, int QB>
__global__ __launch_bounds__(kThreadsI) void indexer_mfma_kernel(IndexerParams p) {
  using G = Geo<FP8, QB>;
  using Smem = ISmem<FP8, QB>;
  constexpr int NB = G::NB;
  // key ranges are whole tiles of TL tokens: one stage for one-row blocks, so that a single
  // short sequence still spreads over every compute unit
  constexpr int TL = QB == 1 ? G::ST : kTile;
  static_assert(kTile % TL == 0, "tile sizes");
  static_assert(NB >= 2 && (NB - 2) * (G::ND + 1) < 64, "ring depth");
  __shared__ __attribute__((aligned(16))) Smem sm;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // One workgroup = QB query rows x one key range (p.tiles_per_wg tiles of one sequence).  Key
  // ranges are numbered over all sequences, kr = b * groups + g, and the grid is ordered so that
  // the Q/QB row groups of one key range get ids 8 apart (ids go to the 8 XCDs round-robin):
  // they run on one XCD, close together, and the groups after the first read the keys from its
  // L2.   id = 8NQ*m + 8*i + j  ->  row group i, key range kr = 8m + j
  const int nq = p.Q / QB;
  const int blk = (int)blockIdx.x / (8 * nq);
  const int rem = (int)blockIdx.x - blk * 8 * nq;
  const int kr = 8 * blk + (rem & 7);
  const int qb0 = (rem >> 3) * QB;            // first query row of the block
  int b, grp_id, tpw;                         // sequence, range within it, tiles per range
  if (p.balanced == 0) {
    if (kr >= p.B * p.groups) return;         // grid padding (uniform)
    b = kr / p.groups;
    grp_id = kr - b * p.groups;
    tpw = p.tiles_per_wg;
  } else {
    // Ranges of T tiles over each sequence's own length: T = ceil(total tiles / p.balanced),
    // sequence b gets ceil(tiles_b / T) ranges, numbered in sequence order.  Every workgroup
    // derives the same partition from seq_lens (thread i holds sequence i; B <= 128).
    const int i = threadIdx.x;
    const int Li = i < p.B ? min(p.seq_lens[i], p.max_seq_len) : 0;
    const int ti = (max(Li, 0) + TL - 1) / TL;
    const int total = block_sum(ti, sm.part);
    // the smallest T (a few tries upwards from total / R) whose ranges fit R = balanced + B;
    // T = ceil(total / balanced) always does
    const int R = p.balanced + p.B;
    int T = max(1, (total + R - 1) / R);
    const int T_safe = max(1, (total + p.balanced - 1) / p.balanced);
    for (int it = 0; it < 4 && T < T_safe; ++it) {
      const int cnt = block_sum((ti + T - 1) / T, sm.part);
      if (cnt <= R) break;
      T = min(T_safe, max(T + 1, (int)(((int64_t)T * cnt + R - 1) / R)));
    }
    if (T < T_safe && block_sum((ti + T - 1) / T, sm.part) > R) T = T_safe;
    const int gi = (ti + T - 1) / T;
    const int incl = block_incl_scan(gi, sm.part);
    if (i < p.B && kr >= incl - gi && kr < incl) {
      sm.part[16] = i;
      sm.part[17] = incl - gi;
    }
    if (i == kThreadsI - 1) sm.part[18] = incl;   // ranges in all
    __syncthreads();
    if (kr >= sm.part[18]) return;            // (uniform)
    b = sm.part[16];
    grp_id = kr - sm.part[17];
    tpw = T;
  }
  const int tile_base = grp_id * tpw * TL;
  const int32_t* ptab_g = p.page_table + (int64_t)b * p.maxP;

  // Stage v covers tokens tile_base + v*ST ..; this thread's load c fills LDS bytes
  // [off, off+16) of the stage, off = ((c*8 + wave)*64 + lane)*16: row r = off / RB and slot
  // off % RB / 16, fetched from piece (slot ^ swz(r)) of that token's key row.
  int lane_row[G::ND];     // stage row of this lane's piece in copy c
  int lane_boff[G::ND];    // byte offset of that piece inside its key row
#pragma unroll
  for (int c = 0; c < G::ND; ++c) {
    const int off = ((c * kWaves + wave) * 64 + lane) * 16;
    const int r = off / G::RB, q = (off % G::RB) / 16;
    lane_row[c] = r;
    lane_boff[c] = 16 * (q ^ swz<FP8>(r));
  }
  const bool scale_wave = FP8 && wave < G::NSW;
  // token whose cache row copy c (c = ND: the scale copy) of stage v starts at
  auto tok = [&](int v, int c) {
    const int t0 = tile_base + v * G::ST;
    if (c == G::ND) return t0 + wave * 64 + lane;
    return CONTIG ? t0 + (lane_row[c] & ~(kSub - 1)) : t0 + lane_row[c];
  };
  constexpr int NL = G::ND + (FP8 ? 1 : 0);
  // the page-table entries of the first NB-1 stages are requested before the sequence length
  // arrives (bounded by max_seq_len alone), so the first copies wait one round trip less
  int32_t pre_pe[NB - 1][NL];
  {
    const int t_cap = min(tile_base + tpw * TL, p.max_seq_len);
#pragma unroll
    for (int v = 0; v < NB - 1; ++v)
#pragma unroll
      for (int c = 0; c < NL; ++c) {
        const int t = tok(v, c);
        pre_pe[v][c] = t < t_cap && (c < G::ND || scale_wave) ? ptab_g[t / p.P] : 0;
      }
  }
  const int L = min(p.seq_lens[b], p.max_seq_len);
  if (tile_base >= L) return;                 // uniform early exit
  const int tile_end = min(L, tile_base + tpw * TL);
  const int pos_last = L - p.Q + qb0 + QB - 1;  // the block's largest position
  const int t_stop = min(tile_end, pos_last + 1);  // tokens at or past this are never scored
  const int nstage = t_stop > tile_base ? (t_stop - tile_base + G::ST - 1) / G::ST : 0;

  const int ri = wave / G::WPR;               // the row this wave scores
  const int wl = wave - ri * G::WPR;
  const int si = wl % G::SPS;                 // its first sub-tile within a stage is si * SPW
  const int mh = wl / G::SPS;                 // its head half (one row), else 0
  const int pos = L - p.Q + qb0 + ri;         // that row sees tokens t <= pos
  const int n_in_sub = lane & 31;
  const int half = lane >> 5;
  const int page0 = tile_base / p.P;
  const int npg = (t_stop > tile_base) ? (t_stop - 1) / p.P - page0 + 1 : 0;
  const __amdgpu_buffer_rsrc_t k_rs = rows_rsrc(p.k_cache, G::RB, p.num_slots);
  const __amdgpu_buffer_rsrc_t s_rs = rows_rsrc(FP8 ? (const void*)p.k_scale : p.k_cache, 4, FP8 ? p.num_slots : 0);

  // Cache rows of this lane's copies of one stage: copy c fetches row slot[c] (CONTIG: the first
  // row of the copy's 32-token run, which the lane offsets by r % 32), the scale copy row sslot.
  struct Rows {
    int32_t slot[G::ND];
    int32_t sslot;
  };
  // copies of one stage into ring stage `dst` (keys, then the scales behind them)
  auto issue = [&](uint8_t* __restrict__ dst, const Rows& rw) {
#pragma unroll
    for (int c = 0; c < G::ND; ++c) {
      const int off = ((c * kWaves + wave) * 64) * 16;     // this copy's 1-KB block of the stage
      const int row = CONTIG ? (int)rw.slot[c] + (lane_row[c] & (kSub - 1)) : (int)rw.slot[c];
      lds_dma16_row(k_rs, row, lane_boff[c], dst + off);
    }
    if constexpr (FP8) {
      if (scale_wave) lds_dma4_row(s_rs, (int)rw.sslot, dst + G::SB + wave * 256);
    }
  };
  // the first NB-1 stages are requested before q is staged, from the prefetched page-table
  // entries
#pragma unroll
  for (int v = 0; v < NB - 1; ++v)
    if (v < nstage) {
      Rows rw;
#pragma unroll
      for (int c = 0; c < G::ND; ++c) {
        const int t = tok(v, c);
        rw.slot[c] = t < t_stop ? pre_pe[v][c] * p.P + t % p.P : 0;
      }
      rw.sslot = 0;
      if constexpr (FP8) {
        const int t = tok(v, G::ND);
        rw.sslot = scale_wave && t < t_stop ? pre_pe[v][G::ND] * p.P + t % p.P : 0;
      }
      issue(sm.ring[v], rw);
    }

  // stage q (bf16), w and the page-table entries of this workgroup's tokens
  {
    const int64_t row0 = (int64_t)b * p.Q + qb0;
    const u32x4* qsrc = (const u32x4*)((const __bf16*)p.q + row0 * kHi * kDi);
    u32x4* qdst = (u32x4*)&sm.q[0][0][0];
    constexpr int kPer = QB * kHi * kDi / 8 / kThreadsI;
    u32x4 qv[kPer];
#pragma unroll
    for (int c = 0; c < kPer; ++c) qv[c] = qsrc[c * kThreadsI + threadIdx.x];
    const float wv = threadIdx.x < QB * kHi ? p.w[row0 * kHi + threadIdx.x] : 0.f;
    constexpr int kPtPer = (kMaxWgPages + kThreadsI - 1) / kThreadsI;
    int32_t pv[kPtPer];
#pragma unroll
    for (int c = 0; c < kPtPer; ++c)   // (uniform: only the blocks of entries the workgroup spans)
      pv[c] = c * kThreadsI < npg ? ptab_g[page0 + min(c * kThreadsI + (int)threadIdx.x, npg - 1)] : 0;
#pragma unroll
    for (int c = 0; c < kPer; ++c) qdst[c * kThreadsI + threadIdx.x] = qv[c];
    if (threadIdx.x < QB * kHi) (&sm.w[0][0])[threadIdx.x] = wv;
#pragma unroll
    for (int c = 0; c < kPtPer; ++c)
      if (c * kThreadsI + (int)threadIdx.x < npg) sm.pt[c * kThreadsI + threadIdx.x] = pv[c];
  }
  __syncthreads();

  // A fragments of this wave's row: lane (head m = lane%32 of M-block mb, half h) holds, for
  // k-step s, q dims [h*64 + s*8, +8) (the contraction index is permuted the same way for keys)
  // (this wave's M-blocks: mh*MBW .. +MBW)
  bf16x8 afrag[G::MBW][8];
#pragma unroll
  for (int mb = 0; mb < G::MBW; ++mb)
#pragma unroll
    for (int s = 0; s < 8; ++s)
      afrag[mb][s] = *(const bf16x8*)&sm.q[ri][(mh * G::MBW + mb) * 32 + n_in_sub][half * 64 + s * 8];
  // head weights of the heads this lane holds: m = (mh*MBW + mb)*32 + g*8 + half*4 + j
  float wr[G::MBW][4][4];
#pragma unroll
  for (int mb = 0; mb < G::MBW; ++mb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 wv = *(const f32x4*)&sm.w[ri][(mh * G::MBW + mb) * 32 + g * 8 + half * 4];
#pragma unroll
      for (int j = 0; j < 4; ++j) wr[mb][g][j] = wv[j];
    }

  const int P = p.P;
  float* out = p.scores + ((int64_t)b * p.Q + qb0 + ri) * p.ld;
  // Rows of the next stage to request are looked up one stage ahead, so the page-table reads
  // from LDS are long done when the copies are issued.  Copy c (c < ND: keys, c = ND: scales)
  // of stage v starts at token tok(v, c); (lk_pg, lk_of) = its page and offset in that page for
  // the stage to look up next, stepped by ST tokens per stage (no division in the loop).
  int lk_pg[NL], lk_of[NL];
#pragma unroll
  for (int c = 0; c < NL; ++c) {
    const int t = tok(NB - 1, c);
    lk_pg[c] = t / P;
    lk_of[c] = t - lk_pg[c] * P;
  }
  const int st_pg = G::ST / P, st_of = G::ST - st_pg * P;
  auto lookup = [&](const Smem* __restrict__ rd, int v) {
    Rows rw;
    rw.sslot = 0;
#pragma unroll
    for (int c = 0; c < NL; ++c) {
      // (tokens at or past t_stop read an entry inside the staged table, or zeros past it,
      // and take row 0)
      const int32_t sl = rd->pt[lk_pg[c] - page0] * P + lk_of[c];
      const int32_t val = tok(v, c) < t_stop ? sl : 0;
      // (CONTIG: the copy's run start is the same for the whole wave)
      if (c < G::ND) rw.slot[c] = CONTIG ? __builtin_amdgcn_readfirstlane(val) : val;
      else rw.sslot = scale_wave ? val : 0;
      lk_pg[c] += st_pg;
      lk_of[c] += st_of;
      if (lk_of[c] >= P) {
        lk_of[c] -= P;
        ++lk_pg[c];
      }
    }
    return rw;
  };
  Rows next = lookup(&sm, NB - 1);

  // The head reduction of a sub-tile runs one stage late: the MFMAs of stage v are issued next
  // to the ReLU / weight / head-sum work of stage v-1, so the matrix core and the vector ALU
  // overlap.  (acc_prev, t_prev, ks_prev) = stage v-1's accumulators, lane token and scale.
  f32x16 acc_prev[G::MBW];
#pragma unroll
  for (int mb = 0; mb < G::MBW; ++mb) acc_prev[mb] = f32x16{};
  int t_prev = -1, par_prev = 0;
  float ks_prev = 0.f;
  // one row (HS = 2): the head half 0 waves keep the head sum of heads 0..31 of stage u (pend_*)
  // until, after the next barrier, the half 1 waves' sum of heads 32..63 is in xs[u & 1]
  float pend_part = 0.f, pend_ks = 0.f;
  int pend_t = -1, pend_par = 0;
  auto store = [&](int t, float part, float ks) {
    if (half == 0 && t >= 0 && t < tile_end) out[t] = t <= pos ? part * ks : -INFINITY;
  };
  auto complete = [&](const Smem* __restrict__ rd) {   // (HS = 2, head half 0)
    if (pend_t >= 0) store(pend_t, pend_part + rd->xs[pend_par][si][n_in_sub], pend_ks);
    pend_t = -1;
  };
  auto finish = [&](Smem* __restrict__ rd, const f32x16 (&acc)[G::MBW], int t, float ks, int par) {
    float part = 0.f;
#pragma unroll
    for (int mb = 0; mb < G::MBW; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)   // ReLU as one integer max on the bits (negatives -> +0)
          part = fmaf(wr[mb][g][jj], __int_as_float(max(__float_as_int(acc[mb][4 * g + jj]), 0)), part);
    // add the other lane half's partial sum (lanes l and l ^ 32 hold the same token)
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
    part = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    if constexpr (G::HS == 1) {
      store(t, part, ks);
    } else if (t >= 0) {
      if (mh == 1) {
        if (half == 0) rd->xs[par][si][n_in_sub] = part;
      } else {
        pend_part = part;
        pend_ks = ks;
        pend_t = t;
        pend_par = par;
      }
    }
  };

  // one stage: request stage v + NB - 1 into ring stage `dst` and look up the rows of stage
  // v + NB; per sub-tile of this wave in stage v: B fragments (lane: token n, half h) from LDS,
  // 32x32x16 MFMAs over the two 32-head M-blocks, then the head reduction of the sub-tile
  // before it
  auto compute = [&](Smem* __restrict__ rd, int v) {
    if constexpr (G::HS == 2) {
      if (mh == 0) complete(rd);   // stage v-2's sum: its other half was written before the barrier
    }
#pragma unroll
    for (int j = 0; j < G::SPW; ++j) {
      const int sub = si * G::SPW + j;
      const int t = tile_base + v * G::ST + sub * kSub + n_in_sub;
      const uint8_t* rows = &rd->ring[v % NB][sub * kSub * G::RB];
      bf16x8 kf[8];
      if constexpr (FP8) {
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {          // dims h*64 + 16*s2 .. +16 = piece 4h + s2
          const u32x4 raw = *(const u32x4*)(rows + n_in_sub * G::RB + 16 * ((4 * half + s2) ^ swz<FP8>(n_in_sub)));
          __bf16 tmp[16];
#pragma unroll
          for (int d = 0; d < 4; ++d) fp8x4_to_bf16x4(raw[d], tmp + 4 * d);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            kf[2 * s2][e] = tmp[e];
            kf[2 * s2 + 1][e] = tmp[8 + e];
          }
        }
      } else {
#pragma unroll
        for (int s = 0; s < 8; ++s)               // dims h*64 + 8s .. +8 = piece 8h + s
          kf[s] = *(const bf16x8*)(rows + n_in_sub * G::RB + 16 * ((8 * half + s) ^ swz<FP8>(n_in_sub)));
      }
      const float ks = FP8 ? ((const float*)(&rd->ring[v % NB][G::SB]))[sub * kSub + n_in_sub] : 1.f;
      // (sub-tiles wholly past the row's position are computed too, on valid rows, and written
      // as -inf by the reduction)
      f32x16 acc[G::MBW];
#pragma unroll
      for (int mb = 0; mb < G::MBW; ++mb) acc[mb] = f32x16{};
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int mb = 0; mb < G::MBW; ++mb)
          acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag[mb][s], kf[s], acc[mb], 0, 0, 0);
      finish(rd, acc_prev, t_prev, ks_prev, par_prev);
#pragma unroll
      for (int mb = 0; mb < G::MBW; ++mb) acc_prev[mb] = acc[mb];
      t_prev = t;
      ks_prev = ks;
      par_prev = v & 1;
    }
  };

  for (int v = 0; v < nstage; ++v) {
    // stage v must have landed: at most the loads of the later stages requested so far
    // (v+1 .. v+NB-2) may still be outstanding (vector-memory loads complete in order)
    const int later = min(NB - 2, nstage - 1 - v);
    if (scale_wave) wait_vmcnt_later<G::ND + 1, NB - 2>(later);
    else wait_vmcnt_later<G::ND, NB - 2>(later);
    lds_barrier();   // stage v landed for every wave; stage v-1 is no longer read
    if (v + NB - 1 < nstage) {
      issue(sm.ring[(v + NB - 1) % NB], next);
      if (v + NB < nstage) next = lookup(&sm, v + NB);
    }
    compute(&sm, v);
  }
  if constexpr (G::HS == 2) {
    // stage nstage-2's other half was written in the last iteration; stage nstage-1's now
    lds_barrier();
    if (mh == 0) complete(&sm);
    finish(&sm, acc_prev, t_prev, ks_prev, par_prev);
    lds_barrier();
    if (mh == 0) complete(&sm);
  } else {
    finish(&sm, acc_prev, t_prev, ks_prev, par_prev);
  }
  // tokens of [tile_base, tile_end) past the block's last position: -inf (their stages are not
  // computed)
  for (int t = max(t_stop, tile_base) + (int)threadIdx.x; t < tile_end; t += kThreadsI)
#pragma unroll
    for (int qq = 0; qq < QB; ++qq) p.scores[((int64_t)b * p.Q + qb0 + qq) * p.ld + t] = -INFINITY;
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
  // id = (b * ranges + range) * query blocks + query block
  const int nqb = (p.Q + kPfQB - 1) / kPfQB;
  const int qb = (int)blockIdx.x % nqb;
  const int rest = (int)blockIdx.x / nqb;
  const int kr = rest % p.groups, b = rest / p.groups;
  const int L = min(p.seq_lens[b], p.max_seq_len);
  const int q0 = qb * kPfQB;
  const int nq = min(kPfQB, p.Q - q0);             // rows of this block
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
  auto pt_global = [&](int pg) { return ptab_g[pg]; };
#pragma unroll
  for (int v = 0; v < kPfNB - kPfSPB; ++v)
    if (v < nstage) issue(sm.ring[v], pt_global);

  // q of this wave's rows (clamped into the chunk; rows past it are computed, never stored):
  // lane (head m of M-block mb, half h) holds dims h*64 + s*8 .. +8 for step s
  bf16x8 afrag[kPfQW][2][8];
#pragma unroll
  for (int qi = 0; qi < kPfQW; ++qi) {
    const int row = min(q0 + wave * kPfQW + qi, p.Q - 1);
    const __bf16* qrow = (const __bf16*)p.q + ((int64_t)b * p.Q + row) * kHi * kDi;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int s = 0; s < 8; ++s)
        afrag[qi][mb][s] = *(const bf16x8*)(qrow + (mb * 32 + n_in_sub) * kDi + half * 64 + s * 8);
  }
  for (int e = threadIdx.x; e < kPfQB * kHi; e += kPfThreads) {
    const int row = min(q0 + e / kHi, p.Q - 1);
    (&sm.w[0][0])[e] = p.w[((int64_t)b * p.Q + row) * kHi + e % kHi];
  }
  for (int e = threadIdx.x; e < npg; e += kPfThreads) sm.pt[e] = ptab_g[page0 + e];
  __syncthreads();

  float* out_b = p.scores + ((int64_t)b * p.Q + q0) * p.ld;
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
#pragma unroll
        for (int s = 0; s < 8; ++s)
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
            acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag[qi][mb][s], kf[s], acc[mb], 0, 0, 0);
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

}  // namespace

bool indexer_uses_mfma(int Hi, int Di, dsa_dtype_t q_dtype, dsa_dtype_t k_dtype) {
  return Hi == kHi && Di == kDi && q_dtype == DSA_BF16 && (k_dtype == DSA_BF16 || k_dtype == DSA_FP8_E4M3FN);
}

hipError_t launch_indexer(const IndexerParams& p0, dsa_dtype_t q_dtype, dsa_dtype_t k_dtype, hipStream_t s) {
  IndexerParams p = p0;
  if (indexer_uses_mfma(p.Hi, p.Di, q_dtype, k_dtype) && k_dtype == DSA_BF16 && p.Q >= kPfQB && p.P % kSub == 0) {
    // many rows per sequence: blocks of 16 rows, key ranges so that about 256 workgroups run
    // (and one range's page-table entries fit the LDS copy)
    const int64_t nqb = (p.Q + kPfQB - 1) / kPfQB;
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
  if (indexer_uses_mfma(p.Hi, p.Di, q_dtype, k_dtype)) {
    // about one round of the 256 workgroups the GPU holds at once (one per CU): a workgroup's
    // q / page-table staging and first copies take several microseconds, paid once per CU
    const bool contig = p.P % kSub == 0;
    const int QB = (p.Q % 2 == 0) ? 2 : 1;
    // tile size of the kernel's key ranges (one stage for one-row blocks)
    static_assert(Geo<false, 1>::ST == 128 && Geo<true, 1>::ST == 128, "one-row stage");
    const int TL = QB == 1 ? 128 : kTile;
    const int64_t tiles = ((int64_t)p.max_seq_len + TL - 1) / TL;
    const int64_t work = tiles * p.B * (p.Q / QB);
    // (the same token spans as kMaxTpw* tiles of kTile tokens: the page-table staging bound)
    const int max_tpw = (contig ? kMaxTpwContig : kMaxTpwAny) * (kTile / TL);
    int tpw = (int)(work / 256);
    tpw = tpw < 1 ? 1 : (tpw > max_tpw ? max_tpw : tpw);
    p.tiles_per_wg = tpw;
    p.p_shift = (p.P & (p.P - 1)) == 0 ? __builtin_ctz((unsigned)p.P) : -1;
    const int64_t groups = (tiles + tpw - 1) / tpw;
    p.groups = (int32_t)groups;
    int64_t ranges = (groups * p.B + 7) / 8 * 8;
    // Several sequences of possibly different lengths: ranges sized from the actual lengths so
    // that all of them run in one round of one workgroup per compute unit.  With
    // T = ceil(total / (R - B)) tiles per range there are at most total/T + B <= R ranges,
    // R = 256 / (row groups); used when B <= R/2 and the largest T the partition can produce,
    // ceil(B * tiles / (R - B)), still fits the page-table staging.
    const int64_t R = 256 / (p.Q / QB);
    p.balanced = 0;
    if (p.B >= 2 && 2 * p.B <= R && (p.B * tiles + (R - p.B) - 1) / (R - p.B) <= max_tpw) {
      p.balanced = (int32_t)(R - p.B);
      ranges = (R + 7) / 8 * 8;
    }
    const dim3 grid((unsigned)(ranges * (p.Q / QB)));
    const bool f8 = k_dtype == DSA_FP8_E4M3FN;
#define DSA_IDX_MFMA(F8, CT, QBV) hipLaunchKernelGGL((indexer_mfma_kernel<F8, CT, QBV>), grid, dim3(kThreadsI), 0, s, p)
    if (QB == 2) {
      if (contig) { if (f8) DSA_IDX_MFMA(true, true, 2); else DSA_IDX_MFMA(false, true, 2); }
      else { if (f8) DSA_IDX_MFMA(true, false, 2); else DSA_IDX_MFMA(false, false, 2); }
    } else {
      if (contig) { if (f8) DSA_IDX_MFMA(true, true, 1); else DSA_IDX_MFMA(false, true, 1); }
      else { if (f8) DSA_IDX_MFMA(true, false, 1); else DSA_IDX_MFMA(false, false, 1); }
    }
#undef DSA_IDX_MFMA
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
