// Sparse MLA decode on gfx950 (the "MLA sparse decode" kernel group of "GLM-52 Runs on RTX
// 4090", section "how did he do it"), over 576-wide compressed latent rows with V = the first
// 512 values, weight-absorbed and without GQA (Show HN "Chay GLM 5.2 tren may tinh cham",
// main-features section).
//
// Kernels (bf16 q; the launcher picks one by row type, row count and chunk length):
//   mla_bf16n_kernel  bf16 rows, at most 16 (query row, 16-head group) pairs, chunks <= 512:
//                     one workgroup per (row, head group, chunk), 128-token tiles staged through
//                     registers, the same fixed-reference softmax.
//   mla_bf16d_kernel  bf16 rows, chunks <= 2048: 8 waves, 32-token tiles copied HBM -> LDS into
//                     a 4-deep ring, S^T per (head group, 16-token block), P.V per 64 output
//                     values over all heads, softmax against a fixed per-head reference.
//   mla_fp8d_kernel   fp8 rows, chunks <= 2048: 8 waves, 32-token e4m3 tiles staged HBM ->
//                     registers -> LDS with coalesced loads, rows widened exactly to bf16 at
//                     each operand read, the same fixed-reference softmax.
//   mla_fp8_kernel    fp8 rows, longer chunks: 8 waves, online softmax with lazy rescaling.
//   mla_mfma_kernel   bf16 rows, longer chunks: 8 waves, rows staged through registers.
// Common to all: S^T = rows . q^T and O^T += V^T . P^T on the bf16 (or e4m3) MFMAs in fp32,
// exp2 with log2 e folded into the scale, V^T operands read with the transposing LDS reads,
// the fp8 per-token scale folded into the logits and into P.  With n_split > 1 each chunk
// writes (m, l, o/l) partials and mla_combine_kernel merges them in a fixed order.
// mla_valu_kernel is the f32 path (any head count), one workgroup per (row, head).
//
// mla_mfma_kernel in detail: one workgroup = 8 waves = one query row x one chunk of its selected
// slots (split-k).  A pair of waves owns 16 heads, one wave per half of the K dims (S^T) and of
// the output dims (P.V).  Per 32-token tile:
//   * the tile's rows are gathered from HBM (16-byte loads, one row = 72 of them; fp8 rows are
//     widened to bf16 in registers) into LDS, double-buffered, with the next two tiles' loads
//     in flight while this one is computed;
//   * S^T on v_mfma_f32_16x16x32_bf16 (M = 16 tokens, N = 16 heads, K = 576 in 18 steps, q held
//     in registers).  The two 16-token blocks are chosen so that each lane ends up with 8
//     consecutive tokens of one head, exactly the K slice the P.V product needs;
//   * online softmax with lazy rescaling: the running maximum moves only when a tile exceeds it
//     by more than 2^8, so the 512-value accumulator is rarely touched;
//   * O^T += V^T . P^T with M = 16 latent dims, N = 16 heads, K = 32 tokens, P from registers.
#include "dsa_internal.hpp"

namespace dsa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRefMargin = 64.f;   // log2 of the largest P relative to the softmax reference R

constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------------------------
// vector path (f32 q)

template <typename KT> struct RowElt;
template <> struct RowElt<float> {
  static __device__ __forceinline__ float get(const void* p, int64_t i) { return ((const float*)p)[i]; }
};
template <> struct RowElt<__bf16> {
  static __device__ __forceinline__ float get(const void* p, int64_t i) {
    return bf16_bits_to_f32(((const uint16_t*)p)[i]);
  }
};
struct Fp8Row {};
template <> struct RowElt<Fp8Row> {
  static __device__ __forceinline__ float get(const void* p, int64_t i) {
    return fp8_to_f32(((const uint8_t*)p)[i]);
  }
};

__device__ __forceinline__ float block_reduce_256(float v, float* red, bool is_max) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float o = __shfl_xor(v, off);
    v = is_max ? fmaxf(v, o) : v + o;
  }
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
  __syncthreads();
  return r;
}

template <typename KT>
__global__ __launch_bounds__(256) void mla_valu_kernel(MlaParams p) {
  extern __shared__ float sm[];     // q [576] | e [k]
  __shared__ float red[4];
  const int r = blockIdx.x, h = blockIdx.y;
  const float* q = (const float*)p.q + ((int64_t)r * p.H + h) * kRowDim;
  float* e = sm + kRowDim;
  for (int d = threadIdx.x; d < kRowDim; d += 256) sm[d] = q[d];
  __syncthreads();
  const int32_t* sl = p.slots + (int64_t)r * p.k;
  float m = -INFINITY;
  for (int j = threadIdx.x; j < p.k; j += 256) {
    const int64_t s = dbg_slot(p.dbg, sl[j], p.num_slots);
    float z = -INFINITY;
    if (s >= 0) {
      float dot = 0.f;
      for (int d = 0; d < kRowDim; ++d) dot = fmaf(sm[d], RowElt<KT>::get(p.kv, s * kRowDim + d), dot);
      if (p.kv_scale) dot *= p.kv_scale[s];
      z = dot * p.sm_scale;
    }
    e[j] = z;
    m = fmaxf(m, z);
  }
  m = block_reduce_256(m, red, true);
  float* out = p.out + ((int64_t)r * p.H + h) * kVDim;
  if (m == -INFINITY) {
    for (int d = threadIdx.x; d < kVDim; d += 256) out[d] = 0.f;
    if (p.lse && threadIdx.x == 0) p.lse[(int64_t)r * p.H + h] = -INFINITY;
    return;
  }
  float l = 0.f;
  for (int j = threadIdx.x; j < p.k; j += 256) {
    const float z = e[j];
    const float x = z == -INFINITY ? 0.f : expf(z - m);
    e[j] = x;
    l += x;
  }
  l = block_reduce_256(l, red, false);   // (the reduction's barrier also publishes e[])
  for (int d = threadIdx.x; d < kVDim; d += 256) {
    float acc = 0.f;
    for (int j = 0; j < p.k; ++j) {
      const int64_t s = dbg_slot(p.dbg, sl[j], p.num_slots, false);
      if (s < 0) continue;
      float v = RowElt<KT>::get(p.kv, s * kRowDim + d);
      if (p.kv_scale) v *= p.kv_scale[s];
      acc = fmaf(e[j], v, acc);
    }
    out[d] = acc / l;
  }
  if (p.lse && threadIdx.x == 0) p.lse[(int64_t)r * p.H + h] = m + logf(l);
}

// ---------------------------------------------------------------------------------------------
// matrix-core path (bf16 q, bf16 or fp8 rows, H = 16 * head groups <= 64)
//
// 512 threads = 8 waves, two per SIMD.  Wave w works on head group hg = w % 4 (heads
// 16hg..16hg+15) and half kh = w / 4: for S^T it covers the K dims [288kh, 288kh+288), for
// P.V the output dims [256kh, 256kh+256).  The two waves of a head group add their S^T halves
// through LDS in a fixed order (half 0 + half 1), so both hold identical logits and run the
// same online softmax.

constexpr int kTT = 32;                          // tokens per tile
constexpr int kPitch = kRowDim * 2 + 16;          // LDS bytes per bf16 row (+16 against bank conflicts)
constexpr int kNT = 512;                          // threads per workgroup
constexpr int kChunksBf16 = kTT * (kRowDim * 2 / 16);   // 2304 16-byte pieces per tile
constexpr int kChunksFp8 = kTT * (kRowDim / 16);        // 1152
constexpr int kKSteps = kRowDim / 32 / 2;               // 9 K steps of 32 per half
constexpr int kDBlocks = kVDim / 16 / 2;                // 16 output blocks of 16 per half

template <bool FP8>
struct TileStage {
  static constexpr int kPer = ((FP8 ? kChunksFp8 : kChunksBf16) + kNT - 1) / kNT;   // 3 or 5
  u32x4 v[kPer];
};

// Gather one tile's rows into registers.  `sl_lds` is the workgroup's chunk of the slot list
// staged in LDS (entry -1 for a skipped slot or a position past the chunk).  Every load is
// issued unconditionally (a skipped slot, or a piece past the tile, reads row 0) and nothing
// here reads the results, so the loads stay in flight until the tile is stored, which is also
// where skipped rows are zeroed.
template <bool FP8>
__device__ __forceinline__ void tile_load(TileStage<FP8>& st, const MlaParams& p, const int32_t* sl_lds,
                                          int tile_off) {
  constexpr int kPiecesPerRow = FP8 ? kRowDim / 16 : kRowDim * 2 / 16;   // 36 or 72
  constexpr int kPieces = kTT * kPiecesPerRow;
  const uint8_t* kv = (const uint8_t*)p.kv;
  int64_t s[TileStage<FP8>::kPer];
#pragma unroll
  for (int c = 0; c < TileStage<FP8>::kPer; ++c) {
    const int g = min(c * kNT + (int)threadIdx.x, kPieces - 1);
    s[c] = sl_lds[tile_off + g / kPiecesPerRow];
  }
#pragma unroll
  for (int c = 0; c < TileStage<FP8>::kPer; ++c) {
    const int g = min(c * kNT + (int)threadIdx.x, kPieces - 1);
    const int piece = g % kPiecesPerRow;
    const int64_t row = s[c] < 0 ? 0 : s[c];
    st.v[c] = __builtin_nontemporal_load((const u32x4*)(kv + row * (FP8 ? kRowDim : 2 * kRowDim)) + piece);
  }
}

template <bool FP8>
__device__ __forceinline__ void tile_store(const TileStage<FP8>& st, uint8_t* lds, const int32_t* sl_lds,
                                           int tile_off) {
  constexpr int kPiecesPerRow = FP8 ? kRowDim / 16 : kRowDim * 2 / 16;
#pragma unroll
  for (int c = 0; c < TileStage<FP8>::kPer; ++c) {
    const int g = c * kNT + threadIdx.x;
    if (g >= kTT * kPiecesPerRow) continue;
    const int tk = g / kPiecesPerRow, piece = g - tk * kPiecesPerRow;
    const bool skip = sl_lds[tile_off + tk] < 0;
    const u32x4 v = skip ? u32x4{0, 0, 0, 0} : st.v[c];
    if constexpr (FP8) {
      __bf16 tmp[16];
#pragma unroll
      for (int d = 0; d < 4; ++d) fp8x4_to_bf16x4(v[d], tmp + 4 * d);
      bf16x8 lo, hi;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        lo[e] = tmp[e];
        hi[e] = tmp[8 + e];
      }
      bf16x8* dst = (bf16x8*)(lds + tk * kPitch + piece * 32);
      dst[0] = lo;
      dst[1] = hi;
    } else {
      *(u32x4*)(lds + tk * kPitch + piece * 16) = v;
    }
  }
}

template <bool FP8>
__global__ __launch_bounds__(kNT) void mla_mfma_kernel(MlaParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[2][kTT * kPitch];
  __shared__ __attribute__((aligned(16))) f32x4 xs[8][2][64];   // each wave's S^T half, per lane
  __shared__ float tok_scale[2][kTT];             // per-token scale (fp8) or 1; 0 marks a skipped slot
  __shared__ int32_t sl_lds[kMaxTopK + kTT];      // this chunk's slots, -1 padded to whole tiles

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hg = wave & 3, kh = wave >> 2;
  const int r = blockIdx.y, split = blockIdx.x;
  const int j0 = split * p.chunk;
  const int j1 = min(p.k, j0 + p.chunk);
  const int ntiles = j1 > j0 ? (j1 - j0 + kTT - 1) / kTT : 0;
  const int32_t* sl = p.slots + (int64_t)r * p.k;
  const bool active = hg * 16 < p.H;              // head groups past the head count only help load
  const int head = hg * 16 + (lane & 15);
  const int grp = lane >> 4;                      // 16-lane group

  // q fragments (B operand of S^T): head lane%16, dims (9kh + s)*32 + grp*8 .. +8
  bf16x8 qf[kKSteps];
  if (active) {
    const bf16x8* qrow = (const bf16x8*)((const __bf16*)p.q + ((int64_t)r * p.H + head) * kRowDim);
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) qf[s] = qrow[(kKSteps * kh + s) * 4 + grp];
  }

  f32x4 o[kDBlocks];
#pragma unroll
  for (int db = 0; db < kDBlocks; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;   // running max of z * log2(e), per head
  float l_run = 0.f;         // this lane group's share of sum exp2(z - m_run)
  const float scale2 = p.sm_scale * kLog2e;

  // stage the chunk's slot list (one coalesced pass, every load issued before any is used)
  {
    const int span = ntiles * kTT;
    for (int e0 = 0; e0 < span; e0 += 4 * kNT) {
      int32_t v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = sl[min(j0 + e0 + u * kNT + (int)threadIdx.x, p.k - 1)];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + u * kNT + threadIdx.x;
        if (e < span) sl_lds[e] = j0 + e < j1 ? dbg_slot(p.dbg, v[u], p.num_slots) : -1;
      }
    }
  }
  __syncthreads();

  // tile t waits in register stage t % 2: while tile it is computed, tile it+1 sits in one stage
  // (loaded an iteration ago) and tile it+2 is being loaded into the other.  The loop is unrolled
  // by two so that the stages swap roles without a register copy (a copy would wait for loads
  // still in flight).
  TileStage<FP8> stage0, stage1;
  auto stage_scales = [&](int buf, int off) {
    if (threadIdx.x < kTT) {
      const int64_t sv = sl_lds[off + threadIdx.x];
      tok_scale[buf][threadIdx.x] = sv < 0 ? 0.f : (FP8 ? p.kv_scale[sv] : 1.f);
    }
  };
  if (ntiles > 0) {
    tile_load<FP8>(stage0, p, sl_lds, 0);
    if (ntiles > 1) tile_load<FP8>(stage1, p, sl_lds, kTT);
    stage_scales(0, 0);
    tile_store<FP8>(stage0, tile[0], sl_lds, 0);
  }
  __syncthreads();

  // one tile: `ld` receives tile it+2, `sv` holds tile it+1
  auto step = [&](int it, TileStage<FP8>& ld, const TileStage<FP8>& sv) {
    const int buf = it & 1;
    if (it + 2 < ntiles) tile_load<FP8>(ld, p, sl_lds, (it + 2) * kTT);
    const uint8_t* T = tile[buf];
    // ---- S^T half for two 16-token blocks; block beta row m holds token 8*(m/4) + 4*beta + m%4.
    // The blocks' K steps are interleaved (independent accumulators) and their LDS operands are
    // read kAhead steps before use.
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    if (active) {
      constexpr int kAhead = 3;
      const int m = lane & 15;
      const uint8_t* base0 = T + (8 * (m >> 2) + (m & 3)) * kPitch + grp * 16 + kh * (kKSteps * 64);
      const uint8_t* base1 = base0 + 4 * kPitch;
      bf16x8 a0[kAhead], a1[kAhead];
#pragma unroll
      for (int s = 0; s < kAhead; ++s) {
        a0[s] = *(const bf16x8*)(base0 + s * 64);
        a1[s] = *(const bf16x8*)(base1 + s * 64);
      }
#pragma unroll
      for (int s = 0; s < kKSteps; ++s) {
        const bf16x8 x0 = a0[s % kAhead], x1 = a1[s % kAhead];
        if (s + kAhead < kKSteps) {
          a0[s % kAhead] = *(const bf16x8*)(base0 + (s + kAhead) * 64);
          a1[s % kAhead] = *(const bf16x8*)(base1 + (s + kAhead) * 64);
        }
        sacc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x0, qf[s], sacc[0], 0, 0, 0);
        sacc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x1, qf[s], sacc[1], 0, 0, 0);
      }
      xs[wave][0][lane] = sacc[0];
      xs[wave][1][lane] = sacc[1];
    }
    __syncthreads();
    if (active) {
      // the full logits: half 0 + half 1, the same sum in both waves of the head group
      const int w0 = hg, w1 = hg + 4;
      const f32x4 s0 = xs[w0][0][lane] + xs[w1][0][lane];
      const f32x4 s1 = xs[w0][1][lane] + xs[w1][1][lane];
      // this lane holds head `head`, tokens 8*grp + 4*beta + j
      float z[8], sc[8];
      float tmax = -INFINITY;
#pragma unroll
      for (int beta = 0; beta < 2; ++beta)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = 8 * grp + 4 * beta + j;
          const float tsc = tok_scale[buf][t];
          sc[4 * beta + j] = tsc;
          const float sv = beta == 0 ? s0[j] : s1[j];
          const float zz = tsc != 0.f ? sv * tsc * scale2 : -INFINITY;
          z[4 * beta + j] = zz;
          tmax = fmaxf(tmax, zz);
        }
      tmax = lanes4_max(tmax);
      // the running maximum moves when this tile exceeds it by more than 2^8 (or on the first
      // live tile, where the accumulator is still zero and needs no rescale)
      const bool first = m_run == -INFINITY && tmax > -INFINITY;
      const bool need = tmax > m_run + 8.f && !first;
      if (__any(need)) {
        const float m_new = need ? tmax : m_run;
        const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < kDBlocks; ++db) o[db] *= alpha;
      }
      m_run = first ? tmax : m_run;
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pe = z[e] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(z[e] - m_run);
        l_run += pe;
        pb[e] = (__bf16)(FP8 ? pe * sc[e] : pe);
      }
      // ---- O^T += V^T . P^T over this wave's 256 output dims; V^T operand via transposing
      // LDS reads (4 tokens x 16 dims per read)
      const int jl = lane & 15;
      const uint8_t* vrow1 = T + (8 * grp + (jl >> 2)) * kPitch + (jl & 3) * 8 + kh * (kDBlocks * 32);
      const uint8_t* vrow2 = vrow1 + 4 * kPitch;
#pragma unroll
      for (int db = 0; db < kDBlocks; ++db) {
        const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (__attribute__((address_space(3))) bf16x4*)(vrow1 + db * 32));
        const bf16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (__attribute__((address_space(3))) bf16x4*)(vrow2 + db * 32));
        const bf16x8 av = __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7);
        o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb, o[db], 0, 0, 0);
      }
    }
    if (it + 1 < ntiles) {
      stage_scales(buf ^ 1, (it + 1) * kTT);
      tile_store<FP8>(sv, tile[buf ^ 1], sl_lds, (it + 1) * kTT);
    }
    __syncthreads();
  };
  for (int it = 0; it < ntiles; it += 2) {
    step(it, stage0, stage1);
    if (it + 1 < ntiles) step(it + 1, stage1, stage0);
  }

  if (!active) return;
  const float l_tot = lanes4_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  // lane holds O^T[d = 256kh + db*16 + grp*4 + j][head]
  if (p.n_split == 1) {
    float* dst = p.out + ((int64_t)r * p.H + head) * kVDim + kh * (kDBlocks * 16) + grp * 4;
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db) *(f32x4*)(dst + db * 16) = o[db] * inv;
    if (p.lse && grp == 0 && kh == 0)
      p.lse[(int64_t)r * p.H + head] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  } else {
    const int64_t prow = ((int64_t)r * p.n_split + split) * p.H + head;
    float* dst = p.part_o + prow * kVDim + kh * (kDBlocks * 16) + grp * 4;
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db) *(f32x4*)(dst + db * 16) = o[db] * inv;
    if (grp == 0 && kh == 0) {
      p.part_m[prow] = l_tot > 0.f ? m_run * kLn2 : -INFINITY;
      p.part_l[prow] = l_tot;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// fp8 rows: the same wave roles as mla_mfma_kernel, but the tile stays in e4m3fn in LDS and is
// widened to bf16 only as MFMA operands, which halves the LDS bytes written and read per token.
//   * Loads go straight from HBM into a ring of kRing tile buffers (direct-to-LDS copies, 16
//     bytes per lane, no register staging); kRing-1 tiles are in flight while one is computed.
//     Each 1 KiB copy reads whole rows (consecutive lanes, consecutive 16-byte pieces).
//   * Layout of a tile buffer: token t's row at t*576, its piece p (16 latent values) in slot
//     p ^ swz(t), swz(t) = bit 2 of t | (bit 3 ^ bit 4 of t) << 1 (a permutation inside each
//     aligned group of 4 pieces).  The S^T operand reads (16 tokens of one block, one piece)
//     and the transposing V^T reads (tokens 4g..4g+3 and 16+4g..16+4g+3 of lane group g) then
//     each cover all 64 LDS banks once per 32 lanes.
//   * S^T block beta holds tokens 16*beta .. 16*beta+15; lane group g of the S^T result holds
//     tokens 4g+j of both blocks, so the P.V contraction runs over the tokens in the order
//     tau(g, e) = 4g + e (e < 4), 16 + 4g + e - 4 (e >= 4), the same order in which the
//     transposing 8-bit read (ds_read_b64_tr_b8: the 16 lanes of a group supply 8 rows of 16
//     bytes, lane L gets column L) hands each lane its 8 V values.
//   * A token past the chunk or with slot -1 loads row 0 and is then zeroed in LDS, and its
//     logit is -inf.

typedef int i32x2 __attribute__((ext_vector_type(2)));
constexpr int kRing = 4;                                  // tile buffers (kRing-1 tiles in flight)
constexpr int kFp8Pieces = kRowDim / 16;                  // 36 pieces of 16 values per row
constexpr int kFp8TileBytes = kFp8Pieces * kTT * 16;      // 18432
constexpr int kFp8Dma = kFp8Pieces / 2;                   // 18 wave-wide 1 KiB copies per tile

__device__ __forceinline__ int fp8_swz(int t) { return ((t >> 2) & 1) | ((((t >> 3) ^ (t >> 4)) & 1) << 1); }
// LDS byte offset of logical piece p of token t inside a tile buffer
__device__ __forceinline__ int fp8_pos(int t, int p) { return t * kRowDim + ((p ^ fp8_swz(t)) << 4); }

// loads one wave issues per tile: copies wave, wave+8, wave+16 (< 18), plus the scales (wave 2)
__device__ __forceinline__ int fp8_loads_of_wave(int wave) { return (wave < 2 || wave == 2) ? 3 : 2; }

__global__ __launch_bounds__(kNT) void mla_fp8_kernel(MlaParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[kRing][kFp8TileBytes];
  __shared__ __attribute__((aligned(16))) float sring[kRing][64];     // per-token scales (token t at t)
  __shared__ __attribute__((aligned(16))) f32x4 xs[8][2][64];         // each wave's S^T half, per lane
  __shared__ int32_t sl_lds[kMaxTopK + kTT];                          // this chunk's slots, -1 padded

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hg = wave & 3, kh = wave >> 2;
  const int r = blockIdx.y, split = blockIdx.x;
  const int j0 = split * p.chunk;
  const int j1 = min(p.k, j0 + p.chunk);
  const int ntiles = j1 > j0 ? (j1 - j0 + kTT - 1) / kTT : 0;
  const int32_t* sl = p.slots + (int64_t)r * p.k;
  const bool active = hg * 16 < p.H;
  const int head = hg * 16 + (lane & 15);
  const int grp = lane >> 4;
  const uint8_t* kv = (const uint8_t*)p.kv;

  // stage the chunk's slot list (one coalesced pass, every load issued before any is used)
  {
    const int span = ntiles * kTT;
    for (int e0 = 0; e0 < span; e0 += 4 * kNT) {
      int32_t v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = sl[min(j0 + e0 + u * kNT + (int)threadIdx.x, p.k - 1)];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + u * kNT + threadIdx.x;
        if (e < span) sl_lds[e] = j0 + e < j1 ? dbg_slot(p.dbg, v[u], p.num_slots) : -1;
      }
    }
  }
  __syncthreads();

  // copies of tile v: lane i of copy c fills LDS slot q = 64c + i, i.e. token q/36, slot q%36,
  // which holds logical piece (q%36) ^ swz(token)
  auto issue = [&](int v) {
    uint8_t* base = ring[v % kRing];
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      const int cc = wave + 8 * c;
      if (cc < kFp8Dma) {
        const int q = cc * 64 + lane;
        const int t = q / kFp8Pieces, sp = q - t * kFp8Pieces;
        const int32_t sv = sl_lds[v * kTT + t];
        const uint8_t* src = kv + (int64_t)(sv < 0 ? 0 : sv) * kRowDim + ((sp ^ fp8_swz(t)) << 4);
        lds_dma16(src, base + cc * 1024);
      }
    }
    if (wave == 2) {
      const int32_t ss = sl_lds[v * kTT + (lane & 31)];
      lds_dma4(p.kv_scale + (ss < 0 ? 0 : ss), sring[v % kRing]);
    }
  };

  // q fragments (B operand of S^T): head lane%16, dims (9kh + s)*32 + grp*8 .. +8
  bf16x8 qf[kKSteps];
  if (active) {
    const bf16x8* qrow = (const bf16x8*)((const __bf16*)p.q + ((int64_t)r * p.H + head) * kRowDim);
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) qf[s] = qrow[(kKSteps * kh + s) * 4 + grp];
  }
#pragma unroll
  for (int v = 0; v < kRing - 1; ++v)
    if (v < ntiles) issue(v);

  f32x4 o[kDBlocks];
#pragma unroll
  for (int db = 0; db < kDBlocks; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;   // running max of z * log2(e), per head
  float l_run = 0.f;         // this lane group's share of sum exp2(z - m_run)
  const float scale2 = p.sm_scale * kLog2e;

  // per-lane LDS offsets inside a tile buffer
  const int m16 = lane & 15;
  // S^T operand of block beta, K step s: logical piece P0 + 2s (P0 = 18kh + grp/2), half grp%2
  // of token 16beta + m16.  Steps of one parity differ by 32 bytes per step (the swizzle only
  // permutes inside aligned groups of 4 pieces), so two bases per block cover all 9 steps.
  const int P0 = 18 * kh + (grp >> 1);
  int a_base[2][2];
#pragma unroll
  for (int beta = 0; beta < 2; ++beta) {
    a_base[beta][0] = fp8_pos(16 * beta + m16, P0) + 8 * (grp & 1);
    a_base[beta][1] = fp8_pos(16 * beta + m16, P0 + 2) + 8 * (grp & 1) - 32;
  }
  // V^T operand of dim block db (logical piece 16kh + db): row e = m16/2 of the group's 8x16
  // block is token tau(grp, e); blocks 4 apart differ by 64 bytes
  const int e_row = m16 >> 1;
  const int tau = e_row < 4 ? 4 * grp + e_row : 16 + 4 * grp + (e_row - 4);
  int v_base[4];
#pragma unroll
  for (int d4 = 0; d4 < 4; ++d4) v_base[d4] = fp8_pos(tau, 16 * kh + d4) + 8 * (m16 & 1);
  const int wl = fp8_loads_of_wave(wave);

  for (int v = 0; v < ntiles; ++v) {
    const int later = min(kRing - 2, ntiles - 1 - v);   // tiles whose loads were issued after v's
    if (wl == 3) {
      if (later >= 2) wait_vmcnt<6>();
      else if (later == 1) wait_vmcnt<3>();
      else wait_vmcnt<0>();
    } else {
      if (later >= 2) wait_vmcnt<4>();
      else if (later == 1) wait_vmcnt<2>();
      else wait_vmcnt<0>();
    }
    lds_barrier();   // tile v landed for every wave; buffer (v-1) % kRing is no longer read
    if (v + kRing - 1 < ntiles) issue(v + kRing - 1);
    const int buf = v % kRing;
    uint8_t* T = ring[buf];
    const int toff = v * kTT;
    // skipped tokens (past the chunk, or slot -1) read row 0: zero their rows
    // (every wave reads the same slot list, so the choice is uniform over the workgroup)
    if (__ballot(lane < kTT && sl_lds[toff + (lane & (kTT - 1))] < 0)) {
      for (int e = threadIdx.x; e < kTT * kFp8Pieces; e += kNT) {
        const int t = e / kFp8Pieces, pc = e - t * kFp8Pieces;
        if (sl_lds[toff + t] < 0) *(u32x4*)(T + t * kRowDim + pc * 16) = u32x4{0u, 0u, 0u, 0u};
      }
      lds_barrier();
    }

    // ---- S^T half for the two 16-token blocks, K steps interleaved, operands read ahead
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    if (active) {
      constexpr int kAhead = 3;
      u32x2 a0[kAhead], a1[kAhead];
#pragma unroll
      for (int s = 0; s < kAhead; ++s) {
        a0[s] = *(const u32x2*)(T + a_base[0][s & 1] + 32 * s);
        a1[s] = *(const u32x2*)(T + a_base[1][s & 1] + 32 * s);
      }
#pragma unroll
      for (int s = 0; s < kKSteps; ++s) {
        const u32x2 x0 = a0[s % kAhead], x1 = a1[s % kAhead];
        if (s + kAhead < kKSteps) {
          a0[s % kAhead] = *(const u32x2*)(T + a_base[0][(s + kAhead) & 1] + 32 * (s + kAhead));
          a1[s % kAhead] = *(const u32x2*)(T + a_base[1][(s + kAhead) & 1] + 32 * (s + kAhead));
        }
        sacc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16x8(x0[0], x0[1]), qf[s], sacc[0], 0, 0, 0);
        sacc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16x8(x1[0], x1[1]), qf[s], sacc[1], 0, 0, 0);
      }
      xs[wave][0][lane] = sacc[0];
      xs[wave][1][lane] = sacc[1];
    }
    lds_barrier();
    if (active) {
      // the full logits: half 0 + half 1, the same sum in both waves of the head group
      const f32x4 s0 = xs[hg][0][lane] + xs[hg + 4][0][lane];
      const f32x4 s1 = xs[hg][1][lane] + xs[hg + 4][1][lane];
      // this lane holds head `head`, tokens 16*beta + 4*grp + j (K index 4*beta + j of P.V)
      float z[8], sc[8];
      float tmax = -INFINITY;
#pragma unroll
      for (int beta = 0; beta < 2; ++beta)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = 16 * beta + 4 * grp + j;
          const bool live = sl_lds[toff + t] >= 0;
          const float tsc = sring[buf][t];
          sc[4 * beta + j] = tsc;
          const float sv = beta == 0 ? s0[j] : s1[j];
          const float zz = live ? sv * tsc * scale2 : -INFINITY;
          z[4 * beta + j] = zz;
          tmax = fmaxf(tmax, zz);
        }
      tmax = lanes4_max(tmax);
      const bool first = m_run == -INFINITY && tmax > -INFINITY;
      const bool need = tmax > m_run + 8.f && !first;
      if (__any(need)) {
        const float m_new = need ? tmax : m_run;
        const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < kDBlocks; ++db) o[db] *= alpha;
      }
      m_run = first ? tmax : m_run;
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pe = z[e] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(z[e] - m_run);
        l_run += pe;
        pb[e] = (__bf16)(pe * sc[e]);
      }
      // ---- O^T += V^T . P^T over this wave's 256 output dims (pieces 16kh .. 16kh+15)
#pragma unroll
      for (int db = 0; db < kDBlocks; ++db) {
        const u32x2 raw = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(T + v_base[db & 3] + 64 * (db >> 2))));
        o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16x8(raw[0], raw[1]), pb, o[db], 0, 0, 0);
      }
    }
  }

  if (!active) return;
  const float l_tot = lanes4_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  // lane holds O^T[d = 256kh + db*16 + grp*4 + j][head]
  if (p.n_split == 1) {
    float* dst = p.out + ((int64_t)r * p.H + head) * kVDim + kh * (kDBlocks * 16) + grp * 4;
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db) *(f32x4*)(dst + db * 16) = o[db] * inv;
    if (p.lse && grp == 0 && kh == 0)
      p.lse[(int64_t)r * p.H + head] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  } else {
    const int64_t prow = ((int64_t)r * p.n_split + split) * p.H + head;
    float* dst = p.part_o + prow * kVDim + kh * (kDBlocks * 16) + grp * 4;
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db) *(f32x4*)(dst + db * 16) = o[db] * inv;
    if (grp == 0 && kh == 0) {
      p.part_m[prow] = l_tot > 0.f ? m_run * kLn2 : -INFINITY;
      p.part_l[prow] = l_tot;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// fp8 rows, chunks of at most kChunkF selected rows: 8 waves (two per SIMD, at most 256
// registers each), 32-token tiles kept as e4m3 in LDS.
//   * Tiles are loaded HBM -> registers (per wave two loads of 1 KiB of whole rows, one of 256
//     bytes and the scales) three steps ahead and stored into one of three LDS slots: while tile
//     v is computed, the loads of tiles v+1 .. v+3 are in flight, and the compiler's wait before
//     each store counts only the later tiles' loads.  A skipped token
//     (slot -1) reads row 0 and is zeroed on the way into LDS.  Layout: row t at t*576, 16-byte
//     piece p in slot p ^ fp8_swz(t) (conflict-free for both operand reads below).
//   * S^T: wave w owns head group hg = w % 4 (heads 16hg .. 16hg+15, q in registers as bf16)
//     and token block tb = w / 4 (tokens 16tb .. 16tb+15) over the full K.  Each 16-byte LDS
//     read gives a lane 16 e4m3 values of its token, widened exactly to bf16 for two K steps of
//     v_mfma_f32_16x16x32_bf16, so every product is exact in the fp32 accumulator.  Lane group
//     g of the result holds tokens 16tb + 4g .. +3 of its head: the half of the P^T operand that
//     the token ordering tau below assigns to it, written to LDS for the other waves.
//   * P.V: wave w owns the output values 64w .. 64w+63 for all 64 heads; the V^T operand
//     (ds_read_b64_tr_b8, tokens in the order tau(g, e) = 4g + e for e < 4, 16 + 4g + e - 4
//     otherwise, then widened) is read once and feeds the four head groups' MFMAs.
//   * Softmax against a fixed per-head reference R (the largest logit of the chunk's first
//     tile over both token blocks, 0 if it has no live token); P = exp2(z - R) stays finite and
//     accurate while the head's logits lie within R +- 64 (log2 units), otherwise the chunk is
//     computed again with R = the head's largest logit.  The accumulators are only touched by
//     the matrix core.
//   * Two barriers per tile (next tile stored; P published).
constexpr int kTF = 32;                                   // tokens per tile
constexpr int kTFBytes = kTF * kRowDim;                   // 18432
constexpr int kNTF = 512;                                 // 8 waves
constexpr int kChunkF = 2048;                             // selected rows staged per workgroup
constexpr int kStepsF = kRowDim / 32;                     // 18 K steps of 32
constexpr int kDBlocksF = kVDim / 16 / 8;                 // 4 output blocks of 16 per wave

struct FDSmem {
  uint8_t ring[3][kTFBytes + kTF * 4];        // tile, then its 32 per-token scales
  int32_t sl[kChunkF + kTF];                  // the chunk's slots, -1 padded
  bf16x8 pex[4][64];                          // P^T operands: head group, lane
  float m0[2][64];                            // largest logit of the first tile, by token block
  float fin_m[2][64], fin_l[2][64];           // per head and token block, after the last tile
  int32_t redo;
};

__global__ __launch_bounds__(kNTF) void mla_fp8d_kernel(MlaParams p) {
  __shared__ __attribute__((aligned(16))) FDSmem sm;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hg = wave & 3, tb = wave >> 2;
  // Blocks go to the 8 XCDs round-robin.  With 8 rows or more, row group u = r / p.group (a
  // sequence's verify rows, or one row) runs on XCD u % 8, so each row's q is read from HBM into
  // one L2, and within an XCD the group's rows take chunk `split` one after another: tokens
  // selected by several rows of a sequence are read from HBM once.  With fewer rows the chunks
  // spread over all XCDs.
  int r, split;
  if (p.rows >= 8) {
    const int xcd = blockIdx.x & 7, jx = blockIdx.x >> 3;
    const int t = jx / p.group, ri = jx - t * p.group;
    const int uu = t / p.n_split;
    split = t - uu * p.n_split;
    r = (8 * uu + xcd) * p.group + ri;
    if (r >= p.rows) return;
  } else {
    r = blockIdx.x / p.n_split;
    split = blockIdx.x - r * p.n_split;
  }
  const int j0 = split * p.chunk;
  const int j1 = min(p.k, j0 + p.chunk);
  const int ntiles = j1 > j0 ? (j1 - j0 + kTF - 1) / kTF : 0;
  const int32_t* sl = p.slots + (int64_t)r * p.k;
  const int ngroups = min(4, p.H / 16);           // live head groups (H is a multiple of 16)
  const bool s_active = hg < ngroups;             // this wave's S^T head group exists
  const int m16 = lane & 15, grp = lane >> 4;

  // The chunk's slots (at most 4 * 512 = kChunkF) are requested, then q of this wave's head
  // group (B operand of S^T: head 16hg + m16, a group past the head count loads the last head
  // and never uses it; K step 2u + h holds dims 64u + 16grp + 8h .. +8, the order in which a
  // lane's 16-byte row piece 4u + grp is widened), then the slots are written to LDS: the wait
  // for the slots (the older loads) leaves q in flight through the barrier and the first tile
  // loads.
  static_assert(kChunkF <= 4 * kNTF, "one round of slot loads");
  const int span = ntiles * kTF;
  int32_t slv[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) slv[u] = sl[min(j0 + u * kNTF + (int)threadIdx.x, p.k - 1)];
  __builtin_amdgcn_sched_barrier(0);   // (the slot loads stay ahead of q's)
  bf16x8 qf[kStepsF];
  {
    const int qhead = min(hg * 16 + m16, p.H - 1);
    const bf16x8* qrow = (const bf16x8*)((const __bf16*)p.q + ((int64_t)r * p.H + qhead) * kRowDim);
#pragma unroll
    for (int u = 0; u < kStepsF / 2; ++u)
#pragma unroll
      for (int h = 0; h < 2; ++h) qf[2 * u + h] = qrow[8 * u + 2 * grp + h];
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = u * kNTF + threadIdx.x;
    if (e < span) sm.sl[e] = j0 + e < j1 ? dbg_slot(p.dbg, slv[u], p.num_slots) : -1;
  }
  if (threadIdx.x == 0) sm.redo = 0;
  if (!s_active && tb == 0) sm.pex[hg][lane] = bf16x8{};   // head groups past the head count: P = 0
  lds_barrier();

  // ---- staging of tile v: every wave issues the same four loads per tile.  Loads 0 and 1 of
  // wave w read the tile's 16-byte pieces q = 64(w + 8c) + lane (1 KiB of whole rows each), load
  // 2 the 4 bytes at tile offset 16384 + 256w + 4 lane, load 3 the scale of token 4w + lane % 4.
  // Tile offset o holds token o / 576 at LDS slot (o % 576) / 16, i.e. the row's logical piece
  // slot ^ fp8_swz(token).  Tiles past the chunk re-read row 0 and are never used, so every
  // step issues the same loads.
  struct Stage {
    u32x4 d[2];
    uint32_t e;
    float sc;
    uint32_t dead;   // bit c: load c belongs to a skipped token
  };
  const int e_off = kTFBytes - 2048 + 256 * wave + 4 * lane;   // tile offset of load 2
  auto row_src = [&](int o, int32_t sv) {                       // global address of tile offset o
    const int t = o / kRowDim, w = o - t * kRowDim;
    return (const uint8_t*)p.kv + (int64_t)(sv < 0 ? 0 : sv) * kRowDim + ((((w >> 4) ^ fp8_swz(t)) << 4) | (w & 15));
  };
  auto load_tile = [&](const FDSmem* __restrict__ rd, Stage& st, int v) {
    const bool real = v < ntiles;
    const int vb = (real ? v : 0) * kTF;          // (a tile past the chunk reads entries it ignores)
    uint32_t dead = 0u;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int o = ((wave + 8 * c) * 64 + lane) * 16;
      const int32_t sl_t = rd->sl[vb + o / kRowDim];
      const int32_t sv = real ? sl_t : 0;
      dead |= (sv < 0 ? 1u : 0u) << c;
      st.d[c] = *(const u32x4*)row_src(o, sv);
    }
    {
      const int32_t sl_t = rd->sl[vb + e_off / kRowDim];
      const int32_t sv = real ? sl_t : 0;
      dead |= (sv < 0 ? 4u : 0u);
      st.e = *(const uint32_t*)row_src(e_off, sv);
    }
    const int32_t sl_s = rd->sl[vb + 4 * wave + (lane & 3)];
    const int32_t ss = real ? sl_s : 0;
    st.sc = p.kv_scale[ss < 0 ? 0 : ss];
    st.dead = dead;
  };
  auto store_tile = [&](const Stage& st, uint8_t* __restrict__ dst) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int o = ((wave + 8 * c) * 64 + lane) * 16;
      *(u32x4*)(dst + o) = (st.dead >> c) & 1u ? u32x4{0u, 0u, 0u, 0u} : st.d[c];
    }
    *(uint32_t*)(dst + e_off) = st.dead & 4u ? 0u : st.e;
    if (lane < 4) *(float*)(dst + kTFBytes + 4 * (4 * wave + lane)) = st.sc;
  };

  Stage X, Y, Z;
  load_tile(&sm, X, 0);
  load_tile(&sm, Y, 1);
  load_tile(&sm, Z, 2);

  // P.V accumulators: head group g, output block db; lane holds O^T[64w + 16db + 4grp + j][16g + m16]
  f32x4 o[4][kDBlocksF];
  const float scale2 = p.sm_scale * kLog2e;
  float ref = 0.f;           // R of this lane's head
  float m_seen = -INFINITY;  // the head's largest logit in this wave's token block
  float l_run = 0.f;         // this lane group's share of sum exp2(z - R)

  // S^T operand: token 16tb + m16, logical piece 4u + grp at a_off + 64u
  const int a_off = fp8_pos(16 * tb + m16, grp);
  // V^T operand of output block db: row e = m16/2 of the group's 8x16 block is token tau(grp, e);
  // value block 4w + db is logical piece db of the 64-byte group at 64w
  const int e_row = m16 >> 1;
  const int tau = e_row < 4 ? 4 * grp + e_row : 16 + 4 * grp + (e_row - 4);
  int v_base[kDBlocksF];
#pragma unroll
  for (int db = 0; db < kDBlocksF; ++db) v_base[db] = fp8_pos(tau, db) + 8 * (m16 & 1) + 64 * wave;

  auto s_tile = [&](const uint8_t* __restrict__ T) -> f32x4 {
    f32x4 acc0 = f32x4{0.f, 0.f, 0.f, 0.f}, acc1 = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr int kAhead = 2;
    u32x4 a[kAhead];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) a[u] = *(const u32x4*)(T + a_off + 64 * u);
#pragma unroll
    for (int u = 0; u < kStepsF / 2; ++u) {
      const u32x4 x = a[u % kAhead];
      if (u + kAhead < kStepsF / 2) a[u % kAhead] = *(const u32x4*)(T + a_off + 64 * (u + kAhead));
      const bf16x8 lo = fp8x8_to_bf16x8(x[0], x[1]);
      const bf16x8 hi = fp8x8_to_bf16x8(x[2], x[3]);
      // two accumulators so that consecutive MFMAs do not wait on each other
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, qf[2 * u], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, qf[2 * u + 1], acc1, 0, 0, 0);
    }
    return acc0 + acc1;
  };
  // lane holds head 16hg + m16, tokens 16tb + 4grp + j: logits (scale folded), -inf if skipped
  auto logits = [&](const FDSmem* __restrict__ rd, const uint8_t* __restrict__ T, int v, const f32x4& sacc,
                    float (&z)[4], float (&sc)[4]) {
    const int t0 = 16 * tb + 4 * grp;
    const int32_t* slt = rd->sl + v * kTF + t0;
    const f32x4 sc4 = *(const f32x4*)(T + kTFBytes + 4 * t0);
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sc[j] = sc4[j];
      z[j] = slt[j] >= 0 ? sacc[j] * sc4[j] * scale2 : -INFINITY;
      tmax = fmaxf(tmax, z[j]);
    }
    return lanes4_max(tmax);   // over the block's 16 tokens
  };
  auto publish = [&](FDSmem* __restrict__ rd, const float (&z)[4], const float (&sc)[4]) {
    bf16x4 pb;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float pe = z[j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(z[j] - ref);
      l_run += pe;
      pb[j] = (__bf16)(pe * sc[j]);
    }
    *(bf16x4*)((uint8_t*)&rd->pex[hg][lane] + 8 * tb) = pb;
  };
  auto pv_tile = [&](const FDSmem* __restrict__ rd, const uint8_t* __restrict__ T) {
    u32x2 raw[kDBlocksF];
#pragma unroll
    for (int db = 0; db < kDBlocksF; ++db)
      raw[db] = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(T + v_base[db])));
    bf16x8 av[kDBlocksF];
#pragma unroll
    for (int db = 0; db < kDBlocksF; ++db) av[db] = fp8x8_to_bf16x8(raw[db][0], raw[db][1]);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const bf16x8 pg = rd->pex[g][lane];
#pragma unroll
      for (int db = 0; db < kDBlocksF; ++db) o[g][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[db], pg, o[g][db], 0, 0, 0);
    }
  };
  // one tile (v, in ring slot T): S^T, the first tile's reference, P, then P.V
  auto tile = [&](FDSmem* __restrict__ rd, const uint8_t* __restrict__ T, int v, bool first) {
    float z[4], sc[4];
    float tmax = -INFINITY;
    if (s_active) tmax = logits(rd, T, v, s_tile(T), z, sc);
    if (first) {
      // the reference: the first tile's largest logit over both token blocks (0 without one)
      if (s_active && grp == 0) rd->m0[tb][hg * 16 + m16] = tmax;
      lds_barrier();
      if (s_active) {
        const float m0 = fmaxf(rd->m0[0][hg * 16 + m16], rd->m0[1][hg * 16 + m16]);
        ref = m0 == -INFINITY ? 0.f : m0;
      }
    }
    if (s_active) {
      m_seen = fmaxf(m_seen, tmax);
      publish(rd, z, sc);
    }
    lds_barrier();   // P of the tile is published
    pv_tile(rd, T);
  };

  // Pipeline: while tile v is computed from ring slot v % 3, the loads of tiles v+2 and v+3 are
  // in flight, and tile v+1 (requested two steps earlier) is stored into slot (v+1) % 3
  // afterwards.  Three steps per loop trip, so X, Y and Z keep their registers.  Pass 0 takes R
  // from the first tile; pass 1 (rare) recomputes the chunk with R = the largest logit.  Each
  // pass has its own copy of the loop (the lambda is expanded twice), so that the compiler sees
  // one fixed set of loads in flight at each loop entry and its waits before the stores stay
  // partial.
  auto run_pass = [&](bool first) {
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int db = 0; db < kDBlocksF; ++db) o[g][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    l_run = 0.f;
    store_tile(X, sm.ring[0]);
    lds_barrier();   // tile 0 landed
    for (int v = 0; v < ntiles; v += 3) {
      load_tile(&sm, X, v + 3);
      tile(&sm, sm.ring[0], v, first && v == 0);
      store_tile(Y, sm.ring[1]);
      lds_barrier();   // tile v + 1 landed; tile v and its P are no longer read
      load_tile(&sm, Y, v + 4);
      if (v + 1 < ntiles) tile(&sm, sm.ring[1], v + 1, false);
      store_tile(Z, sm.ring[2]);
      lds_barrier();   // tile v + 2 landed
      load_tile(&sm, Z, v + 5);
      if (v + 2 < ntiles) tile(&sm, sm.ring[2], v + 2, false);
      store_tile(X, sm.ring[0]);
      lds_barrier();   // tile v + 3 landed
    }
    // does some head's largest logit lie outside R +- 64?
    if (s_active) {
      const float l_blk = lanes4_sum(l_run);   // (all lanes of the wave take part)
      if (grp == 0) {
        sm.fin_m[tb][hg * 16 + m16] = m_seen;
        sm.fin_l[tb][hg * 16 + m16] = l_blk;
      }
    }
    __syncthreads();
  };
  run_pass(true);
  {
    float mx = -INFINITY;
    if (s_active) {
      mx = fmaxf(sm.fin_m[0][hg * 16 + m16], sm.fin_m[1][hg * 16 + m16]);
      if (mx > -INFINITY && (mx > ref + kRefMargin || mx < ref - kRefMargin)) sm.redo = 1;
    }
    __syncthreads();
    if (sm.redo) {
      ref = mx > -INFINITY ? mx : 0.f;
      load_tile(&sm, X, 0);
      load_tile(&sm, Y, 1);
      load_tile(&sm, Z, 2);
      run_pass(false);
    }
  }

  // ---- output: each wave writes its 64 values of every head
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    if (g >= ngroups) break;
    const int head = g * 16 + m16;
    const float mh = fmaxf(sm.fin_m[0][head], sm.fin_m[1][head]);
    const float lh = sm.fin_l[0][head] + sm.fin_l[1][head];
    // R of this head as its S^T waves used it (recomputed from what they published)
    const float m0 = fmaxf(sm.m0[0][head], sm.m0[1][head]);
    const float rh = sm.redo ? (mh > -INFINITY ? mh : 0.f) : (m0 == -INFINITY ? 0.f : m0);
    const float inv = lh > 0.f ? 1.f / lh : 0.f;
    float* dst;
    if (p.n_split == 1) {
      dst = p.out + ((int64_t)r * p.H + head) * kVDim + wave * 64 + grp * 4;
      if (p.lse && wave == 0 && grp == 0)
        p.lse[(int64_t)r * p.H + head] = lh > 0.f ? (rh + log2f(lh)) * kLn2 : -INFINITY;
    } else {
      const int64_t prow = ((int64_t)r * p.n_split + split) * p.H + head;
      dst = p.part_o + prow * kVDim + wave * 64 + grp * 4;
      if (wave == 0 && grp == 0) {
        p.part_m[prow] = lh > 0.f ? rh * kLn2 : -INFINITY;
        p.part_l[prow] = lh;
      }
    }
#pragma unroll
    for (int db = 0; db < kDBlocksF; ++db) *(f32x4*)(dst + db * 16) = o[g][db] * inv;
  }
}

// ---------------------------------------------------------------------------------------------
// bf16 rows, chunks of at most kChunkD selected rows: 8 waves (two per SIMD), 32-token tiles
// copied HBM -> LDS directly into a ring of kRingD tile buffers (three tiles in flight).
//   * Layout of a tile buffer: token t's row at t*1152, its 16-byte piece p in slot
//     p ^ swzd(t), swzd(t) = (bit 4 of t) | (bit 1 of t) << 1 | (bit 3 of t) << 2 (a permutation
//     inside each aligned group of 8 pieces), so that the S^T operand reads (16 tokens of a
//     block, one piece) and the transposing V^T reads (tokens 8g..8g+3 of two lane groups, two
//     pieces) touch every LDS bank once.  Copy c, lane i fills slot q = 64c + i; a skipped slot
//     (-1) reads past the buffer resource's last record, which lands as zeros.
//   * S^T: wave w owns head group hg = w % 4 (heads 16hg .. 16hg+15) and token block
//     tb = w / 4 over the full K (q in registers).  Block tb row m holds token
//     8(m/4) + 4tb + m%4, so lane group g of the result holds tokens 8g + 4tb .. +3 of its head,
//     one half of the P^T operand's 8 tokens 8g .. 8g+7; the two waves of a head group write
//     their halves of it to LDS.
//   * P.V: wave w owns the output values 64w .. 64w+63 for all 64 heads (each V^T operand is
//     read once per workgroup and feeds four head groups' MFMAs).
//   * Softmax without rescaling: P = exp2(z - R) with a fixed reference per head, the largest
//     logit of the chunk's first tile (0 if that tile has no live token).  The accumulators are
//     then only touched by the matrix core.  P, the sums and the accumulators stay finite and
//     accurate while the head's largest logit is within R +- 64 (a factor of 2^64); otherwise
//     the chunk is computed again with R = that largest logit.

constexpr int kRingD = 4;                                 // tile buffers (3 tiles in flight)
constexpr int kChunkD = 2048;                             // selected rows staged per workgroup
constexpr int kTDBytes = kTT * kRowDim * 2;               // 36864
constexpr int kTDCopies = kTDBytes / 1024;                // 36 copies of 1 KiB per tile
constexpr int kStepsD = kRowDim / 32;                     // 18 K steps of 32
constexpr int kDBlocksD = kVDim / 16 / 8;                 // 4 output blocks of 16 per wave
constexpr int kStageLd = kVDim + 16;                       // floats per staged output row
static_assert(64 * kStageLd * 4 <= kRingD * kTDBytes, "the staged output must fit the tile ring");

__device__ __forceinline__ int bf16_swz(int t) { return ((t >> 4) & 1) | (((t >> 1) & 1) << 1) | (((t >> 3) & 1) << 2); }
// LDS byte offset of logical piece p of token t inside a tile buffer
__device__ __forceinline__ int bf16_pos(int t, int p) { return t * (kRowDim * 2) + ((p ^ bf16_swz(t)) << 4); }

struct BDSmem {
  uint8_t ring[kRingD][kTDBytes];
  bf16x8 pex[4][64];                          // P^T operands: head group, lane
  int32_t sl[kChunkD + 3 * kTT];              // the chunk's slots, -1 padded past the chunk
  float m0[2][64];                            // largest logit of the first tile, by token block
  float fin_m[2][64], fin_l[2][64], fin_r[2][64];   // per head and token block, after the last tile
  int32_t redo;
};

__global__ __launch_bounds__(kNT) void mla_bf16d_kernel(MlaParams p) {
  __shared__ __attribute__((aligned(16))) BDSmem sm;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hg = wave & 3, tb = wave >> 2;
  // Blocks go to the 8 XCDs round-robin, as in mla_fp8d_kernel: with 8 rows or more, row group
  // r / p.group runs on XCD (r / p.group) % 8 (the grid covers the groups rounded up to a
  // multiple of 8), its rows taking each chunk one after another; with fewer rows the chunks
  // spread over all XCDs.
  int r, split;
  if (p.rows >= 8) {
    const int xcd = blockIdx.x & 7, jx = blockIdx.x >> 3;
    const int t = jx / p.group, ri = jx - t * p.group;
    const int uu = t / p.n_split;
    split = t - uu * p.n_split;
    r = (8 * uu + xcd) * p.group + ri;
    if (r >= p.rows) return;
  } else {
    r = blockIdx.x / p.n_split;
    split = blockIdx.x - r * p.n_split;
  }
  const int j0 = split * p.chunk;
  const int j1 = min(p.k, j0 + p.chunk);
  const int ntiles = j1 > j0 ? (j1 - j0 + kTT - 1) / kTT : 0;
  const int32_t* sl = p.slots + (int64_t)r * p.k;
  const int ngroups = min(4, p.H / 16);           // live head groups (H is a multiple of 16)
  const bool s_active = hg < ngroups;             // this wave's S^T head group exists
  const int m16 = lane & 15, grp = lane >> 4;

  // The chunk's slots (at most 4 * 512 = kChunkD) are requested, then q of this wave's head
  // group (B operand of S^T: head 16hg + m16, dims 32s + 8grp .. +8; a group past the head count
  // loads the last head and never uses it), then the slots are written to LDS: the wait for
  // the slots (the older loads) leaves q in flight through the barrier and the first tile
  // copies, and the wait for tile 0 covers it.
  static_assert(kChunkD <= 4 * kNT, "one round of slot loads");
  const int span = ntiles * kTT;
  int32_t slv[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) slv[u] = sl[min(j0 + u * kNT + (int)threadIdx.x, p.k - 1)];
  __builtin_amdgcn_sched_barrier(0);   // (the slot loads stay ahead of q's)
  bf16x8 qf[kStepsD];
  {
    const int qhead = min(hg * 16 + m16, p.H - 1);
    const bf16x8* qrow = (const bf16x8*)((const __bf16*)p.q + ((int64_t)r * p.H + qhead) * kRowDim);
#pragma unroll
    for (int s = 0; s < kStepsD; ++s) qf[s] = qrow[4 * s + grp];
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = u * kNT + threadIdx.x;
    if (e < span) sm.sl[e] = j0 + e < j1 ? dbg_slot(p.dbg, slv[u], p.num_slots) : -1;
  }
  if (threadIdx.x == 0) sm.redo = 0;
  if (!s_active) sm.pex[hg][lane] = bf16x8{};   // head groups past the head count: P = 0
  lds_barrier();

  // copies of tile v: wave w issues copies w, w+8, .. (< 36): 5 for waves 0-3, 4 for waves 4-7
  const int nld = wave < kTDCopies - 4 * 8 ? 5 : 4;
  const __amdgpu_buffer_rsrc_t kv_rs = rows_rsrc(p.kv, kRowDim * 2, p.num_slots);
  auto issue_one = [&](const BDSmem* __restrict__ rd, uint8_t* __restrict__ dst, int v, int c) {
    const int cc = wave + 8 * c;
    if (c < 4 || cc < kTDCopies) {
      const int q = cc * 64 + lane;
      const int t = q / 72, sp = q - t * 72;
      const int32_t sv = rd->sl[v * kTT + t];
      // a skipped slot reads past the last record: zeros
      lds_dma16_row(kv_rs, sv < 0 ? 0x7fffffff : sv, (sp ^ bf16_swz(t)) << 4, dst + cc * 1024);
    }
  };
  auto issue = [&](const BDSmem* __restrict__ rd, uint8_t* __restrict__ dst, int v) {
#pragma unroll
    for (int c = 0; c < 5; ++c) issue_one(rd, dst, v, c);
  };
  auto wait_tile = [&](int later) {   // at most `later` later tiles' copies outstanding
    if (nld == 5) wait_vmcnt_later<5, kRingD - 2>(later);
    else wait_vmcnt_later<4, kRingD - 2>(later);
  };

  // P.V accumulators: head group g, output block db; lane holds O^T[64w + 16db + 4grp + j][16g + m16]
  f32x4 o[4][kDBlocksD];
  const float scale2 = p.sm_scale * kLog2e;
  float ref = 0.f;           // R of this lane's head
  float m_seen = -INFINITY;  // the head's largest logit in this wave's token blocks
  float l_run = 0.f;         // this lane group's share of sum exp2(z - R)
  float l_rnd = 0.f;         // the same sum of P as rounded to bf16 for P.V (the output's normaliser)

  // S^T operand of block tb: row m = token 8(m/4) + 4tb + m%4, logical piece 4s + grp
  const int a_tok = 8 * (m16 >> 2) + 4 * tb + (m16 & 3);
  // V^T operand: lane jl of group grp reads token 8grp + jl/4 (+4), bytes 8(jl%4) of the 32-byte
  // block of dims 64w + 16db
  const int v_tok = 8 * grp + (m16 >> 2);

  // S^T of the tile at T; with nv >= 0 the copies of tile nv into dst are issued between the
  // MFMAs (copy c before step 3c + 1), where a wait for room in the memory pipeline overlaps
  // the matrix core's work
  auto s_tile = [&](const BDSmem* __restrict__ rd, const uint8_t* __restrict__ T, uint8_t* __restrict__ dst, int nv) -> f32x4 {
    f32x4 acc0 = f32x4{0.f, 0.f, 0.f, 0.f}, acc1 = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr int kAhead = 4;
    bf16x8 a[kAhead];
#pragma unroll
    for (int s = 0; s < kAhead; ++s) a[s] = *(const bf16x8*)(T + bf16_pos(a_tok, 4 * s + grp));
#pragma unroll
    for (int s = 0; s < kStepsD; ++s) {
      if (s % 3 == 1 && s / 3 < 5 && nv >= 0) issue_one(rd, dst, nv, s / 3);
      const bf16x8 x = a[s % kAhead];
      if (s + kAhead < kStepsD) a[s % kAhead] = *(const bf16x8*)(T + bf16_pos(a_tok, 4 * (s + kAhead) + grp));
      // two accumulators (even / odd steps) so that consecutive MFMAs do not wait on each other
      if (s & 1) acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, qf[s], acc1, 0, 0, 0);
      else acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, qf[s], acc0, 0, 0, 0);
    }
    return acc0 + acc1;
  };
  // lane holds head 16hg + m16, tokens 8grp + 4tb + j: logits, -inf for a skipped slot
  auto logits = [&](const BDSmem* __restrict__ rd, int v, const f32x4& sacc, float (&z)[4]) {
    const int32_t* slt = rd->sl + v * kTT + 8 * grp + 4 * tb;
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      z[j] = slt[j] >= 0 ? sacc[j] * scale2 : -INFINITY;
      tmax = fmaxf(tmax, z[j]);
    }
    return lanes4_max(tmax);   // over the block's 16 tokens
  };
  auto publish = [&](BDSmem* __restrict__ rd, const float (&z)[4]) {
    bf16x4 pb;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float pe = z[j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(z[j] - ref);
      l_run += pe;
      pb[j] = (__bf16)pe;
      l_rnd += (float)pb[j];
    }
    *(bf16x4*)((uint8_t*)&rd->pex[hg][lane] + 8 * tb) = pb;
  };
  auto pv_tile = [&](const BDSmem* __restrict__ rd, const uint8_t* __restrict__ T) {
    bf16x8 av[kDBlocksD];
#pragma unroll
    for (int db = 0; db < kDBlocksD; ++db) {
      const int pc = 8 * wave + 2 * db + ((m16 & 3) >> 1);   // logical piece of this lane's 8 bytes
      const int off = 8 * (m16 & 1);
      const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (__attribute__((address_space(3))) bf16x4*)(T + bf16_pos(v_tok, pc) + off));
      const bf16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (__attribute__((address_space(3))) bf16x4*)(T + bf16_pos(v_tok + 4, pc) + off));
      av[db] = __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    bf16x8 pg[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) pg[g] = rd->pex[g][lane];
#pragma unroll
    for (int db = 0; db < kDBlocksD; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) o[g][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[db], pg[g], o[g][db], 0, 0, 0);
  };

  // pass 0 with R from the first tile; pass 1 (rare) with R = the chunk's largest logit
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int db = 0; db < kDBlocksD; ++db) o[g][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    l_run = 0.f;
    l_rnd = 0.f;
#pragma unroll
    for (int v = 0; v < kRingD - 1; ++v)
      if (v < ntiles) issue(&sm, sm.ring[v], v);

    for (int v = 0; v < ntiles; ++v) {
      wait_tile(min(kRingD - 2, ntiles - 1 - v));
      lds_barrier();   // tile v landed; P and ring slot (v-1) % kRingD are no longer read
      const int nv = v + kRingD - 1 < ntiles ? v + kRingD - 1 : -1;
      uint8_t* dst = sm.ring[(v + kRingD - 1) % kRingD];
      const uint8_t* T = sm.ring[v % kRingD];
      float z[4];
      float tmax = -INFINITY;
      if (s_active) tmax = logits(&sm, v, s_tile(&sm, T, dst, nv), z);
      else if (nv >= 0) issue(&sm, dst, nv);
      if (pass == 0 && v == 0) {
        // the reference: the first tile's largest logit over both token blocks (0 without one)
        if (s_active && grp == 0) sm.m0[tb][hg * 16 + m16] = tmax;
        __syncthreads();
        if (s_active) {
          const float m0 = fmaxf(sm.m0[0][hg * 16 + m16], sm.m0[1][hg * 16 + m16]);
          ref = m0 == -INFINITY ? 0.f : m0;
        }
      }
      if (s_active) {
        m_seen = fmaxf(m_seen, tmax);
        publish(&sm, z);
      }
      lds_barrier();   // P of the tile is published
      pv_tile(&sm, T);
    }
    // does some head's largest logit lie outside R +- 64?
    if (s_active) {
      const float l_blk = lanes4_sum(l_run);   // (all lanes of the wave take part)
      const float r_blk = lanes4_sum(l_rnd);
      if (grp == 0) {
        sm.fin_m[tb][hg * 16 + m16] = m_seen;
        sm.fin_l[tb][hg * 16 + m16] = l_blk;
        sm.fin_r[tb][hg * 16 + m16] = r_blk;
      }
    }
    __syncthreads();
    float mx = -INFINITY;
    if (s_active) {
      mx = fmaxf(sm.fin_m[0][hg * 16 + m16], sm.fin_m[1][hg * 16 + m16]);
      if (mx > -INFINITY && (mx > ref + kRefMargin || mx < ref - kRefMargin)) sm.redo = 1;
    }
    __syncthreads();
    if (pass == 1 || sm.redo == 0) break;
    ref = mx > -INFINITY ? mx : 0.f;
    __syncthreads();
  }

  // ---- output: each wave's 64 values of every head are normalised into the idle tile ring
  // (heads at a padded stride, so the 16 heads of one store fall on different banks), then the
  // workgroup stores whole 2 KiB head rows, 1 KiB per wave instruction.  Written straight from
  // the accumulators, every store would scatter sixteen 64-byte pieces, which took 3.8 us per
  // 128 KiB partial (35 GB/s per compute unit); staged, the partial leaves at the copy rate.
  // (Every wave has passed the barrier after its last read of the ring.)
  float* stage = reinterpret_cast<float*>(&sm.ring[0][0]);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    if (g >= ngroups) break;
    const int head = g * 16 + m16;
    const float mh = fmaxf(sm.fin_m[0][head], sm.fin_m[1][head]);
    const float lh = sm.fin_l[0][head] + sm.fin_l[1][head];
    // R of this head as its S^T waves used it (recomputed from what they published)
    const float m0 = fmaxf(sm.m0[0][head], sm.m0[1][head]);
    const float rh = sm.redo ? (mh > -INFINITY ? mh : 0.f) : (m0 == -INFINITY ? 0.f : m0);
    const float lr = sm.fin_r[0][head] + sm.fin_r[1][head];
    const float inv = lr > 0.f ? 1.f / lr : 0.f;
    if (wave == 0 && grp == 0) {
      if (p.n_split == 1) {
        if (p.lse) p.lse[(int64_t)r * p.H + head] = lh > 0.f ? (rh + log2f(lh)) * kLn2 : -INFINITY;
      } else {
        const int64_t prow = ((int64_t)r * p.n_split + split) * p.H + head;
        p.part_m[prow] = lh > 0.f ? rh * kLn2 : -INFINITY;
        p.part_l[prow] = lh;
      }
    }
#pragma unroll
    for (int db = 0; db < kDBlocksD; ++db)
      *(f32x4*)(stage + head * kStageLd + wave * 64 + db * 16 + grp * 4) = o[g][db] * inv;
  }
  lds_barrier();
  float* dst = p.n_split == 1 ? p.out + (int64_t)r * p.H * kVDim
                              : p.part_o + ((int64_t)r * p.n_split + split) * p.H * kVDim;
  const int n4 = p.H * (kVDim / 4);               // f32x4 pieces of the H rows
  for (int e = threadIdx.x; e < n4; e += kNT) {
    const int head = e >> 7, c = (e & 127) * 4;
    *(f32x4*)(dst + head * kVDim + c) = *(const f32x4*)(stage + head * kStageLd + c);
  }
}

// ---------------------------------------------------------------------------------------------
// bf16 rows, few query rows: one workgroup per (query row, group of 16 heads, chunk of at most
// kChunkN selected rows), 8 waves.  With one or two query rows the 64-head kernel above runs
// few workgroups, each computing every head of its tiles; here the head groups of a chunk run
// on separate compute units (ids 8 apart, so they share one L2 for the chunk's rows), each
// tile's matrix work is a quarter as long, and the partials are per 16 heads.
//   * 128-token tiles: each wave loads the rows of 16 tokens (18 KiB, 1 KiB of consecutive
//     pieces per load) into registers, then stores them into the single LDS tile buffer in the
//     layout of the kernel above (row t at t*1152, piece p in slot p ^ bf16_swz(t)); a skipped
//     slot (-1) reads row 0 and is zeroed on the way in.  The next tile's loads are issued as soon as this one is
//     stored, so they are in flight while it is computed.
//   * q of the 16 heads is read from HBM once per workgroup and passed to the waves through the
//     tile buffer (rows padded to 1168 bytes: conflict-free fragment reads) before the first
//     tile is stored.
//   * S^T: wave w covers 16 tokens of the tile over the full K: row m of its block is token
//     32(w/2) + 8(m/4) + 4(w%2) + m%4, so lane group g of the result holds 4 consecutive tokens,
//     one half of the P^T operand of the 32-token K step w/2 (the other half is wave w^1's).
//   * P.V: wave w owns output values 64w .. 64w+63 of the 16 heads, four K steps per tile, V^T
//     from the transposing LDS reads.
//   * Softmax against a fixed per-head reference (the first tile's largest logit), with the
//     second pass of the kernels above when a head's logits leave R +- 64.

constexpr int kNTN = 512;                                 // threads per workgroup (8 waves)
constexpr int kTN = 128;                                  // tokens per tile
constexpr int kChunkN = 512;                              // selected rows per workgroup at most
constexpr int kTNBytes = kTN * kRowDim * 2;               // 147456
constexpr int kTNLoads = kTNBytes / 1024 / 8;             // 18 loads of 1 KiB per wave and tile
constexpr int kKStepsN = kTN / 32;                        // 4 K steps of P.V per tile
constexpr int kQPitchN = kRowDim * 2 + 16;                // bytes per staged q row
constexpr int kFewHeadRows = 16;                          // rows x head groups served by this kernel
static_assert(16 * kQPitchN <= kTNBytes, "q is staged in the tile buffer");

struct NSmem {
  uint8_t tile[kTNBytes];                     // the tile (q of the head group before the first)
  bf16x8 pex[kKStepsN][64];                   // P^T operands of the tile's K steps
  int32_t sl[kChunkN];                        // the chunk's slots, -1 past the chunk
  float m0[8][16];                            // largest logit of the first tile, by wave
  float fin_m[8][16], fin_l[8][16], fin_r[8][16];   // per wave and head, after the last tile
};

__global__ __launch_bounds__(kNTN) void mla_bf16n_kernel(MlaParams p) {
  __shared__ __attribute__((aligned(16))) NSmem sm;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ks = wave >> 1, half = wave & 1;
  const int m16 = lane & 15, grp = lane >> 4;
  const int ng = p.H / 16;
  // block b: chunk index rs = 8 * ((b / 8) / ng) + b % 8 (row rs / n_split), head group (b / 8) % ng
  const int xq = blockIdx.x & 7, yq = blockIdx.x >> 3;
  const int hg = yq % ng;
  const int rs = 8 * (yq / ng) + xq;
  if (rs >= p.rows * p.n_split) return;          // grid padding (uniform)
  const int r = rs / p.n_split, split = rs - r * p.n_split;
  const int j0 = split * p.chunk;
  const int j1 = min(p.k, j0 + p.chunk);
  const int ntiles = j1 > j0 ? (j1 - j0 + kTN - 1) / kTN : 0;
  const int32_t* sl = p.slots + (int64_t)r * p.k;

  // the chunk's slots (one per thread), then q of the head group into the tile buffer
  static_assert(kChunkN <= kNTN, "one round of slot loads");
  const int32_t slv = sl[min(j0 + (int)threadIdx.x, p.k - 1)];
  __builtin_amdgcn_sched_barrier(0);
  constexpr int kQPieces = 16 * (kRowDim * 2 / 16);       // 1152 pieces of 16 bytes
  u32x4 qv[3];
  const uint8_t* qbase = (const uint8_t*)p.q + ((int64_t)r * p.H + 16 * hg) * (kRowDim * 2);
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    const int e = min(c * kNTN + (int)threadIdx.x, kQPieces - 1);
    qv[c] = *(const u32x4*)(qbase + 16 * e);
  }
  if ((int)threadIdx.x < ntiles * kTN)
    sm.sl[threadIdx.x] = j0 + (int)threadIdx.x < j1 ? dbg_slot(p.dbg, slv, p.num_slots) : -1;
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    const int e = c * kNTN + (int)threadIdx.x;
    if (e < kQPieces) {
      const int h = e / 72, pc = e - h * 72;
      *(u32x4*)(sm.tile + h * kQPitchN + 16 * pc) = qv[c];
    }
  }
  lds_barrier();
  bf16x8 qf[kStepsD];   // S^T B operand: head 16hg + m16, dims 32s + 8grp .. +8

  // tile loads: wave w gathers the rows of tokens 16w .. 16w+15, 1152 pieces of 16 bytes in row
  // order (piece P: row P / 72, piece P % 72); load c, lane i takes piece 64c + i, so each load
  // reads 1 KiB of at most two rows (r0 = 64c / 72 and r0 + 1) and each store writes 1 KiB of
  // LDS with no bank conflict.  The two rows' slots are wave-uniform (read lanes of sv16).
  const uint8_t* kvb = (const uint8_t*)p.kv;
  u32x4 st[kTNLoads];
  uint32_t dead = 0;
  auto load_tile = [&](const NSmem* __restrict__ rd, int v) {
    const int32_t sv16 = rd->sl[v * kTN + 16 * wave + (lane & 15)];
    int ln = lane;
    asm volatile("" : "+v"(ln));   // (keeps the per-load lane arithmetic inside the tile loop)
    dead = 0;
#pragma unroll
    for (int c = 0; c < kTNLoads; ++c) {
      const int r0 = 64 * c / 72, r1 = r0 < 15 ? r0 + 1 : 15;
      const int kb = 72 * (r0 + 1) - 64 * c;        // lanes below kb are in row r0
      const int sa = __builtin_amdgcn_readlane(sv16, r0), sb = __builtin_amdgcn_readlane(sv16, r1);
      const bool lo = ln < kb;
      const int sv = lo ? sa : sb;
      const int pc = ln + (lo ? 64 * c - 72 * r0 : 64 * c - 72 * (r0 + 1));
      dead |= (sv < 0 ? 1u : 0u) << c;
      st[c] = *(const u32x4*)(kvb + (int64_t)max(sv, 0) * (kRowDim * 2) + 16 * pc);
    }
  };
  auto store_tile = [&](NSmem* __restrict__ rd) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int c = 0; c < kTNLoads; ++c) {
      const int r0 = 64 * c / 72;
      const int kb = 72 * (r0 + 1) - 64 * c;
      const bool lo = ln < kb;
      const int t = 16 * wave + (lo ? r0 : r0 + 1);
      const int pc = ln + (lo ? 64 * c - 72 * r0 : 64 * c - 72 * (r0 + 1));
      *(u32x4*)(rd->tile + bf16_pos(t, pc)) = ((dead >> c) & 1u) ? u32x4{0u, 0u, 0u, 0u} : st[c];
    }
  };

  f32x4 o[kDBlocksD];         // lane: O^T[64w + 16db + 4grp + j][head m16]
  const float scale2 = p.sm_scale * kLog2e;
  // l_run: sum of P (for lse and the chunk weight); l_rnd: sum of P as rounded to bf16 for P.V,
  // the normaliser of the output, so that it is an exact convex combination of the V rows
  float ref = 0.f, m_seen = -INFINITY, l_run = 0.f, l_rnd = 0.f;
  const int a_tok = 32 * ks + 8 * (m16 >> 2) + 4 * half + (m16 & 3);
  const int v_tok = 8 * grp + (m16 >> 2);

  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int db = 0; db < kDBlocksD; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    l_run = 0.f;
    l_rnd = 0.f;
    if (ntiles > 0) load_tile(&sm, 0);
    if (pass == 0) {
      // q out of the tile buffer while the first tile's loads are in flight
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < kStepsD; ++s) qf[s] = *(const bf16x8*)(sm.tile + m16 * kQPitchN + 16 * (4 * s + grp));
      lds_barrier();   // every wave has read q
    }
    for (int v = 0; v < ntiles; ++v) {
      wait_vmcnt<0>();
      store_tile(&sm);
      if (v + 1 < ntiles) load_tile(&sm, v + 1);
      lds_barrier();   // tile v stored
      const uint8_t* T = sm.tile;
      // S^T of this wave's 16 tokens
      f32x4 acc0 = f32x4{0.f, 0.f, 0.f, 0.f}, acc1 = f32x4{0.f, 0.f, 0.f, 0.f};
      {
        constexpr int kAhead = 4;
        bf16x8 a[kAhead];
#pragma unroll
        for (int s = 0; s < kAhead; ++s) a[s] = *(const bf16x8*)(T + bf16_pos(a_tok, 4 * s + grp));
#pragma unroll
        for (int s = 0; s < kStepsD; ++s) {
          const bf16x8 x = a[s % kAhead];
          if (s + kAhead < kStepsD) a[s % kAhead] = *(const bf16x8*)(T + bf16_pos(a_tok, 4 * (s + kAhead) + grp));
          if (s & 1) acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, qf[s], acc1, 0, 0, 0);
          else acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, qf[s], acc0, 0, 0, 0);
        }
      }
      const f32x4 sacc = acc0 + acc1;
      // lane: head 16hg + m16, tokens 32ks + 8grp + 4half + j
      float z[4];
      float tmax = -INFINITY;
      {
        const int32_t* slt = sm.sl + v * kTN + 32 * ks + 8 * grp + 4 * half;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          z[j] = slt[j] >= 0 ? sacc[j] * scale2 : -INFINITY;
          tmax = fmaxf(tmax, z[j]);
        }
        tmax = lanes4_max(tmax);
      }
      if (pass == 0 && v == 0) {
        // the reference: the first tile's largest logit of the head (0 without a live token)
        if (grp == 0) sm.m0[wave][m16] = tmax;
        lds_barrier();   // (the next tile's loads stay in flight)
        float m0 = -INFINITY;
#pragma unroll
        for (int w = 0; w < 8; ++w) m0 = fmaxf(m0, sm.m0[w][m16]);
        ref = m0 == -INFINITY ? 0.f : m0;
      }
      m_seen = fmaxf(m_seen, tmax);
      {
        bf16x4 pb;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float pe = z[j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(z[j] - ref);
          l_run += pe;
          pb[j] = (__bf16)pe;
          l_rnd += (float)pb[j];
        }
        *(bf16x4*)((uint8_t*)&sm.pex[ks][lane] + 8 * half) = pb;
      }
      lds_barrier();   // P of the tile is published
#pragma unroll
      for (int kk = 0; kk < kKStepsN; ++kk) {
        const bf16x8 pg = sm.pex[kk][lane];
#pragma unroll
        for (int db = 0; db < kDBlocksD; ++db) {
          const int pc = 8 * wave + 2 * db + ((m16 & 3) >> 1);
          const int off = 8 * (m16 & 1);
          const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (__attribute__((address_space(3))) bf16x4*)(T + bf16_pos(32 * kk + v_tok, pc) + off));
          const bf16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (__attribute__((address_space(3))) bf16x4*)(T + bf16_pos(32 * kk + v_tok + 4, pc) + off));
          o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7),
                                                          pg, o[db], 0, 0, 0);
        }
      }
      if (v + 1 < ntiles) lds_barrier();   // every wave is done with the tile and P
    }
    // does some head's largest logit lie outside R +- 64?
    {
      const float l_blk = lanes4_sum(l_run), r_blk = lanes4_sum(l_rnd);
      if (grp == 0) {
        sm.fin_m[wave][m16] = m_seen;
        sm.fin_l[wave][m16] = l_blk;
        sm.fin_r[wave][m16] = r_blk;
      }
    }
    lds_barrier();
    // every wave reaches the same answer: its lanes cover the 16 heads
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < 8; ++w) mx = fmaxf(mx, sm.fin_m[w][m16]);
    const bool wide = mx > -INFINITY && (mx > ref + kRefMargin || mx < ref - kRefMargin);
    if (pass == 1 || __builtin_amdgcn_ballot_w64(wide) == 0) break;
    ref = mx > -INFINITY ? mx : 0.f;
  }

  // output: lane holds values 64w + 16db + 4grp .. +3 of head 16hg + m16
  const int head = 16 * hg + m16;
  float lh = 0.f, rh = 0.f;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    lh += sm.fin_l[w][m16];
    rh += sm.fin_r[w][m16];
  }
  const float inv = rh > 0.f ? 1.f / rh : 0.f;
  // R as the S^T waves used it: ref (pass 0, or the chunk maximum after a second pass)
  if (wave == 0 && grp == 0) {
    if (p.n_split == 1) {
      if (p.lse) p.lse[(int64_t)r * p.H + head] = lh > 0.f ? (ref + log2f(lh)) * kLn2 : -INFINITY;
    } else {
      const int64_t prow = ((int64_t)r * p.n_split + split) * p.H + head;
      p.part_m[prow] = lh > 0.f ? ref * kLn2 : -INFINITY;
      p.part_l[prow] = lh;
    }
  }
  float* dst = p.n_split == 1 ? p.out + ((int64_t)r * p.H + head) * kVDim
                              : p.part_o + (((int64_t)r * p.n_split + split) * p.H + head) * kVDim;
#pragma unroll
  for (int db = 0; db < kDBlocksD; ++db) *(f32x4*)(dst + 64 * wave + 16 * db + 4 * grp) = o[db] * inv;
}

// ---------------------------------------------------------------------------------------------
// split-k merge.  One 128-thread workgroup per (row, head, 128-value quarter of the output).
// Thread (g, q) merges chunks j = g, g+4, g+8, ... for output values 4q..4q+3 of the quarter: it
// issues the loads of m_j, l_j and o_j for up to 8 chunks at once, keeps a running
// (max, denominator, weighted sum) in fixed j order, and the 4 groups are merged in LDS in a
// fixed order, so the result does not depend on scheduling.  Chunks with l_j = 0 (no live slot)
// are skipped; if none is live the output is 0 and lse = -inf.

constexpr int kCombGroups = 4;
constexpr int kCombBatch = 8;

__device__ __forceinline__ void lse_merge(float& M, float& den, f32x4& acc, float m2, float den2, const f32x4& acc2) {
  // merges (m2, den2, acc2) into (M, den, acc): both are sums scaled by exp(-max)
  if (den2 <= 0.f) return;
  if (den <= 0.f) {
    M = m2;
    den = den2;
    acc = acc2;
    return;
  }
  const float Mn = fmaxf(M, m2);
  const float a = expf(M - Mn), b = expf(m2 - Mn);
  den = den * a + den2 * b;
  acc = acc * a + acc2 * b;
  M = Mn;
}

__global__ __launch_bounds__(128) void mla_combine_kernel(CombineParams p) {
  __shared__ float s_m[kCombGroups][32], s_d[kCombGroups][32];
  __shared__ f32x4 s_a[kCombGroups][32];
  const int dq = blockIdx.x & 3;
  const int rh = blockIdx.x >> 2;
  const int r = rh / p.H, h = rh - (rh / p.H) * p.H;
  const int tid = threadIdx.x;
  const int g = tid >> 5, q = tid & 31;
  const int ns = p.n_split;
  const int64_t base = (int64_t)r * ns * p.H + h;  // partial row of chunk j: base + j * H
  const int col = dq * 128 + q * 4;

  float M = -INFINITY, den = 0.f;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int j0 = g; j0 < ns; j0 += kCombBatch * kCombGroups) {
    float mv[kCombBatch], lv[kCombBatch];
    f32x4 ov[kCombBatch];
#pragma unroll
    for (int u = 0; u < kCombBatch; ++u) {
      const int64_t pr = base + (int64_t)min(j0 + u * kCombGroups, ns - 1) * p.H;
      mv[u] = p.part_m[pr];
      lv[u] = p.part_l[pr];
      ov[u] = *(const f32x4*)(p.part_o + pr * kVDim + col);
    }
#pragma unroll
    for (int u = 0; u < kCombBatch; ++u) {
      const bool live = j0 + u * kCombGroups < ns && lv[u] > 0.f;
      // o_j is normalised by l_j: its weight in the merged sum is l_j exp(m_j - M)
      if (live) lse_merge(M, den, acc, mv[u], lv[u], ov[u] * lv[u]);
    }
  }
  s_m[g][q] = M;
  s_d[g][q] = den;
  s_a[g][q] = acc;
  __syncthreads();
  if (g == 0) {
#pragma unroll
    for (int gg = 1; gg < kCombGroups; ++gg) lse_merge(M, den, acc, s_m[gg][q], s_d[gg][q], s_a[gg][q]);
    float* dst = p.out + ((int64_t)r * p.H + h) * kVDim + col;
    const bool live = den > 0.f;
    *(f32x4*)dst = live ? acc * (1.f / den) : f32x4{0.f, 0.f, 0.f, 0.f};
    if (p.lse && dq == 0 && q == 0) p.lse[(int64_t)r * p.H + h] = live ? M + logf(den) : -INFINITY;
  }
}

// Few chunks (n_split <= kFewSplits): one 256-thread workgroup per (row, two heads); thread
// (head e, quad q) merges all chunks of output values 4q..4q+3 of its head, in chunk order,
// with every chunk's loads issued at once.  (Measured: 128 rows x 2 chunks merge in 8.4 us
// against 16.4 us with the quarter-row workgroups above, whose 32K launches of 128 threads
// cost more than the loads; at 8 chunks the quarter-row kernel stays faster, 11.0 against
// 13.0 us for 32 rows.)
constexpr int kFewSplits = 4;

__global__ __launch_bounds__(256) void mla_combine_few_kernel(CombineParams p) {
  const int tid = threadIdx.x;
  const int e = tid >> 7, q = tid & 127;
  const int hp = p.H >> 1;                          // head pairs per row (H is even)
  const int r = blockIdx.x / hp, h = 2 * (blockIdx.x - r * hp) + e;
  const int ns = p.n_split;
  const int64_t base = (int64_t)r * ns * p.H + h;  // partial row of chunk j: base + j * H
  float mv[kFewSplits], lv[kFewSplits];
  f32x4 ov[kFewSplits];
#pragma unroll
  for (int j = 0; j < kFewSplits; ++j) {
    lv[j] = 0.f;
    if (j < ns) {   // (uniform)
      const int64_t pr = base + (int64_t)j * p.H;
      mv[j] = p.part_m[pr];
      lv[j] = p.part_l[pr];
      ov[j] = *(const f32x4*)(p.part_o + pr * kVDim + 4 * q);
    }
  }
  float M = -INFINITY, den = 0.f;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kFewSplits; ++j)
    if (lv[j] > 0.f) lse_merge(M, den, acc, mv[j], lv[j], ov[j] * lv[j]);
  float* dst = p.out + ((int64_t)r * p.H + h) * kVDim + 4 * q;
  const bool live = den > 0.f;
  *(f32x4*)dst = live ? acc * (1.f / den) : f32x4{0.f, 0.f, 0.f, 0.f};
  if (p.lse && q == 0) p.lse[(int64_t)r * p.H + h] = live ? M + logf(den) : -INFINITY;
}

}  // namespace

bool mla_uses_narrow(int rows, int H, dsa_dtype_t kv_dtype) {
  return kv_dtype == DSA_BF16 && H % 16 == 0 && H <= 64 && (int64_t)rows * (H / 16) <= kFewHeadRows;
}

int mla_default_split(int rows, int H, int k, dsa_dtype_t kv_dtype) {
  if (mla_uses_narrow(rows, H, kv_dtype)) {
    // one 128-token tile per chunk, at most about one workgroup per compute unit
    const int per = rows * (H / 16);
    const int cap = per > 0 ? std::max(1, 256 / per) : 1;
    return std::max(1, std::min((k + kTN - 1) / kTN, cap));
  }
  // about one workgroup per compute unit, at least 64 selected rows per chunk, and for fp8 rows
  // at most kChunkF (the fp8 ring kernel's staging limit)
  int ns = 256 / (rows > 0 ? rows : 1);
  const int max_ns = (k + 63) / 64;
  if (ns > max_ns) ns = max_ns;
  const int min_ns = kv_dtype == DSA_FP8_E4M3FN ? (k + kChunkF - 1) / kChunkF : 1;
  if (ns < min_ns) ns = min_ns;
  if (ns < 1) ns = 1;
  return ns;
}

hipError_t launch_mla(const MlaParams& p0, dsa_dtype_t q_dtype, dsa_dtype_t kv_dtype, hipStream_t s) {
  MlaParams p = p0;
  if (q_dtype == DSA_F32) {
    p.n_split = 1;
    const dim3 grid((unsigned)p.rows, (unsigned)p.H);
    const size_t shm = (size_t)(kRowDim + p.k) * sizeof(float);
    if (kv_dtype == DSA_F32) hipLaunchKernelGGL(mla_valu_kernel<float>, grid, dim3(256), shm, s, p);
    else if (kv_dtype == DSA_BF16) hipLaunchKernelGGL(mla_valu_kernel<__bf16>, grid, dim3(256), shm, s, p);
    else hipLaunchKernelGGL(mla_valu_kernel<Fp8Row>, grid, dim3(256), shm, s, p);
    return hipGetLastError();
  }
  int chunk = (p.k + p.n_split - 1) / p.n_split;
  chunk = (chunk + kTT - 1) / kTT * kTT;
  p.chunk = chunk;
  if (p.group < 1 || p.rows % p.group != 0) p.group = 1;
  const dim3 grid((unsigned)p.n_split, (unsigned)p.rows);
  // XCD-mapped launches: the row groups rounded up to a multiple of 8, times group and n_split
  const unsigned xgrid = (unsigned)((p.rows >= 8 ? (p.rows / p.group + 7) / 8 * 8 * p.group : p.rows) * p.n_split);
  if (kv_dtype == DSA_FP8_E4M3FN) {
    if (chunk <= kChunkF)
      hipLaunchKernelGGL(mla_fp8d_kernel, dim3(xgrid), dim3(kNTF), 0, s, p);
    else hipLaunchKernelGGL(mla_fp8_kernel, grid, dim3(kNT), 0, s, p);
  }
  else if (mla_uses_narrow(p.rows, p.H, kv_dtype) && chunk <= kChunkN) {
    const int64_t rs = (int64_t)p.rows * p.n_split;
    hipLaunchKernelGGL(mla_bf16n_kernel, dim3((unsigned)((rs + 7) / 8 * 8 * (p.H / 16))), dim3(kNTN), 0, s, p);
  } else if (chunk <= kChunkD)
    hipLaunchKernelGGL(mla_bf16d_kernel, dim3(xgrid), dim3(kNT), 0, s, p);
  else hipLaunchKernelGGL(mla_mfma_kernel<false>, grid, dim3(kNT), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_split == 1) return e;
  CombineParams c{p.part_o, p.part_m, p.part_l, p.out, p.lse, p.rows, p.H, p.n_split};
  return launch_combine(c, s);
}

hipError_t launch_combine(const CombineParams& c, hipStream_t s) {
  if (c.rows == 0) return hipSuccess;
  if (c.n_split <= kFewSplits && c.H % 2 == 0)
    hipLaunchKernelGGL(mla_combine_few_kernel, dim3((unsigned)(c.rows * (c.H / 2))), dim3(256), 0, s, c);
  else
    hipLaunchKernelGGL(mla_combine_kernel, dim3((unsigned)(c.rows * c.H * 4)), dim3(128), 0, s, c);
  return hipGetLastError();
}

}  // namespace dsa
