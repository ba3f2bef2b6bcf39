// Latent up-projection after attention (the step after the sparse MLA decode): with MLA weight
// absorption the query has absorbed kv_b, so the attention output is still in the 512-wide latent
// space and is projected afterwards, per head by that head's value block of kv_b (W_UV), then by
// o_proj (W_O) (Show HN page "Chay GLM 5.2 tren may tinh cham", main-features section, MLA weight
// absorption bullet).
//
//   v[r, h, j] = sum_d W_UV[h, j, d] * o[r, h, d]          (d over the 512 latent values)
//   y[r, m]    = sum_{h, j} W_O[m, h*Dv + j] * v[r, h, j]
//
// Both are products C[r, n] = sum_k A[r, k] * B[n, k] with f32 activations A and bf16 weights B
// (B row n contiguous along k), run by one tiled kernel, up_gemm_kernel, on
// v_mfma_f32_16x16x32_bf16.  The activations enter the matrix core as two bf16 parts,
// hi = bf16(a) and lo = bf16(a - hi), so a = hi + lo to 2^-18 relative and each product is exact
// in the fp32 accumulator: the result is an fp32-accurate projection.
//   * A workgroup (4 waves) owns a tile of up to 128 rows x 128 columns (x 256 when there are
//     many rows) and a range of k.  Each 128-wide (64-wide) chunk of k of the tile's activations
//     is loaded once, split into its two bf16 parts and stored in LDS (rows padded by 16 bytes,
//     so the operand reads are free of bank conflicts); wave w reads the weights of its 32 (64)
//     columns into registers, with tiles of up to 64 rows as 1 KiB runs that it turns around
//     through its own LDS area into the operand layout.
//     Weights are therefore read once per row tile (once in decode, where the rows are few), and
//     the next chunk's loads are in flight while the current one is multiplied.
//   * v: one group of tiles per head (A = o[:, h, :], B = W_UV[h], K = 512).  y: K = H * Dv is
//     split over workgroups when the tiles alone would not fill the GPU; up_reduce_kernel adds
//     the partial sums in split order, so the result is deterministic.
// One or two rows take up_gemv_kernel instead (below): matrix-vector products on the vector ALU.
#include "dsa_internal.hpp"

namespace dsa {

namespace {

constexpr int kGT = 256;              // threads per workgroup (4 waves)

// C[g][split][r][n] = sum over k in the split's range of A[g][r][k] * B[g][n][k]
struct GemmArgs {
  const float* A;
  int64_t lda, a_gs;                  // row r of group g: A + g*a_gs + r*lda
  const __bf16* B;
  int64_t ldb, b_gs;                  // column n of group g: B + g*b_gs + n*ldb
  float* C;
  int64_t ldc, c_gs, c_ks;            // C + g*c_gs + split*c_ks + r*ldc + n
  int32_t R, N, K, k_chunk, ksplit;
};

// RB blocks of 16 rows per tile (1, 2, 4 or 8), CB blocks of 16 columns per wave (2 or 4), KC
// contraction values per staged chunk (64 or 128)
template <int RB, int CB, int KC>
__global__ __launch_bounds__(kGT) void up_gemm_kernel(GemmArgs g) {
  constexpr int kGN = 4 * 16 * CB;    // columns per tile
  constexpr int kPitch = KC + 8;      // bf16 per staged row (144 or 272 bytes: conflict-free reads)
  constexpr int kS = KC / 32;         // k steps per chunk
  constexpr int kF4 = KC / 4;         // float4 per staged row
  __shared__ __attribute__((aligned(16))) __bf16 as[2][2][RB * 16][kPitch];   // [buffer][hi, lo][row][k]
  // Tiles of up to 64 rows (where the weight stream sets the time): weights go HBM -> registers
  // with 1 KiB loads of consecutive 16-byte pieces (whole column runs of the chunk), then turn
  // around in a per-wave LDS area into the operand layout (one row: 42.8 -> 29.6 us).  128-row
  // tiles load the operand layout directly (64 bytes of 16 columns per load), as the LDS
  // traffic of the turnaround costs more than the coalescing gains there.
  constexpr bool kTT = RB <= 4;
  constexpr int kPPC = KC / 8;                       // 16-byte pieces of a column in one chunk
  constexpr int kWL = CB * 16 * kPPC / 64;           // 1 KiB loads per wave and chunk
  constexpr int kColsPer256 = 16 / kPPC;             // columns in 256 bytes of the area
  __shared__ __attribute__((aligned(16))) uint8_t wt[kTT ? 4 : 1][kTT ? CB * 16 * KC * 2 : 16];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n16 = lane & 15, grp = lane >> 4;
  const int col0 = blockIdx.x * kGN;
  const int row0 = blockIdx.y * (RB * 16);
  const int gz = blockIdx.z / g.ksplit, split = blockIdx.z - gz * g.ksplit;
  const int k0 = split * g.k_chunk, k1 = min(g.K, k0 + g.k_chunk);   // k1 > k0 (host), both multiples of 32
  const int nrows = min(RB * 16, g.R - row0);
  const int nch = (k1 - k0 + KC - 1) / KC;
  const float* A = g.A + gz * g.a_gs + (int64_t)row0 * g.lda;
  const __bf16* B = g.B + gz * g.b_gs;

  // activations of chunk c: float4 e = j*256 + thread is row e / kF4, values 4(e % kF4) .. +4;
  // rows past the tile and values past the range read a valid address and are replaced by 0
  constexpr int kAL = RB * 16 * kF4 / kGT;
  f32x4 ar[kAL];
  auto load_a = [&](int c) {
    const int kb = k0 + c * KC;
#pragma unroll
    for (int j = 0; j < kAL; ++j) {
      const int e = j * kGT + threadIdx.x;
      const int r = e / kF4, k = kb + 4 * (e % kF4);
      const f32x4 x = *(const f32x4*)(A + (int64_t)min(r, nrows - 1) * g.lda + min(k, k1 - 4));
      ar[j] = (r < nrows && k < k1) ? x : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int j = 0; j < kAL; ++j) {
      const int e = j * kGT + threadIdx.x;
      const int r = e / kF4, kk = 4 * (e % kF4);
      bf16x4 hi, lo;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const __bf16 h = (__bf16)ar[j][i];
        hi[i] = h;
        lo[i] = (__bf16)(ar[j][i] - (float)h);
      }
      *(bf16x4*)&as[buf][0][r][kk] = hi;
      *(bf16x4*)&as[buf][1][r][kk] = lo;
    }
  };
  // turned-around layout: column c of the wave at c * 2KC bytes, its piece q in slot
  // q ^ ((c / kColsPer256) % kPPC), so that the 16 columns of one operand read fall on distinct
  // banks and each 1 KiB store is a permutation of a contiguous KiB
  auto wt_off = [](int c, int q) { return c * (2 * KC) + ((q ^ ((c / kColsPer256) & (kPPC - 1))) << 4); };
  // chunk c's weights of this wave: load j, lane i takes piece 64j + i of the wave's columns in
  // column order (column (64j + i) / kPPC, values 8 * ((64j + i) % kPPC) .. +8; 0 past the range)
  auto load_raw = [&](u32x4 (&raw)[kWL], int c) {
    const int kb = k0 + c * KC;
#pragma unroll
    for (int j = 0; j < kWL; ++j) {
      const int pc = 64 * j + lane;
      const int cl = pc / kPPC, q = pc - cl * kPPC;
      const int n = min(col0 + 16 * CB * wave + cl, g.N - 1);
      const int k = kb + 8 * q;
      const u32x4 x = *(const u32x4*)(B + (int64_t)n * g.ldb + min(k, k1 - 8));
      raw[j] = k < k1 ? x : u32x4{0u, 0u, 0u, 0u};
    }
  };
  // weights of chunk c for this wave's CB column blocks: lane (n16, grp) of block cb, k step s
  // reads column col0 + 16(CB w + cb) + n16, values kb + 32s + 8grp .. +8 (0 past the range)
  auto load_b = [&](bf16x8 (&bb)[CB][kS], int c) {
    const int kb = k0 + c * KC;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int n = min(col0 + 16 * (CB * wave + cb) + n16, g.N - 1);
#pragma unroll
      for (int s = 0; s < kS; ++s) {
        const int k = kb + 32 * s + 8 * grp;
        const bf16x8 x = *(const bf16x8*)(B + (int64_t)n * g.ldb + min(k, k1 - 8));
        bb[cb][s] = k < k1 ? x : bf16x8{};
      }
    }
  };

  f32x4 acc[RB][CB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // lane (n16, grp) supplies row 16rb + n16, values 32s + 8grp .. +8 of both parts
  auto compute = [&](int buf, const bf16x8 (&bb)[CB][kS]) {
#pragma unroll
    for (int s = 0; s < kS; ++s)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const bf16x8 ah = *(const bf16x8*)&as[buf][0][16 * rb + n16][32 * s + 8 * grp];
        const bf16x8 al = *(const bf16x8*)&as[buf][1][16 * rb + n16][32 * s + 8 * grp];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bb[cb][s], acc[rb][cb], 0, 0, 0);
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bb[cb][s], acc[rb][cb], 0, 0, 0);
        }
      }
  };

  if constexpr (kTT) {
    // the wave's weights through its LDS area (a wave's LDS accesses complete in order: no
    // barrier), then the same MFMAs with the operands read per k step
    uint8_t* my = wt[kTT ? wave : 0];
    auto compute_tt = [&](int buf, const u32x4 (&raw)[kWL]) {
#pragma unroll
      for (int j = 0; j < kWL; ++j) {
        const int pc = 64 * j + lane;
        const int cl = pc / kPPC, q = pc - cl * kPPC;
        *(u32x4*)(my + wt_off(cl, q)) = raw[j];
      }
#pragma unroll
      for (int s = 0; s < kS; ++s) {
        bf16x8 bb[CB];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) bb[cb] = *(const bf16x8*)(my + wt_off(16 * cb + n16, 4 * s + grp));
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const bf16x8 ah = *(const bf16x8*)&as[buf][0][16 * rb + n16][32 * s + 8 * grp];
          const bf16x8 al = *(const bf16x8*)&as[buf][1][16 * rb + n16][32 * s + 8 * grp];
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bb[cb], acc[rb][cb], 0, 0, 0);
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bb[cb], acc[rb][cb], 0, 0, 0);
          }
        }
      }
    };
    u32x4 rx[kWL], ry[kWL];
    load_a(0);
    load_raw(rx, 0);
    store_a(0);
    lds_barrier();
    for (int c = 0; c < nch; c += 2) {
      load_a(min(c + 1, nch - 1));
      load_raw(ry, min(c + 1, nch - 1));
      compute_tt(0, rx);
      store_a(1);
      lds_barrier();   // chunk c + 1 staged; buffer 0 is no longer read
      load_a(min(c + 2, nch - 1));
      load_raw(rx, min(c + 2, nch - 1));
      if (c + 1 < nch) compute_tt(1, ry);
      store_a(0);
      lds_barrier();   // chunk c + 2 staged; buffer 1 is no longer read
    }
  } else {
    // two chunks per loop trip, so that the two weight buffers keep their registers; every step
    // issues the same loads (the chunk index is clamped past the end)
    bf16x8 bx[CB][kS], by[CB][kS];
    load_a(0);
    load_b(bx, 0);
    store_a(0);
    lds_barrier();
    for (int c = 0; c < nch; c += 2) {
      load_a(min(c + 1, nch - 1));
      load_b(by, min(c + 1, nch - 1));
      compute(0, bx);
      store_a(1);
      lds_barrier();   // chunk c + 1 staged; buffer 0 is no longer read
      load_a(min(c + 2, nch - 1));
      load_b(bx, min(c + 2, nch - 1));
      if (c + 1 < nch) compute(1, by);
      store_a(0);
      lds_barrier();   // chunk c + 2 staged; buffer 1 is no longer read
    }
  }

  // lane (n16, grp) holds C[16rb + 4grp + j][16(CB w + cb) + n16]
  float* C = g.C + gz * g.c_gs + split * g.c_ks;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int n = col0 + 16 * (CB * wave + cb) + n16;
    if (n >= g.N) continue;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * rb + 4 * grp + j;
        if (r < nrows) C[(int64_t)(row0 + r) * g.ldc + n] = acc[rb][cb][j];
      }
  }
}

// One or two rows (decode): C[g][r][n] = sum_k A[g][r][k] * B[g][n][k] as a matrix-vector product
// on the vector ALU, where the matrix core would compute 16 rows for every one used and only the
// weight stream matters.  A workgroup (8 waves) stages its group's RR activation rows in LDS and
// owns 8 columns, one per wave; lane l of a wave reads the 16-byte pieces 64i + l of its column's
// weights (all K / 512 of them requested at once, whole 1 KiB runs per load instruction) and
// accumulates their 8 products with the matching activations in fp32 (each fma rounds once),
// then the wave adds its lanes' sums.  K = 512 NI with NI a power of two up to 16.
template <int RR, int NI>
__global__ __launch_bounds__(512) void up_gemv_kernel(GemmArgs g) {
  constexpr int K = 512 * NI;
  __shared__ __attribute__((aligned(16))) float as[RR * K];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int gz = blockIdx.y;
  const float* A = g.A + gz * g.a_gs;
  for (int e = threadIdx.x; e < RR * K / 4; e += 512) {
    const int r = e / (K / 4), c = e - r * (K / 4);
    *(f32x4*)&as[r * K + 4 * c] = r < g.R ? *(const f32x4*)(A + r * g.lda + 4 * c) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int n = blockIdx.x * 8 + wave;
  const bool live = n < g.N;
  const __bf16* Bn = g.B + gz * g.b_gs + (int64_t)(live ? n : 0) * g.ldb;
  u32x4 w[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) w[i] = __builtin_nontemporal_load((const u32x4*)(Bn + 512 * i + 8 * lane));
  __syncthreads();
  float acc[RR];
#pragma unroll
  for (int r = 0; r < RR; ++r) acc[r] = 0.f;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const bf16x8 wb = __builtin_bit_cast(bf16x8, w[i]);
#pragma unroll
    for (int r = 0; r < RR; ++r) {
      const f32x4 a0 = *(const f32x4*)&as[r * K + 512 * i + 8 * lane];
      const f32x4 a1 = *(const f32x4*)&as[r * K + 512 * i + 8 * lane + 4];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[r] = fmaf((float)wb[j], a0[j], acc[r]);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[r] = fmaf((float)wb[4 + j], a1[j], acc[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < RR; ++r) {
    float v = acc[r];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    if (lane == 0 && live && r < g.R) g.C[gz * g.c_gs + (int64_t)r * g.ldc + n] = v;
  }
}

// y = sum over the K splits of the partial sums, in split order.
__global__ __launch_bounds__(256) void up_reduce_kernel(UpProjParams p) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)p.R * p.Dm;
  if (e >= total) return;
  float s = 0.f;
  for (int ks = 0; ks < p.ksplit; ++ks) s += p.part[(int64_t)ks * total + e];
  p.y[e] = s;
}

// rows per tile in blocks of 16: up to 128 rows in tiles of at most 64 (whose weights take the
// LDS turnaround; 128 rows: 88.8 -> 84.6 us although the weights are read by two tiles)
int rows_per_tile_blocks(int R) { return R <= 16 ? 1 : R <= 32 ? 2 : R <= 128 ? 4 : 8; }
// column blocks per wave: with at least two rounds of 128 x 256 tiles (many rows), 64 columns
// per wave, so that each activation operand read from LDS feeds twice the matrix work;
// otherwise 32, which keeps more workgroups in flight
int col_blocks_per_wave(int R, int N) {
  return (int64_t)((N + 255) / 256) * ((R + 127) / 128) >= 512 ? 4 : 2;
}

template <int RB, int CB, int KC>
hipError_t launch_gemm_t(const GemmArgs& a, int groups, hipStream_t s) {
  const dim3 grid((unsigned)((a.N + 64 * CB - 1) / (64 * CB)), (unsigned)((a.R + RB * 16 - 1) / (RB * 16)),
                  (unsigned)(groups * a.ksplit));
  hipLaunchKernelGGL((up_gemm_kernel<RB, CB, KC>), grid, dim3(kGT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& a, int groups, hipStream_t s) {
  switch (rows_per_tile_blocks(a.R)) {
    case 1: return launch_gemm_t<1, 2, 128>(a, groups, s);
    case 2: return launch_gemm_t<2, 2, 128>(a, groups, s);
    case 4: return launch_gemm_t<4, 2, 128>(a, groups, s);
    default:
      if (col_blocks_per_wave(a.R, a.N) == 4)
        return launch_gemm_t<8, 4, 64>(a, groups, s);   // (chunks of 64 keep 128 x 64 per wave in registers)
      return launch_gemm_t<8, 2, 128>(a, groups, s);
  }
}

// K values per split of a product (a multiple of 32)
int up_proj_kchunk(int K, int ks) { return ((K + ks - 1) / ks + 31) / 32 * 32; }

// the matrix-vector path: one row with K = 512 times a power of two up to 16, or two rows up
// to 8 (two rows of 16 would not fit the registers)
bool up_proj_gemv(int R, int K) {
  const int ni = K / 512;
  return K % 512 == 0 && (ni & (ni - 1)) == 0 && ((R == 1 && ni <= 16) || (R == 2 && ni <= 8));
}

template <int RR>
hipError_t launch_gemv_r(const GemmArgs& a, int groups, hipStream_t s) {
  const dim3 grid((unsigned)((a.N + 7) / 8), (unsigned)groups);
  switch (a.K / 512) {
    case 1: hipLaunchKernelGGL((up_gemv_kernel<RR, 1>), grid, dim3(512), 0, s, a); break;
    case 2: hipLaunchKernelGGL((up_gemv_kernel<RR, 2>), grid, dim3(512), 0, s, a); break;
    case 4: hipLaunchKernelGGL((up_gemv_kernel<RR, 4>), grid, dim3(512), 0, s, a); break;
    case 8: hipLaunchKernelGGL((up_gemv_kernel<RR, 8>), grid, dim3(512), 0, s, a); break;
    default:
      if constexpr (RR == 1) hipLaunchKernelGGL((up_gemv_kernel<1, 16>), grid, dim3(512), 0, s, a);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_gemv(const GemmArgs& a, int groups, hipStream_t s) {
  return a.R == 1 ? launch_gemv_r<1>(a, groups, s) : launch_gemv_r<2>(a, groups, s);
}

}  // namespace

int up_proj_ksplit(int R, int Dm, int K) {
  if (up_proj_gemv(R, K)) return 1;   // (every column is one wave's whole sum)
  // enough workgroups for one full round (tiles of up to 32 rows fit two workgroups per compute
  // unit), splits of at least 512 values, partial sums of at most a quarter of the weight bytes
  // (2 * ks * R * Dm floats against Dm * K bf16), at most 16 splits; every split non-empty
  const int rb = rows_per_tile_blocks(R);
  const int64_t occupancy = rb <= 2 ? 2 : 1;
  const int cols = rb == 8 ? 64 * col_blocks_per_wave(R, Dm) : 128;
  const int64_t tiles = (int64_t)((Dm + cols - 1) / cols) * ((R + 16 * rb - 1) / (16 * rb));
  int64_t ks = 256 * occupancy / tiles;
  if (ks > K / 512) ks = K / 512;
  if (ks > K / (16 * (int64_t)R)) ks = K / (16 * (int64_t)R);
  if (ks > 16) ks = 16;
  if (ks < 1) ks = 1;
  const int kc = up_proj_kchunk(K, (int)ks);
  return (K + kc - 1) / kc;
}

hipError_t launch_up_proj(const UpProjParams& p, hipStream_t s) {
  const int K = p.H * p.Dv;
  // v[r, h, :] = W_UV[h] . o[r, h, :]: one group of tiles per head
  GemmArgs v{};
  v.A = p.o;
  v.lda = (int64_t)p.H * kVDim;
  v.a_gs = kVDim;
  v.B = (const __bf16*)p.w_uv;
  v.ldb = kVDim;
  v.b_gs = (int64_t)p.Dv * kVDim;
  v.C = p.v;
  v.ldc = K;
  v.c_gs = p.Dv;
  v.c_ks = 0;
  v.R = p.R;
  v.N = p.Dv;
  v.K = kVDim;
  v.k_chunk = kVDim;
  v.ksplit = 1;
  hipError_t e = up_proj_gemv(p.R, kVDim) ? launch_gemv(v, p.H, s) : launch_gemm(v, p.H, s);
  if (e != hipSuccess) return e;
  // y (or its K-split partial sums) = v . W_O^T
  GemmArgs y{};
  y.A = p.v;
  y.lda = K;
  y.a_gs = 0;
  y.B = (const __bf16*)p.w_o;
  y.ldb = K;
  y.b_gs = 0;
  y.C = p.ksplit == 1 ? p.y : p.part;
  y.ldc = p.Dm;
  y.c_gs = 0;
  y.c_ks = (int64_t)p.R * p.Dm;
  y.R = p.R;
  y.N = p.Dm;
  y.K = K;
  y.k_chunk = up_proj_kchunk(K, p.ksplit);
  y.ksplit = p.ksplit;
  e = up_proj_gemv(p.R, K) && p.ksplit == 1 ? launch_gemv(y, 1, s) : launch_gemm(y, 1, s);
  if (e != hipSuccess || p.ksplit == 1) return e;
  const int64_t total = (int64_t)p.R * p.Dm;
  hipLaunchKernelGGL(up_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace dsa
