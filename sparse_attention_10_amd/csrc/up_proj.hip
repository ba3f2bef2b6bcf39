// Latent up-projection after attention (the step after the sparse MLA decode): with MLA weight
// absorption the query has absorbed kv_b, so the attention output is still in the 512-wide latent
// space and is projected afterwards, per head by that head's value block of kv_b (W_UV), then by
// o_proj (W_O) (Show HN page "Chay GLM 5.2 tren may tinh cham", main-features section, MLA weight
// absorption bullet).
//
//   v[r, h, j] = sum_d W_UV[h, j, d] * o[r, h, d]          (d over the 512 latent values)
//   y[r, m]    = sum_{h, j} W_O[m, h*Dv + j] * v[r, h, j]
//
// Both products run on v_mfma_f32_16x16x32_bf16 (16 rows of r as M, 16 output columns as N).
// The weights are bf16; the activations (o, and v in between) are f32, fed as two bf16 parts
// hi = bf16(a), lo = bf16(a - hi), so a = hi + lo to 2^-18 relative and each product is exact
// in the fp32 accumulator: the result is an fp32-accurate projection.  In decode the rows are few
// (1-128) and the kernels stream the weights once (8 MB of W_UV and 100 MB of W_O at 64 heads,
// Dv = 128, Dm = 6144), so they are bounded by HBM; up_y_kernel splits K over workgroups when the
// rows alone would not fill the GPU, and up_reduce_kernel adds the partial sums in a fixed order.
#include <type_traits>

#include "dsa_internal.hpp"

namespace dsa {

namespace {

constexpr int kUT = 256;   // threads per workgroup (4 waves, 16 output columns each)

// 8 f32 values -> bf16 hi and lo parts (round to nearest even both times)
__device__ __forceinline__ void split8(const f32x4& a0, const f32x4& a1, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = e < 4 ? a0[e] : a1[e - 4];
    const __bf16 h = (__bf16)x;
    hi[e] = h;
    lo[e] = (__bf16)(x - (float)h);
  }
}

// One wave: C[16 rows x 16 cols] += A[rows, k0:k1] . B[cols, k0:k1]^T with A f32 rows of stride
// lda (rows >= nrows read as zero) and B bf16 rows of stride ldb.  Lane (n = l % 16, g = l / 16)
// supplies, for each 32-wide k step, A row n and B row n at k + 8g .. +8.
__device__ __forceinline__ f32x4 mma_rows(const float* __restrict__ A, int64_t lda, int nrows,
                                          const __bf16* __restrict__ Bm, int64_t ldb, int k0, int k1) {
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const bool live = n < nrows;
  const float* a = A + (int64_t)n * lda + 8 * g;
  const __bf16* bp = Bm + (int64_t)n * ldb + 8 * g;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  // U steps per round: every load of the round is issued before its first MFMA
  auto round = [&](int k, auto U) {
    constexpr int NU = decltype(U)::value;
    f32x4 a0[NU], a1[NU];
    bf16x8 b[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      a0[u] = live ? *(const f32x4*)(a + k + 32 * u) : f32x4{0.f, 0.f, 0.f, 0.f};
      a1[u] = live ? *(const f32x4*)(a + k + 32 * u + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
      b[u] = *(const bf16x8*)(bp + k + 32 * u);
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      bf16x8 hi, lo;
      split8(a0[u], a1[u], hi, lo);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, b[u], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, b[u], acc, 0, 0, 0);
    }
  };
  int k = k0;
  for (; k + 256 <= k1; k += 256) round(k, std::integral_constant<int, 8>{});
  for (; k < k1; k += 32) round(k, std::integral_constant<int, 1>{});
  return acc;
}

// v = per-head W_UV . o.  Workgroup (head h, 16-row block, 64-column block of Dv); wave w takes
// value columns 64 cb + 16 w .. +16.
__global__ __launch_bounds__(kUT) void up_v_kernel(UpProjParams p) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int h = blockIdx.x, r0 = blockIdx.y * 16;
  const int c0 = blockIdx.z * 64 + wave * 16;
  if (c0 >= p.Dv) return;                          // (uniform per wave)
  const int nrows = min(16, p.R - r0);
  const float* A = p.o + ((int64_t)r0 * p.H + h) * kVDim;          // rows of stride H*512
  const __bf16* Bm = (const __bf16*)p.w_uv + ((int64_t)h * p.Dv + c0) * kVDim;
  const f32x4 acc = mma_rows(A, (int64_t)p.H * kVDim, nrows, Bm, kVDim, 0, kVDim);
  // lane holds C[row 4g + jx][col n]
  const int n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int jx = 0; jx < 4; ++jx) {
    const int r = 4 * g + jx;
    if (r < nrows) p.v[((int64_t)(r0 + r) * p.H + h) * p.Dv + c0 + n] = acc[jx];
  }
}

// y (or its K-split partial sums) = v . W_O^T.  Workgroup (64-column block, 16-row block,
// K split ks); wave w takes output columns 64 cb + 16 w .. +16 over its K range.
__global__ __launch_bounds__(kUT) void up_y_kernel(UpProjParams p) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int c0 = blockIdx.x * 64 + wave * 16;
  const int r0 = blockIdx.y * 16, ks = blockIdx.z;
  if (c0 >= p.Dm) return;                          // (uniform per wave)
  const int K = p.H * p.Dv;
  const int k0 = ks * p.k_chunk, k1 = min(K, k0 + p.k_chunk);
  const int nrows = min(16, p.R - r0);
  const float* A = p.v + (int64_t)r0 * K;
  const __bf16* Bm = (const __bf16*)p.w_o + (int64_t)c0 * K;
  const f32x4 acc = k0 < k1 ? mma_rows(A, K, nrows, Bm, K, k0, k1) : f32x4{0.f, 0.f, 0.f, 0.f};
  const int n = lane & 15, g = lane >> 4;
  float* dst = p.ksplit == 1 ? p.y : p.part + (int64_t)ks * p.R * p.Dm;
#pragma unroll
  for (int jx = 0; jx < 4; ++jx) {
    const int r = 4 * g + jx;
    if (r < nrows) dst[(int64_t)(r0 + r) * p.Dm + c0 + n] = acc[jx];
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

}  // namespace

int up_proj_ksplit(int R, int Dm, int K) {
  // enough workgroups for the 256 compute units (about two rounds), chunks of at least 512
  const int64_t wg = (int64_t)((Dm + 63) / 64) * ((R + 15) / 16);
  int ks = (int)((512 + wg - 1) / wg);
  const int max_ks = K / 512 > 1 ? K / 512 : 1;
  if (ks > max_ks) ks = max_ks;
  if (ks < 1) ks = 1;
  return ks;
}

hipError_t launch_up_proj(const UpProjParams& p0, hipStream_t s) {
  UpProjParams p = p0;
  const int K = p.H * p.Dv;
  hipLaunchKernelGGL(up_v_kernel, dim3((unsigned)p.H, (unsigned)((p.R + 15) / 16), (unsigned)((p.Dv + 63) / 64)),
                     dim3(kUT), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // K chunks of whole 32-wide steps
  p.k_chunk = ((K + p.ksplit - 1) / p.ksplit + 31) / 32 * 32;
  hipLaunchKernelGGL(up_y_kernel, dim3((unsigned)((p.Dm + 63) / 64), (unsigned)((p.R + 15) / 16), (unsigned)p.ksplit),
                     dim3(kUT), 0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess || p.ksplit == 1) return e;
  const int64_t total = (int64_t)p.R * p.Dm;
  hipLaunchKernelGGL(up_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace dsa
