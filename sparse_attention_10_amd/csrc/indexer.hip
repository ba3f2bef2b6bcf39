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
// matrix-core path: Hi = 64, Di = 128, QB query rows per workgroup (M = 64 * QB)

constexpr int kHi = 64, kDi = 128;
constexpr int kSub = 32;                  // tokens per wave sub-tile (the MFMA N)
constexpr int kWaves = 4;
constexpr int kTile = kSub * kWaves;      // tokens per workgroup tile

template <bool FP8>
struct KeyFrag {
  // 8 k-steps of 8 bf16 (B operand), covering dims [h*64, h*64+64) of the lane's token
  bf16x8 v[8];
};

// Issue the loads of one sub-tile's key fragment.  Raw bits are kept so the fp8 widening can
// run after the loads have landed.
template <bool FP8>
struct KeyRaw {
  u32x4 r[FP8 ? 4 : 8];
};

template <bool FP8>
__device__ __forceinline__ void load_keys(KeyRaw<FP8>& raw, const uint8_t* kc, int64_t slot, bool valid,
                                          int half) {
  if (valid) {
    const u32x4* src = (const u32x4*)(kc + slot * (FP8 ? kDi : 2 * kDi) + half * (FP8 ? 64 : 128));
#pragma unroll
    for (int c = 0; c < (FP8 ? 4 : 8); ++c) raw.r[c] = __builtin_nontemporal_load(src + c);
  } else {
#pragma unroll
    for (int c = 0; c < (FP8 ? 4 : 8); ++c) raw.r[c] = u32x4{0, 0, 0, 0};
  }
}

template <bool FP8>
__device__ __forceinline__ void widen_keys(const KeyRaw<FP8>& raw, KeyFrag<FP8>& f) {
  if constexpr (FP8) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      __bf16 tmp[16];
#pragma unroll
      for (int d = 0; d < 4; ++d) fp8x4_to_bf16x4(raw.r[c][d], tmp + 4 * d);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        f.v[2 * c][j] = tmp[j];
        f.v[2 * c + 1][j] = tmp[8 + j];
      }
    }
  } else {
#pragma unroll
    for (int s = 0; s < 8; ++s) f.v[s] = __builtin_bit_cast(bf16x8, raw.r[s]);
  }
}

template <int QB, bool FP8>
__global__ __launch_bounds__(256) void indexer_mfma_kernel(IndexerParams p) {
  __shared__ __attribute__((aligned(16))) __bf16 q_lds[QB][kHi][kDi];
  __shared__ float w_lds[QB][kHi];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int b = blockIdx.z;
  const int qb0 = blockIdx.y * QB;            // first query row of this block within the sequence
  const int L = min(p.seq_lens[b], p.max_seq_len);
  const int tile_base = blockIdx.x * p.tiles_per_wg * kTile;
  if (tile_base >= L) return;                 // uniform early exit
  const int tile_end = min(L, tile_base + p.tiles_per_wg * kTile);
  const int nrows = QB;                       // the launcher picks QB dividing Q
  const int pos_last = L - p.Q + qb0 + nrows - 1;   // largest position in the block

  const int n_in_sub = lane & 31;
  const int half = lane >> 5;
  const uint8_t* kc = (const uint8_t*)p.k_cache;
  const int32_t* ptab = p.page_table + (int64_t)b * p.maxP;

  // first sub-tile's keys are requested before q is staged, so both latencies overlap
  int t_cur = tile_base + wave * kSub + n_in_sub;
  auto slot_of = [&](int t) -> int64_t { return (int64_t)ptab[t / p.P] * p.P + t % p.P; };
  bool v_cur = t_cur < tile_end && t_cur <= pos_last;
  int64_t s_cur = v_cur ? slot_of(t_cur) : 0;
  KeyRaw<FP8> raw_cur;
  load_keys<FP8>(raw_cur, kc, s_cur, v_cur, half);

  // stage q (bf16) and w for the block's query rows (QB divides Q, so the block is always
  // QB full rows); all loads are issued before the first LDS store
  {
    const int64_t row0 = (int64_t)b * p.Q + qb0;
    const u32x4* qsrc = (const u32x4*)((const __bf16*)p.q + row0 * kHi * kDi);
    u32x4* qdst = (u32x4*)&q_lds[0][0][0];
    constexpr int kPer = QB * kHi * kDi / 8 / 256;
    u32x4 qv[kPer];
#pragma unroll
    for (int c = 0; c < kPer; ++c) qv[c] = qsrc[c * 256 + threadIdx.x];
    const float wv = threadIdx.x < QB * kHi ? p.w[row0 * kHi + threadIdx.x] : 0.f;
#pragma unroll
    for (int c = 0; c < kPer; ++c) qdst[c * 256 + threadIdx.x] = qv[c];
    if (threadIdx.x < QB * kHi) (&w_lds[0][0])[threadIdx.x] = wv;
  }
  __syncthreads();

  // A fragments: lane (head m = lane%32 of M-block mb, half h) holds, for k-step s,
  // q dims [h*64 + s*8, +8)
  bf16x8 afrag[2 * QB][8];
#pragma unroll
  for (int mb = 0; mb < 2 * QB; ++mb)
#pragma unroll
    for (int s = 0; s < 8; ++s)
      afrag[mb][s] = *(const bf16x8*)&q_lds[mb >> 1][(mb & 1) * 32 + n_in_sub][half * 64 + s * 8];

  // heads held by this lane in each 32-row M-block: m(j) = (j/4)*8 + half*4 + j%4
  for (int sub = tile_base + wave * kSub; sub < tile_end; sub += kTile) {
    const int t_nxt = sub + kTile + n_in_sub;
    const bool v_nxt = t_nxt < tile_end && t_nxt <= pos_last;
    const int64_t s_nxt = v_nxt ? slot_of(t_nxt) : 0;
    KeyRaw<FP8> raw_nxt;
    load_keys<FP8>(raw_nxt, kc, s_nxt, v_nxt, half);   // prefetch the next sub-tile

    KeyFrag<FP8> kf;
    widen_keys<FP8>(raw_cur, kf);
    f32x16 acc[2 * QB];
#pragma unroll
    for (int mb = 0; mb < 2 * QB; ++mb) {
      acc[mb] = f32x16{};
#pragma unroll
      for (int s = 0; s < 8; ++s)
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag[mb][s], kf.v[s], acc[mb], 0, 0, 0);
    }
    const float kscale = (FP8 && v_cur) ? p.k_scale[s_cur] : 1.f;
#pragma unroll
    for (int qi = 0; qi < QB; ++qi) {
      float part = 0.f;
#pragma unroll
      for (int mbl = 0; mbl < 2; ++mbl) {
        const int mb = 2 * qi + mbl;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 wv = *(const f32x4*)&w_lds[qi][mbl * 32 + g * 8 + half * 4];
#pragma unroll
          for (int j = 0; j < 4; ++j) part = fmaf(wv[j], fmaxf(acc[mb][4 * g + j], 0.f), part);
        }
      }
      part += __shfl_xor(part, 32);
      if (half == 0 && qi < nrows && t_cur < tile_end) {
        const int pos = L - p.Q + qb0 + qi;
        float* dst = p.scores + ((int64_t)b * p.Q + qb0 + qi) * p.ld;
        dst[t_cur] = t_cur <= pos ? part * kscale : -INFINITY;
      }
    }
    raw_cur = raw_nxt;
    t_cur = t_nxt;
    v_cur = v_nxt;
    s_cur = s_nxt;
  }
}

}  // namespace

bool indexer_uses_mfma(int Hi, int Di, dsa_dtype_t q_dtype, dsa_dtype_t k_dtype) {
  return Hi == kHi && Di == kDi && q_dtype == DSA_BF16 && (k_dtype == DSA_BF16 || k_dtype == DSA_FP8_E4M3FN);
}

hipError_t launch_indexer(const IndexerParams& p0, dsa_dtype_t q_dtype, dsa_dtype_t k_dtype, hipStream_t s) {
  IndexerParams p = p0;
  if (indexer_uses_mfma(p.Hi, p.Di, q_dtype, k_dtype)) {
    const int QB = (p.Q % 2 == 0) ? 2 : 1;
    const int64_t tiles = ((int64_t)p.max_seq_len + kTile - 1) / kTile;
    const int64_t work = tiles * p.B * ((p.Q + QB - 1) / QB);
    // keep >= ~4 workgroups per compute unit, then give each workgroup several tiles
    int tpw = (int)(work / 2048);
    tpw = tpw < 1 ? 1 : (tpw > 8 ? 8 : tpw);
    p.tiles_per_wg = tpw;
    dim3 grid((unsigned)((tiles + tpw - 1) / tpw), (unsigned)((p.Q + QB - 1) / QB), (unsigned)p.B);
    const bool f8 = k_dtype == DSA_FP8_E4M3FN;
    if (QB == 2) {
      if (f8) hipLaunchKernelGGL((indexer_mfma_kernel<2, true>), grid, dim3(256), 0, s, p);
      else hipLaunchKernelGGL((indexer_mfma_kernel<2, false>), grid, dim3(256), 0, s, p);
    } else {
      if (f8) hipLaunchKernelGGL((indexer_mfma_kernel<1, true>), grid, dim3(256), 0, s, p);
      else hipLaunchKernelGGL((indexer_mfma_kernel<1, false>), grid, dim3(256), 0, s, p);
    }
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
