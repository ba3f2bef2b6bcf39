// Cache append: the write that precedes the sparse path on every decode step.  Each new token's
// 576-wide latent row and its indexer key go to the token's paged slot; an fp8 cache receives a
// per-token scale, max |row| / 448, and the nearest-even e4m3fn codes of row / scale (the
// renning22/glm-5.2-4090 README, usage section, serves with an fp8_e4m3 KV cache; one f32 scale
// per token row is this library's choice of granularity, not something the pages specify).
//
// One wave per (token, cache): the wave loads the row as 8-value chunks (lane l takes chunks l
// and l + 64), reduces the row maximum across its 64 lanes, and stores the converted chunks
// with one 8-, 16- or 32-byte store per chunk.  The work is a few KB per decode step, so the
// kernel is bounded by its two dependent reads (sequence length, page-table entry) and the
// row's own load; at prefill sizes (thousands of tokens) it streams at the copy rate.
#include "dsa_internal.hpp"

namespace dsa {
namespace {

constexpr float kE4m3Max = 448.0f;
// A row whose largest magnitude is below 2^-100 keeps the scale 1 (as an all-zero row does):
// its values all encode to signed zeros, and no scale underflows the binary32 range.
constexpr float kScaleFloor = 0x1p-100f;

// binary32 -> OCP e4m3fn code: magnitude clamped to 448, then rounded to nearest with ties to
// the even code; the sign bit is kept, so -0 and small negatives give 0x80.
__device__ inline uint32_t e4m3fn_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fminf(fabsf(y), kE4m3Max);
  uint32_t mag;
  if (a < 0x1p-6f) {
    // subnormal grid m * 2^-9 (m = 8 is the smallest normal, code 0x08); a * 512 is exact
    mag = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    // keep 3 of the 23 mantissa bits with round-half-even on the dropped 20 (a carry moves
    // into the exponent), then rebias the exponent from 127 to 7: (127 - 7) << 3 = 960
    const uint32_t bits = __float_as_uint(a);
    mag = ((bits + 0x7FFFFu + ((bits >> 20) & 1u)) >> 20) - 960u;
  }
  return mag | sign;
}

__device__ inline void load8(const void* src, int dtype, int64_t off, float (&v)[8]) {
  if (dtype == DSA_BF16) {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + off);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(w[e] << 16);
      v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  } else {
    const float4* f = reinterpret_cast<const float4*>(static_cast<const float*>(src) + off);
    const float4 a = f[0], b = f[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

__global__ __launch_bounds__(256) void cache_append_kernel(AppendParams p) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t task = (int64_t)blockIdx.x * 4 + wave;
  if (task >= 2 * p.rows) return;
  // tasks alternate latent row / indexer key of the same token, so both waves of a token read
  // the same length and page-table entry
  const bool key = (task & 1) != 0;
  const int64_t row = task >> 1;
  const void* src = key ? p.k_src : p.kv_src;
  void* dst = key ? p.k_dst : p.kv_dst;
  float* scale = key ? p.k_scale : p.kv_scale;
  const int width = key ? p.k_width : p.kv_width;
  const int sdt = key ? p.k_src_dtype : p.kv_src_dtype;
  const int ddt = key ? p.k_dst_dtype : p.kv_dst_dtype;
  if (dst == nullptr) return;
  const int b = (int)(row / p.Q), i = (int)(row - (int64_t)b * p.Q);
  const int Lb = p.seq_lens[b];
#ifdef DSA_DEBUG
  // a length or page id out of range (flagged) writes nothing for this token
  if (Lb < p.Q || Lb > p.max_seq_len) {
    if (lane == 0) dbg_flag(p.dbg, kDbgSeqLen);
    return;
  }
#endif
  const int pos = Lb - p.Q + i;
  const int pe = p.page_table[(int64_t)b * p.maxP + pos / p.P];
#ifdef DSA_DEBUG
  if (pe < 0 || (int64_t)pe >= p.num_slots / p.P) {
    if (lane == 0) dbg_flag(p.dbg, kDbgPageId);
    return;
  }
#endif
  const int64_t slot = (int64_t)pe * p.P + pos % p.P;
  const int nchunk = width >> 3;
  float v[2][8];
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = lane + 64 * j;
    if (c < nchunk) {
      load8(src, sdt, row * width + c * 8, v[j]);
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[j][e]));
    }
  }
  if (ddt == DSA_FP8_E4M3FN) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
    // IEEE (round-to-nearest-even) binary32 divisions, for the scale and for each value
    const float sc = amax >= kScaleFloor ? __fdiv_rn(amax, kE4m3Max) : 1.0f;
    uint8_t* d = static_cast<uint8_t*>(dst) + slot * width;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = lane + 64 * j;
      if (c < nchunk) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lo |= e4m3fn_code(__fdiv_rn(v[j][e], sc)) << (8 * e);
          hi |= e4m3fn_code(__fdiv_rn(v[j][e + 4], sc)) << (8 * e);
        }
        *reinterpret_cast<uint2*>(d + c * 8) = make_uint2(lo, hi);
      }
    }
    if (lane == 0) scale[slot] = sc;
  } else if (ddt == DSA_BF16) {
    // bf16 rows into a bf16 cache: the stored bits, unchanged
    uint16_t* d = static_cast<uint16_t*>(dst) + slot * width;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = lane + 64 * j;
      if (c < nchunk) {
        uint4 u;
        u.x = (__float_as_uint(v[j][0]) >> 16) | (__float_as_uint(v[j][1]) & 0xFFFF0000u);
        u.y = (__float_as_uint(v[j][2]) >> 16) | (__float_as_uint(v[j][3]) & 0xFFFF0000u);
        u.z = (__float_as_uint(v[j][4]) >> 16) | (__float_as_uint(v[j][5]) & 0xFFFF0000u);
        u.w = (__float_as_uint(v[j][6]) >> 16) | (__float_as_uint(v[j][7]) & 0xFFFF0000u);
        *reinterpret_cast<uint4*>(d + c * 8) = u;
      }
    }
  } else {
    float* d = static_cast<float*>(dst) + slot * width;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = lane + 64 * j;
      if (c < nchunk) {
        float4* o = reinterpret_cast<float4*>(d + c * 8);
        o[0] = make_float4(v[j][0], v[j][1], v[j][2], v[j][3]);
        o[1] = make_float4(v[j][4], v[j][5], v[j][6], v[j][7]);
      }
    }
  }
}

}  // namespace

hipError_t launch_cache_append(const AppendParams& p, hipStream_t s) {
  if (p.rows == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((2 * p.rows + 3) / 4);
  hipLaunchKernelGGL(cache_append_kernel, dim3(blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace dsa
