// Internal declarations shared by the gfx950 kernels of the DSA decode path and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dsa.h"

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kRowDim = 576;   // compressed latent row: 512 latent + 64 RoPE values
constexpr int kVDim = 512;     // V = first 512 values of the row
constexpr int kMaxTopK = 8192;
constexpr int kMaxTopkSeq = 262144;

// ---------------------------------------------------------------------------------------------
// element decoders (exact)

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// 4 e4m3fn codes packed in a dword -> 4 bf16 (exact: every e4m3fn value is a bf16 value).
__device__ __forceinline__ void fp8x4_to_bf16x4(uint32_t w, __bf16* out) {
  bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  out[0] = lo[0]; out[1] = lo[1]; out[2] = hi[0]; out[3] = hi[1];
}

__device__ __forceinline__ float fp8_to_f32(uint32_t code) {
  return __builtin_amdgcn_cvt_f32_fp8(code, 0);
}

// ---------------------------------------------------------------------------------------------
// launch parameter blocks (plain structs passed by value to the kernels)

struct IndexerParams {
  const int32_t* seq_lens;
  const int32_t* page_table;
  const void* q;
  const float* w;
  const void* k_cache;
  const float* k_scale;
  float* scores;
  int64_t ld;
  int32_t B, Q, max_seq_len, P, maxP;
  int32_t Hi, Di;
  int32_t tiles_per_wg;   // matrix-core path: 128-token tiles per workgroup
  int32_t groups_padded;  // matrix-core path: tile groups per sequence, rounded up to 8
  int32_t p_shift;        // log2(P) when the page size is a power of two, else -1
};

struct TopkParams {
  const float* scores;
  int64_t ld;
  const int32_t* seq_lens;
  const int32_t* page_table;
  int32_t* idx;
  int32_t* slots;   // may be null
  int32_t Q, k, P, maxP;
};

struct MlaParams {
  const void* q;
  const void* kv;
  const float* kv_scale;
  const int32_t* slots;
  float* out;        // [rows, H, 512] when n_split == 1
  float* lse;        // [rows, H] or null (n_split == 1)
  float* part_o;     // [rows, n_split, H, 512] when n_split > 1
  float* part_m;     // [rows, n_split, H]
  float* part_l;     // [rows, n_split, H]
  int32_t rows, H, k, n_split, chunk;
  float sm_scale;
};

struct CombineParams {
  const float* part_o;
  const float* part_m;
  const float* part_l;
  float* out;
  float* lse;
  int32_t rows, H, n_split;
};

// launchers (return hipGetLastError() of the launch)
hipError_t launch_indexer(const IndexerParams& p, dsa_dtype_t q_dtype, dsa_dtype_t k_dtype,
                          hipStream_t s);
bool indexer_uses_mfma(int Hi, int Di, dsa_dtype_t q_dtype, dsa_dtype_t k_dtype);
// Top-k: `ws` is topk_workspace_bytes(rows, max_seq_len) bytes of zero-filled device memory
// (left zero-filled by the launch), or unused when that size is 0.
size_t topk_workspace_bytes(int64_t rows, int max_seq_len);
hipError_t launch_topk(const TopkParams& p, int rows, int max_seq_len, void* ws, hipStream_t s);
hipError_t launch_page_map(const int32_t* idx, int64_t total, int k, int Q, const int32_t* pt,
                           int maxP, int P, int32_t* slots, hipStream_t s);
hipError_t launch_mla(const MlaParams& p, dsa_dtype_t q_dtype, dsa_dtype_t kv_dtype, hipStream_t s);
hipError_t launch_combine(const CombineParams& p, hipStream_t s);
int mla_default_split(int rows, int H, int k);

}  // namespace dsa
