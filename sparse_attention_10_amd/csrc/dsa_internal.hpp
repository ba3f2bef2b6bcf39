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
typedef int i32x8 __attribute__((ext_vector_type(8)));
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

// 8 e4m3fn bytes (two words) -> 8 bf16, exact
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Direct global -> LDS copies: every lane reads `size` bytes at its own address and lane i's
// bytes land at lds_base + i*size (lds_base must be uniform).  Tracked by the vector-memory
// count like any load.
__device__ __forceinline__ void lds_dma16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void lds_dma4(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_base, 4, 0, 0);
}

// The same copy through a buffer resource over `rows` records of `stride` bytes: lane i reads
// 16 (or 4) bytes at record `row`, byte `off` inside it, and they land at lds_base + i*16 (i*4).
// A record index past the resource's last record reads zeros.  Unlike the global form, the
// compiler does not count these copies as pending LDS operations, so the waits it places for
// later LDS reads stay partial.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, int stride, int64_t rows) {
  const int n = rows > 0x7fffffffLL ? 0x7fffffff : (int)rows;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)stride, n, 0x00020000);
}
__device__ __forceinline__ void lds_dma16_row(__amdgpu_buffer_rsrc_t rsrc, int row, int off, void* lds_base) {
  __builtin_amdgcn_struct_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds_base, 16, row, off, 0, 0,
                                              0);
}
__device__ __forceinline__ void lds_dma4_row(__amdgpu_buffer_rsrc_t rsrc, int row, void* lds_base) {
  __builtin_amdgcn_struct_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds_base, 4, row, 0, 0, 0, 0);
}

// s_waitcnt with only the vector-memory count limited (gfx9 encoding: vmcnt bits 3:0 and 15:14,
// expcnt 6:4 and lgkmcnt 11:8 at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Reductions over the lanes l, l ^ 16, l ^ 32 and l ^ 48 of a wave, on the VALU (row swaps of
// v_permlane16_swap / v_permlane32_swap; no LDS traffic).  Every lane gets the result.
__device__ __forceinline__ float lanes4_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float lanes4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Wait until at most later*PER vector-memory operations are outstanding, later in 0..MAXL
// (a runtime count, resolved into immediate waits).
template <int PER, int MAXL>
__device__ __forceinline__ void wait_vmcnt_later(int later) {
  if constexpr (MAXL <= 0) {
    wait_vmcnt<0>();
  } else {
    if (later >= MAXL) wait_vmcnt<MAXL * PER>();
    else wait_vmcnt_later<PER, MAXL - 1>(later);
  }
}

// Workgroup barrier for rings filled by direct-to-LDS copies.  It waits only for this wave's
// LDS operations (lgkmcnt 0), not for vector-memory operations in flight, which the caller
// bounds with wait_vmcnt beforehand: a __syncthreads also orders global memory, which here
// means waiting for every load in flight, copies into later ring slots included.  The memory
// clobber keeps the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);   // vmcnt 63, expcnt 7, lgkmcnt 0
  asm volatile("s_barrier" ::: "memory");
}

// ---------------------------------------------------------------------------------------------
// Opt-in device-side checks of the data preconditions (builds with DSA_DEBUG defined, the
// library libdsa_debug.so).  A kernel that meets a violation sets its bit in the error word the
// launch passes (dbg) and clamps the offending value into range, so that no access leaves its
// buffer; the host reads and clears the word with dsa_debug_check.  Without DSA_DEBUG these
// compile to nothing and dbg is unused.
enum : uint32_t {
  kDbgSeqLen = 1u,      // seq_lens[b] outside [q_per_seq, max_seq_len]
  kDbgPageId = 2u,      // a page-table entry outside [0, num_slots / page_size)
  kDbgSlot = 4u,        // a slot of dsa_sparse_mla_decode outside [-1, num_slots)
  kDbgNanScore = 8u,    // a NaN among the scores a top-k ranks
  kDbgTopkIndex = 16u,  // an index of dsa_page_map outside [-1, seq_lens[b])
};

__device__ __forceinline__ void dbg_flag(uint32_t* dbg, uint32_t bit) {
#ifdef DSA_DEBUG
  __hip_atomic_fetch_or(dbg, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#else
  (void)dbg;
  (void)bit;
#endif
}
// v if it lies in [lo, hi]; otherwise (DSA_DEBUG builds) flags `bit` and returns v clamped
__device__ __forceinline__ int dbg_clamp(uint32_t* dbg, int v, int lo, int hi, uint32_t bit) {
#ifdef DSA_DEBUG
  if (v < lo || v > hi) {
    dbg_flag(dbg, bit);
    return v < lo ? lo : hi;
  }
#else
  (void)dbg;
  (void)lo;
  (void)hi;
  (void)bit;
#endif
  return v;
}
// a page-table entry, checked against the pool's page count
__device__ __forceinline__ int dbg_page(uint32_t* dbg, int pe, int64_t num_slots, int P) {
  return dbg_clamp(dbg, pe, 0, (int)(num_slots / P) - 1, kDbgPageId);
}
// a slot of the sparse MLA's selection: one outside [-1, num_slots) is flagged (when `flag`) and
// skipped like -1
__device__ __forceinline__ int32_t dbg_slot(uint32_t* dbg, int32_t sv, int64_t num_slots, bool flag = true) {
#ifdef DSA_DEBUG
  if (sv < -1 || sv >= num_slots) {
    if (flag) dbg_flag(dbg, kDbgSlot);
    return -1;
  }
#else
  (void)dbg;
  (void)num_slots;
  (void)flag;
#endif
  return sv;
}
// a sequence length, checked against [Q, max_seq_len] (flag only: every kernel already keeps its
// accesses inside the rows that max_seq_len sizes)
__device__ __forceinline__ void dbg_seq_len(uint32_t* dbg, int L, int Q, int max_seq_len) {
#ifdef DSA_DEBUG
  if (L < Q || L > max_seq_len) dbg_flag(dbg, kDbgSeqLen);
#else
  (void)dbg;
  (void)L;
  (void)Q;
  (void)max_seq_len;
#endif
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
  int64_t num_slots;      // rows of k_cache (and k_scale)
  int32_t B, Q, max_seq_len, P, maxP;
  int32_t Hi, Di;
  int32_t tiles_per_wg;   // matrix-core paths: key tiles (stages) per workgroup
  int32_t groups;         // matrix-core paths: key ranges (workgroups per row group) per sequence
  int32_t p_shift;        // log2(P) when the page size is a power of two, else -1
  // matrix-core decode path, several sequences: key ranges sized from the actual lengths.
  // 0 = ranges of tiles_per_wg tiles over max_seq_len for every sequence; else the number of
  // ranges to aim for (each workgroup derives the partition from seq_lens, see the kernel)
  int32_t balanced;
  // rows i in [q_begin, q_begin + q_count) of every sequence (chunked prefill in row blocks;
  // the many-rows kernel only): scores row (b, i) at scores + (b*q_count + i - q_begin)*ld.
  // q_count = 0: all Q rows
  int32_t q_begin, q_count;
  uint32_t* dbg;          // DSA_DEBUG error word
};

struct TopkParams {
  const float* scores;
  int64_t ld;
  const int32_t* seq_lens;
  const int32_t* page_table;
  int32_t* idx;
  int32_t* slots;   // may be null
  int32_t Q, k, P, maxP;
  // long rows in two passes: chunks of chunk_len columns (nchunks per row) each keep their
  // own top min(k, chunk_len) as candidates (score, column) in ascending column order, then one
  // pass per row selects among the candidates
  int32_t chunk_len, nchunks;
  float* cand_score;      // [rows, cand_ld]
  int32_t* cand_col;      // [rows, cand_ld]
  int64_t cand_ld;
  int64_t num_slots;      // cache rows (DSA_DEBUG page-id checks)
  int32_t max_seq_len;
  // rows i in [q_begin, q_begin + q_count) of every sequence: scores (and candidates) of row
  // (b, i) at local row b*q_count + i - q_begin, idx and slots at row b*Q + i.  q_count = 0:
  // all Q rows
  int32_t q_begin, q_count;
  uint32_t* dbg;          // DSA_DEBUG error word
};

struct MlaParams {
  const void* q;
  const void* kv;
  const float* kv_scale;
  const int32_t* slots;
  int64_t num_slots; // rows of kv (and kv_scale)
  float* out;        // [rows, H, 512] when n_split == 1
  float* lse;        // [rows, H] or null (n_split == 1)
  float* part_o;     // [rows, n_split, H, 512] when n_split > 1
  float* part_m;     // [rows, n_split, H]
  float* part_l;     // [rows, n_split, H]
  int32_t rows, H, k, n_split, chunk;
  int32_t group;     // rows per XCD group: a sequence's verify rows (rows / group sequences,
                     // a multiple of 8), or 1
  float sm_scale;
  uint32_t* dbg;     // DSA_DEBUG error word
};

struct CombineParams {
  const float* part_o;
  const float* part_m;
  const float* part_l;
  float* out;
  float* lse;
  int32_t rows, H, n_split;
};

// Cache append: row r = b*Q + i of each source goes to slot(b, L_b - Q + i) of its cache.  A
// NULL destination skips that cache.  Widths are multiples of 8, at most 1024.
struct AppendParams {
  const int32_t* seq_lens;
  const int32_t* page_table;
  const void* kv_src;
  void* kv_dst;
  float* kv_scale;
  const void* k_src;
  void* k_dst;
  float* k_scale;
  int64_t rows;
  int32_t Q, P, maxP;
  int32_t kv_width, k_width;
  int32_t kv_src_dtype, kv_dst_dtype, k_src_dtype, k_dst_dtype;
  int64_t num_slots;      // cache rows (DSA_DEBUG page-id checks)
  int32_t max_seq_len;
  uint32_t* dbg;          // DSA_DEBUG error word
};

// Latent up-projection after attention: o [R, H, 512] f32 -> v [R, H, Dv] f32 (workspace) ->
// y [R, Dm] f32, with K = H * Dv split into ksplit chunks whose partial sums (part, [ksplit, R,
// Dm], workspace) are added in order when ksplit > 1.
struct UpProjParams {
  const float* o;
  const void* w_uv;   // [H, Dv, 512] bf16
  const void* w_o;    // [Dm, H*Dv] bf16
  float* v;
  float* part;
  float* y;
  int32_t R, H, Dv, Dm, ksplit;
};

// launchers (return hipGetLastError() of the launch)
hipError_t launch_indexer(const IndexerParams& p, dsa_dtype_t q_dtype, dsa_dtype_t k_dtype,
                          hipStream_t s);
bool indexer_uses_mfma(int Hi, int Di, dsa_dtype_t q_dtype, dsa_dtype_t k_dtype);
// the many-rows (chunked prefill) kernel, the one that takes row windows (q_begin, q_count)
bool indexer_uses_prefill(int Hi, int Di, int Q, int P, dsa_dtype_t q_dtype, dsa_dtype_t k_dtype);
// Top-k: `ws` is topk_workspace_bytes(rows, max_seq_len, k) bytes of device memory (the
// candidates of the two-pass plan for long rows; no initial contents), or unused when that
// size is 0.
size_t topk_workspace_bytes(int64_t rows, int max_seq_len, int k);
hipError_t launch_topk(const TopkParams& p, int rows, int max_seq_len, void* ws, hipStream_t s);
hipError_t launch_page_map(const int32_t* idx, int64_t total, int k, int Q, const int32_t* pt,
                           int maxP, int P, int32_t* slots, const int32_t* seq_lens, int64_t num_slots,
                           uint32_t* dbg, hipStream_t s);
hipError_t launch_mla(const MlaParams& p, dsa_dtype_t q_dtype, dsa_dtype_t kv_dtype, hipStream_t s);
hipError_t launch_combine(const CombineParams& p, hipStream_t s);
int mla_default_split(int rows, int H, int k, dsa_dtype_t kv_dtype);
// bf16 rows and at most 16 (query row, 16-head group) pairs: the few-rows kernel (16 heads per
// workgroup, 128-token tiles)
bool mla_uses_narrow(int rows, int H, dsa_dtype_t kv_dtype);
hipError_t launch_cache_append(const AppendParams& p, hipStream_t s);
int up_proj_ksplit(int R, int Dm, int K);
hipError_t launch_up_proj(const UpProjParams& p, hipStream_t s);

}  // namespace dsa
