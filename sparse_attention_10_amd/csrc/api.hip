// C ABI of the DSA decode path: argument validation, status reporting, workspace layout and
// dispatch to the gfx950 kernels.  Nothing is enqueued unless every check passes.
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "dsa_internal.hpp"

using namespace dsa;

namespace {

thread_local char g_err[512] = "";

dsa_status_t fail(dsa_status_t s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

#define DSA_REQUIRE(cond, ...)                                  \
  do {                                                          \
    if (!(cond)) return fail(DSA_ERR_INVALID_ARGUMENT, __VA_ARGS__); \
  } while (0)

#define DSA_SUPPORT(cond, ...)                               \
  do {                                                       \
    if (!(cond)) return fail(DSA_ERR_UNSUPPORTED, __VA_ARGS__); \
  } while (0)

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Per-device answer to "is this a gfx950": 0 unknown, 1 yes, 2 no.
constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_ok[kMaxDevices];

dsa_status_t check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(DSA_ERR_UNSUPPORTED, "device ordinal %d out of range", dev);
  int st = g_dev_ok[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(DSA_ERR_HIP, "hipGetDeviceProperties failed: %s", hipGetErrorString(e));
    st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_dev_ok[dev].store(st, std::memory_order_release);
  }
  if (st != 1) return fail(DSA_ERR_UNSUPPORTED, "device %d is not a gfx950 (MI355X) GPU", dev);
  return DSA_OK;
}

// The error word of the opt-in device-side checks (DSA_DEBUG builds): one per device, zero when
// the library is loaded, reached by host code only through the address hipGetSymbolAddress
// returns for the current device.  Other builds pass no word (nullptr).
#ifdef DSA_DEBUG
static __device__ uint32_t g_dbg_word;
std::atomic<uint32_t*> g_dbg_ptr[kMaxDevices];
#endif

dsa_status_t debug_word(uint32_t** out) {
  *out = nullptr;
#ifdef DSA_DEBUG
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(DSA_ERR_UNSUPPORTED, "device ordinal %d out of range", dev);
  uint32_t* p = g_dbg_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void* v = nullptr;
    e = hipGetSymbolAddress(&v, HIP_SYMBOL(g_dbg_word));
    if (e != hipSuccess || v == nullptr)
      return fail(DSA_ERR_HIP, "hipGetSymbolAddress(debug word) failed on device %d: %s", dev, hipGetErrorString(e));
    p = (uint32_t*)v;
    g_dbg_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
#endif
  return DSA_OK;
}

dsa_status_t launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return DSA_OK;
}

bool valid_dtype(dsa_dtype_t d) { return d == DSA_F32 || d == DSA_BF16 || d == DSA_FP8_E4M3FN; }
size_t dtype_size(dsa_dtype_t d) { return d == DSA_F32 ? 4 : (d == DSA_BF16 ? 2 : 1); }

dsa_status_t check_batch(const dsa_batch_t* b) {
  DSA_REQUIRE(b != nullptr, "batch is NULL");
  DSA_REQUIRE(b->batch >= 1, "batch.batch must be >= 1 (got %d)", b->batch);
  DSA_REQUIRE(b->q_per_seq >= 1, "batch.q_per_seq must be >= 1 (got %d)", b->q_per_seq);
  DSA_REQUIRE(b->max_seq_len >= b->q_per_seq, "batch.max_seq_len (%d) must be >= q_per_seq (%d)",
              b->max_seq_len, b->q_per_seq);
  DSA_REQUIRE(b->page_size >= 1, "batch.page_size must be >= 1 (got %d)", b->page_size);
  DSA_REQUIRE((int64_t)b->max_pages_per_seq * b->page_size >= b->max_seq_len,
              "batch.max_pages_per_seq (%d) * page_size (%d) must cover max_seq_len (%d)",
              b->max_pages_per_seq, b->page_size, b->max_seq_len);
  DSA_REQUIRE(b->num_slots >= 1, "batch.num_slots must be >= 1");
  DSA_REQUIRE(b->seq_lens != nullptr, "batch.seq_lens is NULL");
  DSA_REQUIRE(b->page_table != nullptr, "batch.page_table is NULL");
  DSA_REQUIRE(aligned(b->seq_lens, 4) && aligned(b->page_table, 4), "batch arrays must be 4-byte aligned");
  return DSA_OK;
}

#define DSA_TRY(x)                 \
  do {                             \
    dsa_status_t _s = (x);         \
    if (_s != DSA_OK) return _s;   \
  } while (0)

dsa_status_t check_indexer(const dsa_batch_t* b, const void* q, dsa_dtype_t q_dtype, const float* w,
                           const void* k_cache, dsa_dtype_t k_dtype, const float* k_scale, int32_t Hi,
                           int32_t Di, const float* scores, int64_t ld) {
  DSA_TRY(check_batch(b));
  DSA_REQUIRE(q && w && k_cache && scores, "indexer: q, w, k_cache and scores must be non-NULL");
  DSA_REQUIRE(q_dtype == DSA_F32 || q_dtype == DSA_BF16, "indexer: q dtype must be f32 or bf16");
  DSA_REQUIRE(valid_dtype(k_dtype), "indexer: unknown key dtype %d", (int)k_dtype);
  DSA_REQUIRE(k_dtype != DSA_FP8_E4M3FN || k_scale != nullptr, "indexer: fp8 keys need k_scale");
  DSA_REQUIRE(Hi >= 1 && Di >= 1, "indexer: n_heads and head_dim must be >= 1");
  DSA_SUPPORT(Hi <= 128 && Di <= 256 && (int64_t)Hi * Di <= 16000,
              "indexer: n_heads=%d head_dim=%d outside the supported set (<=128, <=256, product <= 16000)", Hi, Di);
  DSA_REQUIRE(ld >= b->max_seq_len, "indexer: scores_ld (%lld) < max_seq_len (%d)", (long long)ld, b->max_seq_len);
  DSA_REQUIRE(aligned(w, 4) && aligned(scores, 4) && (!k_scale || aligned(k_scale, 4)),
              "indexer: f32 arrays must be 4-byte aligned");
  if (indexer_uses_mfma(Hi, Di, q_dtype, k_dtype))
    DSA_REQUIRE(aligned(q, 16) && aligned(k_cache, 16), "indexer: q and k_cache must be 16-byte aligned");
  else
    DSA_REQUIRE(aligned(q, dtype_size(q_dtype)) && aligned(k_cache, dtype_size(k_dtype)),
                "indexer: q / k_cache misaligned for their dtype");
  return DSA_OK;
}

dsa_status_t check_topk(const dsa_batch_t* b, const float* scores, int64_t ld, int32_t k, const int32_t* idx) {
  DSA_TRY(check_batch(b));
  DSA_REQUIRE(scores && idx, "topk: scores and topk_idx must be non-NULL");
  DSA_REQUIRE(k >= 1, "topk: k must be >= 1 (got %d)", k);
  DSA_SUPPORT(k <= kMaxTopK, "topk: k=%d above the supported maximum %d", k, kMaxTopK);
  DSA_SUPPORT(b->max_seq_len <= kMaxTopkSeq, "topk: max_seq_len=%d above the supported maximum %d",
              b->max_seq_len, kMaxTopkSeq);
  DSA_REQUIRE(ld >= b->max_seq_len, "topk: scores_ld (%lld) < max_seq_len (%d)", (long long)ld, b->max_seq_len);
  DSA_REQUIRE(aligned(scores, 4) && aligned(idx, 4), "topk: arrays must be 4-byte aligned");
  return DSA_OK;
}

bool mla_uses_mfma(dsa_dtype_t q_dtype) { return q_dtype == DSA_BF16; }

dsa_status_t check_mla(int32_t B, int32_t Q, const void* q, dsa_dtype_t q_dtype, const void* kv,
                       dsa_dtype_t kv_dtype, const float* kv_scale, int64_t num_slots, const int32_t* slots,
                       int32_t k, int32_t H, float sm_scale, const float* out, const float* lse, int32_t n_split) {
  DSA_REQUIRE(B >= 1 && Q >= 1, "mla: batch and q_per_seq must be >= 1");
  DSA_REQUIRE(q && kv && slots && out, "mla: q, kv_cache, slots and out must be non-NULL");
  DSA_REQUIRE(q_dtype == DSA_F32 || q_dtype == DSA_BF16, "mla: q dtype must be f32 or bf16");
  DSA_REQUIRE(valid_dtype(kv_dtype), "mla: unknown kv dtype %d", (int)kv_dtype);
  DSA_REQUIRE(kv_dtype != DSA_FP8_E4M3FN || kv_scale != nullptr, "mla: fp8 rows need kv_scale");
  DSA_REQUIRE(num_slots >= 1, "mla: num_slots must be >= 1");
  DSA_REQUIRE(k >= 1, "mla: k must be >= 1 (got %d)", k);
  DSA_SUPPORT(k <= kMaxTopK, "mla: k=%d above the supported maximum %d", k, kMaxTopK);
  DSA_REQUIRE(H >= 1, "mla: n_heads must be >= 1");
  DSA_REQUIRE(std::isfinite(sm_scale), "mla: sm_scale must be finite");
  DSA_REQUIRE(n_split >= 0 && n_split <= 1024, "mla: n_split must be in 0..1024 (got %d)", n_split);
  if (mla_uses_mfma(q_dtype)) {
    DSA_SUPPORT(H == 16 || H == 32 || H == 48 || H == 64,
                "mla: bf16 q supports n_heads in {16,32,48,64} (got %d)", H);
    DSA_SUPPORT(kv_dtype != DSA_F32, "mla: bf16 q needs bf16 or fp8 rows");
    DSA_REQUIRE(aligned(q, 16) && aligned(kv, 16), "mla: q and kv_cache must be 16-byte aligned");
  } else {
    DSA_SUPPORT(H <= 128, "mla: f32 q supports n_heads <= 128 (got %d)", H);
    DSA_REQUIRE(aligned(q, 4) && aligned(kv, dtype_size(kv_dtype)), "mla: q / kv_cache misaligned");
  }
  DSA_REQUIRE(aligned(out, 16) && aligned(slots, 4) && (!lse || aligned(lse, 4)) &&
                  (!kv_scale || aligned(kv_scale, 4)),
              "mla: out must be 16-byte aligned, slots / lse / kv_scale 4-byte aligned");
  return DSA_OK;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct MlaWs {
  size_t o_bytes, ml_bytes, total;
};

MlaWs mla_ws(int64_t rows, int32_t H, int32_t ns) {
  MlaWs w{0, 0, 0};
  if (ns <= 1) return w;
  w.o_bytes = align_up((size_t)rows * ns * H * kVDim * sizeof(float), 256);
  w.ml_bytes = align_up((size_t)rows * ns * H * sizeof(float), 256);
  w.total = w.o_bytes + 2 * w.ml_bytes;
  return w;
}

int32_t effective_split(int64_t rows, int32_t H, int32_t k, int32_t n_split, dsa_dtype_t q_dtype,
                        dsa_dtype_t kv_dtype) {
  if (!mla_uses_mfma(q_dtype)) return 1;
  int32_t ns = n_split > 0 ? n_split : mla_default_split((int)rows, H, k, kv_dtype);
  // never more chunks than 32-row tiles
  const int32_t max_ns = (k + 31) / 32;
  return ns > max_ns ? max_ns : ns;
}

dsa_status_t run_mla(int64_t rows, int32_t q_per_seq, const void* q, dsa_dtype_t q_dtype, const void* kv, dsa_dtype_t kv_dtype,
                     const float* kv_scale, int64_t num_slots, const int32_t* slots, int32_t k, int32_t H, float sm_scale, float* out,
                     float* lse, int32_t ns, void* ws, size_t ws_bytes, uint32_t* dbg, hipStream_t s) {
  MlaWs w = mla_ws(rows, H, ns);
  if (ws_bytes < w.total || (w.total > 0 && ws == nullptr))
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "mla: workspace needs %zu bytes (got %zu)", w.total, ws_bytes);
  if (w.total > 0 && !aligned(ws, 256)) return fail(DSA_ERR_INVALID_ARGUMENT, "mla: workspace must be 256-byte aligned");
  MlaParams p{};
  p.q = q;
  p.kv = kv;
  p.kv_scale = kv_dtype == DSA_FP8_E4M3FN ? kv_scale : nullptr;
  p.num_slots = num_slots;
  p.slots = slots;
  p.out = out;
  p.lse = lse;
  p.rows = (int32_t)rows;
  // The verify rows of a sequence share one XCD when the sequences fill the 8 XCDs evenly:
  // row i's chunk j runs beside the other rows' chunk j, so a token that several rows of the
  // sequence selected is fetched from HBM once and read again from that XCD's L2.
  const int64_t nseq = q_per_seq > 0 ? rows / q_per_seq : 0;
  p.group = q_per_seq > 1 && nseq >= 8 && nseq % 8 == 0 ? q_per_seq : 1;
  p.H = H;
  p.k = k;
  p.n_split = ns;
  p.sm_scale = sm_scale;
  p.dbg = dbg;
  if (ns > 1) {
    uint8_t* base = (uint8_t*)ws;
    p.part_o = (float*)base;
    p.part_m = (float*)(base + w.o_bytes);
    p.part_l = (float*)(base + w.o_bytes + w.ml_bytes);
  }
  return launched(launch_mla(p, q_dtype, kv_dtype, s), "sparse MLA");
}

// One side (latent rows or indexer keys) of a cache append.
dsa_status_t check_append_side(const char* what, const void* src, dsa_dtype_t sdt, const void* dst,
                               dsa_dtype_t ddt, const float* scale, int32_t width) {
  if (src == nullptr && dst == nullptr) return DSA_OK;
  DSA_REQUIRE(src && dst, "cache_append: %s rows and cache must both be given or both be NULL", what);
  DSA_REQUIRE(valid_dtype(sdt) && valid_dtype(ddt), "cache_append: invalid %s dtype", what);
  DSA_SUPPORT(sdt == DSA_F32 || sdt == DSA_BF16, "cache_append: %s rows must be f32 or bf16", what);
  DSA_SUPPORT(ddt == sdt || ddt == DSA_FP8_E4M3FN,
              "cache_append: %s rows of dtype %d cannot go into a cache of dtype %d", what, (int)sdt, (int)ddt);
  DSA_SUPPORT(width >= 8 && width <= 1024 && width % 8 == 0,
              "cache_append: %s width %d must be a multiple of 8 in 8..1024", what, width);
  DSA_REQUIRE(ddt != DSA_FP8_E4M3FN || scale != nullptr, "cache_append: an fp8 %s cache needs its scale", what);
  DSA_REQUIRE(aligned(src, 16) && aligned(dst, 16) && (!scale || aligned(scale, 4)),
              "cache_append: %s arrays must be 16-byte aligned", what);
  return DSA_OK;
}

}  // namespace

extern "C" {

const char* dsa_status_string(dsa_status_t s) {
  switch (s) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_ARGUMENT: return "DSA_ERR_INVALID_ARGUMENT";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED";
    case DSA_ERR_WORKSPACE_TOO_SMALL: return "DSA_ERR_WORKSPACE_TOO_SMALL";
    case DSA_ERR_HIP: return "DSA_ERR_HIP";
  }
  return "DSA_ERR_UNKNOWN";
}

const char* dsa_last_error(void) { return g_err; }

int32_t dsa_abi_version(void) { return DSA_ABI_VERSION; }

dsa_status_t dsa_indexer_scores(const dsa_batch_t* b, const void* q, dsa_dtype_t q_dtype, const float* w,
                                const void* k_cache, dsa_dtype_t k_dtype, const float* k_scale, int32_t n_heads,
                                int32_t head_dim, float* scores, int64_t scores_ld, void* stream) {
  DSA_TRY(check_indexer(b, q, q_dtype, w, k_cache, k_dtype, k_scale, n_heads, head_dim, scores, scores_ld));
  DSA_TRY(check_device());
  uint32_t* dbg = nullptr;
  DSA_TRY(debug_word(&dbg));
  IndexerParams p{};
  p.dbg = dbg;
  p.seq_lens = b->seq_lens;
  p.page_table = b->page_table;
  p.q = q;
  p.w = w;
  p.k_cache = k_cache;
  p.k_scale = k_dtype == DSA_FP8_E4M3FN ? k_scale : nullptr;
  p.num_slots = b->num_slots;
  p.scores = scores;
  p.ld = scores_ld;
  p.B = b->batch;
  p.Q = b->q_per_seq;
  p.max_seq_len = b->max_seq_len;
  p.P = b->page_size;
  p.maxP = b->max_pages_per_seq;
  p.Hi = n_heads;
  p.Di = head_dim;
  return launched(launch_indexer(p, q_dtype, k_dtype, (hipStream_t)stream), "indexer");
}

size_t dsa_topk_workspace_size(const dsa_batch_t* b, int32_t k) {
  if (!b || b->batch < 1 || b->q_per_seq < 1 || b->max_seq_len < 1 || k < 1) return 0;
  return topk_workspace_bytes((int64_t)b->batch * b->q_per_seq, b->max_seq_len, k);
}

dsa_status_t dsa_topk(const dsa_batch_t* b, const float* scores, int64_t scores_ld, int32_t k, int32_t* topk_idx,
                      int32_t* topk_slots, void* workspace, size_t workspace_bytes, void* stream) {
  DSA_TRY(check_topk(b, scores, scores_ld, k, topk_idx));
  DSA_REQUIRE(!topk_slots || aligned(topk_slots, 4), "topk: topk_slots must be 4-byte aligned");
  const size_t need = topk_workspace_bytes((int64_t)b->batch * b->q_per_seq, b->max_seq_len, k);
  if (workspace_bytes < need || (need > 0 && workspace == nullptr))
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "topk: workspace needs %zu bytes (got %zu)", need, workspace_bytes);
  DSA_REQUIRE(need == 0 || aligned(workspace, 256), "topk: workspace must be 256-byte aligned");
  DSA_TRY(check_device());
  uint32_t* dbg = nullptr;
  DSA_TRY(debug_word(&dbg));
  TopkParams p{scores, scores_ld, b->seq_lens, b->page_table, topk_idx, topk_slots,
               b->q_per_seq, k, b->page_size, b->max_pages_per_seq, 0, 0, nullptr, nullptr, 0,
               b->num_slots, b->max_seq_len, 0, 0, dbg};
  return launched(launch_topk(p, b->batch * b->q_per_seq, b->max_seq_len, workspace, (hipStream_t)stream),
                  "top-k");
}

dsa_status_t dsa_page_map(const dsa_batch_t* b, const int32_t* topk_idx, int32_t k, int32_t* slots, void* stream) {
  DSA_TRY(check_batch(b));
  DSA_REQUIRE(topk_idx && slots, "page_map: topk_idx and slots must be non-NULL");
  DSA_REQUIRE(k >= 1, "page_map: k must be >= 1");
  DSA_REQUIRE(aligned(topk_idx, 4) && aligned(slots, 4), "page_map: arrays must be 4-byte aligned");
  DSA_TRY(check_device());
  uint32_t* dbg = nullptr;
  DSA_TRY(debug_word(&dbg));
  const int64_t total = (int64_t)b->batch * b->q_per_seq * k;
  return launched(launch_page_map(topk_idx, total, k, b->q_per_seq, b->page_table, b->max_pages_per_seq,
                                  b->page_size, slots, b->seq_lens, b->num_slots, dbg, (hipStream_t)stream),
                  "page map");
}

int32_t dsa_sparse_mla_default_split(int32_t batch, int32_t q_per_seq, int32_t n_heads, int32_t k,
                                     dsa_dtype_t kv_dtype) {
  if (batch < 1 || q_per_seq < 1 || k < 1) return 1;
  return effective_split((int64_t)batch * q_per_seq, n_heads, k, 0, DSA_BF16, kv_dtype);
}

size_t dsa_sparse_mla_workspace_size(int32_t batch, int32_t q_per_seq, int32_t n_heads, int32_t k, int32_t n_split,
                                     dsa_dtype_t q_dtype, dsa_dtype_t kv_dtype) {
  if (batch < 1 || q_per_seq < 1 || n_heads < 1 || k < 1) return 0;
  const int64_t rows = (int64_t)batch * q_per_seq;
  return mla_ws(rows, n_heads, effective_split(rows, n_heads, k, n_split, q_dtype, kv_dtype)).total;
}

dsa_status_t dsa_sparse_mla_decode(int32_t batch, int32_t q_per_seq, const void* q, dsa_dtype_t q_dtype,
                                   const void* kv_cache, dsa_dtype_t kv_dtype, const float* kv_scale,
                                   int64_t num_slots, const int32_t* slots, int32_t k, int32_t n_heads,
                                   float sm_scale, float* out, float* lse, int32_t n_split, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  DSA_TRY(check_mla(batch, q_per_seq, q, q_dtype, kv_cache, kv_dtype, kv_scale, num_slots, slots, k, n_heads,
                    sm_scale, out, lse, n_split));
  const int64_t rows = (int64_t)batch * q_per_seq;
  const int32_t ns = effective_split(rows, n_heads, k, n_split, q_dtype, kv_dtype);
  const MlaWs w = mla_ws(rows, n_heads, ns);
  if (workspace_bytes < w.total || (w.total > 0 && workspace == nullptr))
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "mla: workspace needs %zu bytes (got %zu)", w.total, workspace_bytes);
  DSA_TRY(check_device());
  uint32_t* dbg = nullptr;
  DSA_TRY(debug_word(&dbg));
  return run_mla(rows, q_per_seq, q, q_dtype, kv_cache, kv_dtype, kv_scale, num_slots, slots, k, n_heads, sm_scale, out, lse, ns,
                 workspace, workspace_bytes, dbg, (hipStream_t)stream);
}

dsa_status_t dsa_mla_combine(int32_t rows, int32_t n_heads, int32_t n_split, const float* part_o, const float* part_m,
                             const float* part_l, float* out, float* lse, void* stream) {
  DSA_REQUIRE(rows >= 0 && n_heads >= 1 && n_split >= 1, "combine: rows >= 0, n_heads >= 1, n_split >= 1");
  DSA_SUPPORT(n_split <= 1024, "combine: n_split=%d above the supported maximum 1024", n_split);
  DSA_REQUIRE(part_o && part_m && part_l && out, "combine: partial arrays and out must be non-NULL");
  DSA_REQUIRE(aligned(part_o, 16) && aligned(out, 16) && aligned(part_m, 4) && aligned(part_l, 4) &&
                  (!lse || aligned(lse, 4)),
              "combine: part_o and out 16-byte aligned, others 4-byte aligned");
  DSA_TRY(check_device());
  CombineParams c{part_o, part_m, part_l, out, lse, rows, n_heads, n_split};
  return launched(launch_combine(c, (hipStream_t)stream), "combine");
}

namespace {

struct StepWs {
  int64_t ld;
  size_t topk_off, scores_off, idx_off, slots_off, mla_off, total;
  int32_t ns;
  int32_t q_block;   // query rows per sequence scored and ranked together (q_per_seq: one block)
};

constexpr size_t kPrefillBlockBytes = (size_t)72 << 20;   // scores per block (stays in the 256 MB cache)

StepWs step_ws(const dsa_decode_step_args_t* a) {
  StepWs w{};
  const dsa_batch_t& b = a->batch;
  const int64_t rows = (int64_t)b.batch * b.q_per_seq;
  w.ld = b.max_seq_len;
  // chunked prefill: blocks of rows whose scores fit kPrefillBlockBytes (or the caller's size)
  w.q_block = b.q_per_seq;
  if (!a->debug_scores && indexer_uses_prefill(a->idx_heads, a->idx_dim, b.q_per_seq, b.page_size, a->q_idx_dtype,
                                               a->k_dtype)) {
    int64_t qb = a->prefill_rows_per_block;
    if (qb <= 0) qb = (int64_t)(kPrefillBlockBytes / ((size_t)b.batch * w.ld * sizeof(float)));
    if (qb < b.q_per_seq) {
      qb = qb / 16 * 16;
      if (qb < 16) qb = 16;
      if (qb < b.q_per_seq) w.q_block = (int32_t)qb;
    }
  }
  const int64_t block_rows = (int64_t)b.batch * w.q_block;
  const int32_t last_q = b.q_per_seq % w.q_block;
  size_t off = 0;
  w.topk_off = off;   // top-k candidates of long rows (for the largest need of a block)
  size_t topk_bytes = topk_workspace_bytes(block_rows, b.max_seq_len, a->top_k);
  if (last_q) {
    const size_t last_bytes = topk_workspace_bytes((int64_t)b.batch * last_q, b.max_seq_len, a->top_k);
    if (last_bytes > topk_bytes) topk_bytes = last_bytes;
  }
  off += align_up(topk_bytes, 256);
  w.scores_off = off;
  if (!a->debug_scores) off += align_up((size_t)block_rows * w.ld * sizeof(float), 256);
  w.idx_off = off;
  if (!a->debug_idx) off += align_up((size_t)rows * a->top_k * sizeof(int32_t), 256);
  w.slots_off = off;
  if (!a->debug_slots) off += align_up((size_t)rows * a->top_k * sizeof(int32_t), 256);
  w.mla_off = off;
  w.ns = effective_split(rows, a->mla_heads, a->top_k, a->n_split, a->q_mla_dtype, a->kv_dtype);
  off += mla_ws(rows, a->mla_heads, w.ns).total;
  w.total = off;
  return w;
}

}  // namespace

size_t dsa_decode_step_workspace_size(const dsa_decode_step_args_t* a) {
  if (!a || a->batch.batch < 1 || a->batch.q_per_seq < 1 || a->top_k < 1 || a->mla_heads < 1 ||
      a->batch.max_seq_len < 1)
    return 0;
  return step_ws(a).total;
}

}  // extern "C"

namespace {

// Argument checks of the fused step (everything but the workspace).
dsa_status_t check_step(const dsa_decode_step_args_t* a) {
  DSA_REQUIRE(a != nullptr, "decode_step: args is NULL");
  const dsa_batch_t* b = &a->batch;
  DSA_TRY(check_indexer(b, a->q_idx, a->q_idx_dtype, a->w, a->k_cache, a->k_dtype, a->k_scale, a->idx_heads,
                        a->idx_dim, a->debug_scores ? a->debug_scores : (const float*)16, b->max_seq_len));
  DSA_TRY(check_topk(b, (const float*)16, b->max_seq_len, a->top_k, (const int32_t*)16));
  DSA_TRY(check_mla(b->batch, b->q_per_seq, a->q_mla, a->q_mla_dtype, a->kv_cache, a->kv_dtype, a->kv_scale,
                    b->num_slots, (const int32_t*)16, a->top_k, a->mla_heads, a->sm_scale, a->out, a->lse,
                    a->n_split));
  DSA_REQUIRE(a->prefill_rows_per_block >= 0, "decode_step: prefill_rows_per_block must be >= 0 (got %d)",
              a->prefill_rows_per_block);
  DSA_REQUIRE((!a->debug_idx || aligned(a->debug_idx, 4)) && (!a->debug_slots || aligned(a->debug_slots, 4)),
              "decode_step: debug arrays must be 4-byte aligned");
  return DSA_OK;
}

// The launches of the fused step into a checked workspace of step_ws(a).total bytes or more.
dsa_status_t launch_step(const dsa_decode_step_args_t* a, const StepWs& w, void* workspace, size_t workspace_bytes,
                         hipStream_t s) {
  const dsa_batch_t* b = &a->batch;
  uint8_t* ws = (uint8_t*)workspace;
  float* scores = a->debug_scores ? a->debug_scores : (float*)(ws + w.scores_off);
  int32_t* idx = a->debug_idx ? a->debug_idx : (int32_t*)(ws + w.idx_off);
  int32_t* slots = a->debug_slots ? a->debug_slots : (int32_t*)(ws + w.slots_off);

  uint32_t* dbg = nullptr;
  DSA_TRY(debug_word(&dbg));
  IndexerParams ip{};
  ip.dbg = dbg;
  ip.seq_lens = b->seq_lens;
  ip.page_table = b->page_table;
  ip.q = a->q_idx;
  ip.w = a->w;
  ip.k_cache = a->k_cache;
  ip.k_scale = a->k_dtype == DSA_FP8_E4M3FN ? a->k_scale : nullptr;
  ip.num_slots = b->num_slots;
  ip.scores = scores;
  ip.ld = w.ld;
  ip.B = b->batch;
  ip.Q = b->q_per_seq;
  ip.max_seq_len = b->max_seq_len;
  ip.P = b->page_size;
  ip.maxP = b->max_pages_per_seq;
  ip.Hi = a->idx_heads;
  ip.Di = a->idx_dim;
  TopkParams tp{scores, w.ld, b->seq_lens, b->page_table, idx, slots,
                b->q_per_seq, a->top_k, b->page_size, b->max_pages_per_seq, 0, 0, nullptr, nullptr, 0,
                b->num_slots, b->max_seq_len, 0, 0, dbg};
  // rows in blocks of q_block per sequence, each block's scores in the same buffer
  for (int32_t q0 = 0; q0 < b->q_per_seq; q0 += w.q_block) {
    const int32_t qn = b->q_per_seq - q0 < w.q_block ? b->q_per_seq - q0 : w.q_block;
    ip.q_begin = tp.q_begin = q0;
    ip.q_count = tp.q_count = qn;
    DSA_TRY(launched(launch_indexer(ip, a->q_idx_dtype, a->k_dtype, s), "indexer"));
    DSA_TRY(launched(launch_topk(tp, b->batch * qn, b->max_seq_len, ws + w.topk_off, s), "top-k"));
  }

  const int64_t rows = (int64_t)b->batch * b->q_per_seq;
  const size_t mla_bytes = workspace_bytes - w.mla_off;
  return run_mla(rows, b->q_per_seq, a->q_mla, a->q_mla_dtype, a->kv_cache, a->kv_dtype, a->kv_scale, b->num_slots, slots, a->top_k,
                 a->mla_heads, a->sm_scale, a->out, a->lse, w.ns, ws + w.mla_off, mla_bytes, dbg, s);
}

// Scratch memory of dsa_decode_step_noalloc: one copy per device, zero-initialised when the
// library is loaded on that device and kept until the process ends.  Host code reaches it
// only through the device address hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = (size_t)128 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
std::atomic<void*> g_scratch[kMaxDevices];

dsa_status_t scratch_of_current_device(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(DSA_ERR_UNSUPPORTED, "device ordinal %d out of range", dev);
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(DSA_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
    g_scratch[dev].store(p, std::memory_order_release);   // (a racing first call stores the same address)
  }
  *ptr = p;
  return DSA_OK;
}

}  // namespace

extern "C" {

dsa_status_t dsa_decode_step(const dsa_decode_step_args_t* a, void* workspace, size_t workspace_bytes, void* stream) {
  DSA_TRY(check_step(a));
  const StepWs w = step_ws(a);
  if (workspace_bytes < w.total || (w.total > 0 && workspace == nullptr))
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "decode_step: workspace needs %zu bytes (got %zu)", w.total,
                workspace_bytes);
  DSA_REQUIRE(w.total == 0 || aligned(workspace, 256), "decode_step: workspace must be 256-byte aligned");
  DSA_TRY(check_device());
  return launch_step(a, w, workspace, workspace_bytes, (hipStream_t)stream);
}

size_t dsa_decode_step_noalloc_max_bytes(void) { return kScratchBytes; }

dsa_status_t dsa_decode_step_noalloc(const dsa_decode_step_args_t* a, void* stream) {
  DSA_TRY(check_step(a));
  const StepWs w = step_ws(a);
  if (w.total > kScratchBytes)
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL,
                "decode_step_noalloc: the step needs %zu bytes of scratch, above the library's fixed %zu "
                "(use dsa_decode_step with a caller workspace)", w.total, kScratchBytes);
  DSA_TRY(check_device());
  void* ptr = nullptr;
  DSA_TRY(scratch_of_current_device(&ptr));
  return launch_step(a, w, ptr, kScratchBytes, (hipStream_t)stream);
}

namespace {

struct UpWs {
  size_t v_bytes, part_bytes, total;
  int32_t ksplit;
};

UpWs up_ws(int32_t R, int32_t H, int32_t Dv, int32_t Dm) {
  UpWs w{};
  w.ksplit = up_proj_ksplit(R, Dm, H * Dv);
  w.v_bytes = align_up((size_t)R * H * Dv * sizeof(float), 256);
  w.part_bytes = w.ksplit > 1 ? align_up((size_t)w.ksplit * R * Dm * sizeof(float), 256) : 0;
  w.total = w.v_bytes + w.part_bytes;
  return w;
}

}  // namespace

size_t dsa_latent_up_projection_workspace_size(int32_t rows, int32_t n_heads, int32_t v_dim, int32_t d_model) {
  if (rows < 1 || n_heads < 1 || v_dim < 1 || d_model < 1) return 0;
  return up_ws(rows, n_heads, v_dim, d_model).total;
}

dsa_status_t dsa_latent_up_projection(int32_t rows, int32_t n_heads, int32_t v_dim, int32_t d_model,
                                      const float* attn_out, const void* w_uv, const void* w_o, float* y,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  DSA_REQUIRE(rows >= 1 && n_heads >= 1 && v_dim >= 1 && d_model >= 1,
              "up_projection: rows, n_heads, v_dim and d_model must be >= 1");
  DSA_REQUIRE(attn_out && w_uv && w_o && y, "up_projection: attn_out, w_uv, w_o and y must be non-NULL");
  DSA_SUPPORT(n_heads <= 128 && v_dim % 32 == 0 && v_dim <= 1024 && d_model % 16 == 0 && d_model <= 65536 &&
                  rows <= 1000000,
              "up_projection: n_heads=%d v_dim=%d d_model=%d rows=%d outside the supported set (n_heads <= 128, "
              "v_dim a multiple of 32 up to 1024, d_model a multiple of 16 up to 65536, rows <= 1000000)",
              n_heads, v_dim, d_model, rows);
  DSA_REQUIRE(aligned(attn_out, 16) && aligned(w_uv, 16) && aligned(w_o, 16) && aligned(y, 4),
              "up_projection: attn_out, w_uv and w_o must be 16-byte aligned, y 4-byte aligned");
  const UpWs w = up_ws(rows, n_heads, v_dim, d_model);
  if (workspace_bytes < w.total || workspace == nullptr)
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "up_projection: workspace needs %zu bytes (got %zu)", w.total,
                workspace_bytes);
  DSA_REQUIRE(aligned(workspace, 256), "up_projection: workspace must be 256-byte aligned");
  DSA_TRY(check_device());
  UpProjParams p{};
  p.o = attn_out;
  p.w_uv = w_uv;
  p.w_o = w_o;
  p.v = (float*)workspace;
  p.part = w.ksplit > 1 ? (float*)((uint8_t*)workspace + w.v_bytes) : nullptr;
  p.y = y;
  p.R = rows;
  p.H = n_heads;
  p.Dv = v_dim;
  p.Dm = d_model;
  p.ksplit = w.ksplit;
  return launched(launch_up_proj(p, (hipStream_t)stream), "up-projection");
}

dsa_status_t dsa_kv_cache_append(const dsa_batch_t* b, const void* kv_new, dsa_dtype_t kv_new_dtype, void* kv_cache,
                                 dsa_dtype_t kv_dtype, float* kv_scale, const void* k_new, dsa_dtype_t k_new_dtype,
                                 int32_t head_dim, void* k_cache, dsa_dtype_t k_dtype, float* k_scale,
                                 void* stream) {
  DSA_TRY(check_batch(b));
  DSA_REQUIRE(kv_new || k_new, "cache_append: no latent rows and no indexer keys given");
  DSA_TRY(check_append_side("latent", kv_new, kv_new_dtype, kv_cache, kv_dtype, kv_scale, (int32_t)kRowDim));
  DSA_TRY(check_append_side("key", k_new, k_new_dtype, k_cache, k_dtype, k_scale, head_dim));
  DSA_TRY(check_device());
  AppendParams p{};
  p.seq_lens = b->seq_lens;
  p.page_table = b->page_table;
  p.kv_src = kv_new;
  p.kv_dst = kv_new ? kv_cache : nullptr;
  p.kv_scale = kv_dtype == DSA_FP8_E4M3FN ? kv_scale : nullptr;
  p.k_src = k_new;
  p.k_dst = k_new ? k_cache : nullptr;
  p.k_scale = k_dtype == DSA_FP8_E4M3FN ? k_scale : nullptr;
  p.rows = (int64_t)b->batch * b->q_per_seq;
  p.Q = b->q_per_seq;
  p.P = b->page_size;
  p.maxP = b->max_pages_per_seq;
  p.kv_width = (int32_t)kRowDim;
  p.k_width = head_dim;
  p.kv_src_dtype = kv_new_dtype;
  p.kv_dst_dtype = kv_dtype;
  p.k_src_dtype = k_new_dtype;
  p.k_dst_dtype = k_dtype;
  p.num_slots = b->num_slots;
  p.max_seq_len = b->max_seq_len;
  DSA_TRY(debug_word(&p.dbg));
  return launched(launch_cache_append(p, (hipStream_t)stream), "cache append");
}

dsa_status_t dsa_debug_check(uint32_t* flags, void* stream) {
  if (flags) *flags = 0u;
#ifdef DSA_DEBUG
  DSA_TRY(check_device());
  uint32_t* dbg = nullptr;
  DSA_TRY(debug_word(&dbg));
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "debug_check: stream synchronisation failed: %s", hipGetErrorString(e));
  uint32_t word = 0u;
  const uint32_t zero = 0u;
  e = hipMemcpy(&word, dbg, sizeof(word), hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemcpy(dbg, &zero, sizeof(zero), hipMemcpyHostToDevice);
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "debug_check: reading the error word failed: %s", hipGetErrorString(e));
  if (flags) *flags = word;
  if (word == 0u) return DSA_OK;
  return fail(DSA_ERR_INVALID_ARGUMENT, "debug_check: violated data preconditions (flags 0x%x):%s%s%s%s%s", word,
              word & kDbgSeqLen ? " seq_lens outside [q_per_seq, max_seq_len];" : "",
              word & kDbgPageId ? " page-table entry outside [0, num_slots / page_size);" : "",
              word & kDbgSlot ? " slot outside [-1, num_slots);" : "",
              word & kDbgNanScore ? " NaN score;" : "",
              word & kDbgTopkIndex ? " top-k index outside [-1, seq_lens[b]);" : "");
#else
  (void)stream;
  return fail(DSA_ERR_UNSUPPORTED, "debug_check: this library was built without DSA_DEBUG (load libdsa_debug.so)");
#endif
}

int32_t dsa_debug_enabled(void) {
#ifdef DSA_DEBUG
  return 1;
#else
  return 0;
#endif
}

}  // extern "C"
