/*
 * dsa.h - C ABI of the DeepSeek-Sparse-Attention (DSA) decode path on MI355X (gfx950).
 *
 * The path has the three kernel groups named in "GLM-52 Runs on RTX 4090" (section "how did
 * he do it") and in the renning22/glm-5.2-4090 README (section "how it works"): the
 * lightning-indexer GEMM, the top-k + page-mapping transform, and MLA sparse decode; plus the
 * split-k merge of the decode partials and one call that runs the whole step.
 *
 * Conventions shared by every call
 *   - Array arguments are DEVICE pointers (hipMalloc'd or torch CUDA tensors), row-major and
 *     densely packed, 16-byte aligned unless stated.  Struct arguments live in host memory.
 *   - The caller owns every buffer, workspaces included.  The library never allocates, frees
 *     or keeps a pointer after a call returns.  Its only global state is a per-device cache
 *     of "is this a gfx950" answers and a thread-local error string.
 *   - Every call enqueues work on `stream` (a hipStream_t; NULL is the default stream) and
 *     returns without synchronising and without reading device memory on the host.
 *     Per-sequence lengths therefore stay on the device; host-side sizes (max_seq_len, k)
 *     size the grids.  No call records a memset, so every call may be captured in a HIP graph.
 *   - Arguments are validated before anything is enqueued: a status other than DSA_OK means
 *     nothing was launched.  dsa_last_error() then describes the problem.  A launch failure
 *     returns DSA_ERR_HIP.  A device that is not gfx950 returns DSA_ERR_UNSUPPORTED.
 *   - Data preconditions that would need a device read to check are the caller's duty:
 *     page ids < num_slots / page_size, q_per_seq <= seq_lens[b] <= max_seq_len, slot ids in
 *     [-1, num_slots), no NaN scores, top-k indices in [-1, seq_lens[b]).  libdsa.so does not
 *     check them.  libdsa_debug.so, the same sources built with DSA_DEBUG defined, checks them
 *     on the device (dsa_debug_check below).
 *
 * Notation: B = batch, Q = query tokens per sequence, L_b = seq_lens[b] = cached tokens of
 * sequence b INCLUDING its Q new tokens, pos(b,i) = L_b - Q + i is the position of query i
 * (it sees tokens t <= pos(b,i)), P = page_size,
 * slot(b,t) = page_table[b * max_pages_per_seq + t / P] * P + t % P.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 1

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARGUMENT = 1,   /* NULL, negative or inconsistent sizes, misalignment */
  DSA_ERR_UNSUPPORTED = 2,        /* valid request outside the supported set, or not gfx950 */
  DSA_ERR_WORKSPACE_TOO_SMALL = 3,
  DSA_ERR_HIP = 4                 /* a HIP runtime call or a launch failed */
} dsa_status_t;

typedef enum {
  DSA_F32 = 0,
  DSA_BF16 = 1,
  DSA_FP8_E4M3FN = 2              /* OCP e4m3fn codes; always paired with a per-token f32 scale */
} dsa_dtype_t;

/* A ragged, paged batch of sequences (host struct; the two arrays are device pointers). */
typedef struct {
  int32_t batch;                  /* B >= 1 */
  int32_t q_per_seq;              /* Q >= 1 (1 decode, 2 speculative verify, 4096 prefill chunk) */
  int32_t max_seq_len;            /* host bound >= every seq_lens[b]; sizes grids only */
  int32_t page_size;              /* P >= 1 */
  int32_t max_pages_per_seq;      /* row stride of page_table, >= ceil(max_seq_len / P) */
  int64_t num_slots;              /* cache rows in the pool (pages * P) */
  const int32_t *seq_lens;        /* [B] L_b */
  const int32_t *page_table;      /* [B, max_pages_per_seq] physical page ids */
} dsa_batch_t;

/*
 * Lightning indexer ("GLM-52 Runs on RTX 4090", "how did he do it": the lightning-indexer GEMM).
 *   scores[b,i,t] = sum_h w[b,i,h] * max(0, q[b,i,h,:] . k~[slot(b,t),:])   for t <= pos(b,i)
 *   scores[b,i,t] = -inf                                                   for pos(b,i) < t < L_b
 * Columns t >= L_b are not written.  k~ is the key row; for fp8 keys k~ = k_scale[slot] * code,
 * and because the scale is positive it is applied after the ReLU and the head sum.
 *   q        [B, Q, n_heads, head_dim]  f32 or bf16
 *   w        [B, Q, n_heads]            f32 head weights
 *   k_cache  [num_slots, head_dim]      f32, bf16 or fp8 (paged by the same table as the latent cache)
 *   k_scale  [num_slots] f32            required for fp8 keys, NULL otherwise
 *   scores   [B, Q, scores_ld] f32      scores_ld >= max_seq_len
 * Supported: n_heads in 1..128 and head_dim in 1..256 (any dtype pair; vector path), with the
 * matrix-core path taken for n_heads = 64, head_dim = 128, bf16 q, bf16 or fp8 keys.
 */
dsa_status_t dsa_indexer_scores(const dsa_batch_t *batch,
                                const void *q, dsa_dtype_t q_dtype,
                                const float *w,
                                const void *k_cache, dsa_dtype_t k_dtype, const float *k_scale,
                                int32_t n_heads, int32_t head_dim,
                                float *scores, int64_t scores_ld,
                                void *stream);

/*
 * Top-k per query row ("how did he do it": the top-k transform).
 * Row (b,i) ranks its pos(b,i)+1 visible scores by (score descending, token index ascending):
 * equal scores go to the lower token index, and -0.0 equals +0.0.  The min(k, pos+1) winners
 * are written to topk_idx[b,i,:] in ascending token order, padded with -1.
 * If topk_slots is not NULL the page map is fused in (the README's fused page-mapping
 * transform): topk_slots[b,i,j] = slot(b, topk_idx[b,i,j]), -1 for padding.
 *   scores     [B, Q, scores_ld] f32 (only columns t <= pos(b,i) are read; no NaN)
 *   topk_idx   [B, Q, k] int32;  topk_slots [B, Q, k] int32 or NULL
 * Supported: 1 <= k <= 8192, max_seq_len <= 262144.  Up to 128 rows of 64K+
 * columns are ranked in two passes whose candidates (score, column) live in the workspace of
 * dsa_topk_workspace_size() bytes, 256-byte aligned, no initial contents; workspace may be
 * NULL when that size is 0.
 */
dsa_status_t dsa_topk(const dsa_batch_t *batch, const float *scores, int64_t scores_ld, int32_t k,
                      int32_t *topk_idx, int32_t *topk_slots,
                      void *workspace, size_t workspace_bytes, void *stream);
size_t dsa_topk_workspace_size(const dsa_batch_t *batch, int32_t k);

/*
 * Page map ("how did he do it": the page-mapping transform from logical tokens to physical
 * KV-cache slots): slots[b,i,j] = slot(b, topk_idx[b,i,j]); -1 stays -1.
 *   topk_idx [B, Q, k] int32 -> slots [B, Q, k] int32
 */
dsa_status_t dsa_page_map(const dsa_batch_t *batch, const int32_t *topk_idx, int32_t k,
                          int32_t *slots, void *stream);

/*
 * Sparse MLA decode ("how did he do it": MLA sparse decode; Show HN "Chay GLM 5.2 tren may
 * tinh cham", main features: 576 values per cached token, 64 heads and no GQA, weight
 * absorption so the query meets the compressed rows directly).
 * For each query row r = b*Q + i and head h, over the selected slots s = slots[r, j] != -1:
 *   z_s = sm_scale * (q[r,h,:] . c~[s,:])          (576 values)
 *   out[r,h,:] = sum_s softmax(z)_s * c~[s, 0:512]  (V is the first 512 values of the row)
 *   lse[r,h]   = log sum_s exp(z_s)                 (natural log)
 * c~ = kv_cache row, or kv_scale[s] * code for fp8.  A row with no valid slot gives out = 0
 * and lse = -inf.  On the matrix cores (bf16 q) the logits are exact products summed in f32;
 * the softmax weights enter the weighted sum of V as bf16 (fp8 rows: with the row's scale
 * folded in), and for bf16 rows the output is divided by the sum of those rounded weights, so
 * it stays a convex combination of the selected rows; lse uses the unrounded sum.
 *   q         [B, Q, n_heads, 576] f32 or bf16
 *   kv_cache  [num_slots, 576] f32, bf16 or fp8;  kv_scale [num_slots] f32 for fp8, else NULL
 *   slots     [B, Q, k] int32 (any order; -1 entries are skipped)
 *   out       [B, Q, n_heads, 512] f32;  lse [B, Q, n_heads] f32 or NULL
 *   n_split   chunks of the selected set processed in parallel and merged (split-k);
 *             0 picks a value for the GPU's 256 compute units.
 * Supported: bf16 q with bf16 or fp8 rows and n_heads in {16, 32, 48, 64} (matrix cores);
 * f32 q with any row dtype and n_heads in 1..128 (vector path, n_split ignored).
 * 1 <= k <= 8192.  The workspace holds the split partials (dsa_sparse_mla_workspace_size).
 */
dsa_status_t dsa_sparse_mla_decode(int32_t batch, int32_t q_per_seq,
                                   const void *q, dsa_dtype_t q_dtype,
                                   const void *kv_cache, dsa_dtype_t kv_dtype, const float *kv_scale,
                                   int64_t num_slots,
                                   const int32_t *slots, int32_t k,
                                   int32_t n_heads, float sm_scale,
                                   float *out, float *lse, int32_t n_split,
                                   void *workspace, size_t workspace_bytes, void *stream);
size_t dsa_sparse_mla_workspace_size(int32_t batch, int32_t q_per_seq, int32_t n_heads, int32_t k,
                                     int32_t n_split, dsa_dtype_t q_dtype, dsa_dtype_t kv_dtype);
/* The n_split that dsa_sparse_mla_decode uses when passed 0: about one workgroup per compute
 * unit; fp8 rows keep at most 2048 selected rows per chunk; bf16 rows with at most 16 (query
 * row, 16-head group) pairs in all take chunks of 128 selected rows (one workgroup per row,
 * head group and chunk). */
int32_t dsa_sparse_mla_default_split(int32_t batch, int32_t q_per_seq, int32_t n_heads, int32_t k,
                                     dsa_dtype_t kv_dtype);

/*
 * Split-k merge of softmax partials (the step that joins the chunks of the selected set).
 * For each row r and head h, over chunks j with l[r,j,h] > 0:
 *   M = max_j m_j,  a_j = exp(m_j - M) * l_j,
 *   out[r,h,:] = sum_j a_j * o[r,j,h,:] / sum_j a_j,   lse[r,h] = M + log sum_j a_j.
 * m is in natural-log units.  If no chunk has l > 0: out = 0, lse = -inf.  The kernel keeps
 * running (max, sum) pairs over fixed groups of chunks and merges them in a fixed order, which
 * equals the formula up to rounding and makes results deterministic.
 *   part_o [rows, n_split, n_heads, 512] f32 (each chunk normalised by its own l)
 *   part_m, part_l [rows, n_split, n_heads] f32
 *   out [rows, n_heads, 512] f32;  lse [rows, n_heads] f32 or NULL
 */
dsa_status_t dsa_mla_combine(int32_t rows, int32_t n_heads, int32_t n_split,
                             const float *part_o, const float *part_m, const float *part_l,
                             float *out, float *lse, void *stream);

/*
 * The whole decode step on one stream: indexer -> top-k with the fused page map -> sparse MLA
 * (-> split-k merge), with no host synchronisation.  With many query rows per sequence (a
 * chunked-prefill step: bf16 keys, q_per_seq >= 16) the rows are scored and ranked in blocks
 * that reuse one score buffer small enough to stay in the 256 MB Infinity Cache, instead of
 * writing the whole [B,Q,max_seq_len] score array at once.
 * Optional debug outputs: when debug_scores / debug_idx / debug_slots are not NULL, the step
 * keeps its intermediate [B,Q,max_seq_len] scores (ld = max_seq_len), [B,Q,top_k] indices and
 * slots there instead of in the workspace, so a caller can inspect exactly what was used.
 */
typedef struct {
  dsa_batch_t batch;
  /* indexer */
  const void *q_idx;     dsa_dtype_t q_idx_dtype;   /* [B,Q,idx_heads,idx_dim] */
  const float *w;                                   /* [B,Q,idx_heads] */
  const void *k_cache;   dsa_dtype_t k_dtype;       /* [num_slots, idx_dim] */
  const float *k_scale;                             /* [num_slots] for fp8 keys, else NULL */
  int32_t idx_heads, idx_dim;
  /* selection */
  int32_t top_k;
  /* sparse MLA */
  const void *q_mla;     dsa_dtype_t q_mla_dtype;   /* [B,Q,mla_heads,576] */
  const void *kv_cache;  dsa_dtype_t kv_dtype;      /* [num_slots,576] */
  const float *kv_scale;                            /* [num_slots] for fp8 rows, else NULL */
  int32_t mla_heads;
  float sm_scale;
  int32_t n_split;                                  /* 0 = automatic */
  float *out;                                       /* [B,Q,mla_heads,512] */
  float *lse;                                       /* [B,Q,mla_heads] or NULL */
  /* optional debug outputs (device pointers or NULL) */
  float *debug_scores;                              /* [B,Q,max_seq_len] */
  int32_t *debug_idx;                               /* [B,Q,top_k] */
  int32_t *debug_slots;                             /* [B,Q,top_k] */
  /* chunked prefill: rows per sequence whose scores are formed and ranked together (rounded
   * down to a multiple of 16, at least 16; 0 = automatic, about 72 MiB of scores per block;
   * ignored with debug_scores or when the many-rows indexer does not apply) */
  int32_t prefill_rows_per_block;
} dsa_decode_step_args_t;

dsa_status_t dsa_decode_step(const dsa_decode_step_args_t *args,
                             void *workspace, size_t workspace_bytes, void *stream);
size_t dsa_decode_step_workspace_size(const dsa_decode_step_args_t *args);

/*
 * The fused step for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same launches and results as
 * dsa_decode_step, with the workspace taken from a scratch buffer of fixed size that the
 * library holds on every device it runs on (dsa_decode_step_noalloc_max_bytes() = 128 MiB,
 * held until the process ends).  The call allocates and frees nothing.
 *   - A step whose workspace (dsa_decode_step_workspace_size) exceeds the scratch size is
 *     rejected with DSA_ERR_WORKSPACE_TOO_SMALL before anything is enqueued; such steps (a
 *     4096-row prefill chunk, whose score rows alone take 1 GiB) need dsa_decode_step.
 *   - Every call on one GPU uses that GPU's single scratch buffer, whose contents carry over
 *     between calls (no call relies on them).  Calls that may overlap on one GPU (several
 *     streams or threads) race on it: the caller must order them, e.g. on one stream.
 */
dsa_status_t dsa_decode_step_noalloc(const dsa_decode_step_args_t *args, void *stream);
size_t dsa_decode_step_noalloc_max_bytes(void);

/*
 * Cache append: the write that precedes the path on every decode step (the renning22/glm-5.2-4090
 * README's usage section serves with an fp8_e4m3 KV cache; one f32 scale per token row is this
 * library's choice of granularity, which the pages do not fix).  The row of new
 * token i of sequence b goes to slot(b, pos(b,i)), pos(b,i) = L_b - Q + i, so seq_lens must
 * already count the Q new tokens.
 *   kv_new  [B, Q, 576]       f32 or bf16 new latent rows, or NULL to leave the latent cache
 *   k_new   [B, Q, head_dim]  f32 or bf16 new indexer keys, or NULL to leave the key cache
 *   kv_cache, k_cache         the paged caches of dsa_sparse_mla_decode / dsa_indexer_scores
 *   kv_scale, k_scale         [num_slots] f32, written for fp8 caches, NULL otherwise
 * Per destination dtype:
 *   same dtype as the rows    the stored bits are copied (f32 -> f32, bf16 -> bf16)
 *   DSA_FP8_E4M3FN            scale = max|row| / 448 (1 when max|row| < 2^-100, e.g. an
 *                             all-zero row); codes = e4m3fn(row / scale), round to nearest
 *                             with ties to even, magnitudes clamped to 448, the sign kept
 *                             (-0 gives 0x80); both divisions are IEEE binary32 divisions
 * Other pairs (f32 rows into a bf16 cache, anything into f32 from bf16) are DSA_ERR_UNSUPPORTED.
 * Supported: head_dim a multiple of 8 in 8..1024.  Rows that are NaN or infinite are outside
 * the supported set.  Two new tokens must not map to one slot (a valid page table ensures it).
 * Every other slot is left as it was.
 */
dsa_status_t dsa_kv_cache_append(const dsa_batch_t *batch,
                                 const void *kv_new, dsa_dtype_t kv_new_dtype,
                                 void *kv_cache, dsa_dtype_t kv_dtype, float *kv_scale,
                                 const void *k_new, dsa_dtype_t k_new_dtype, int32_t head_dim,
                                 void *k_cache, dsa_dtype_t k_dtype, float *k_scale,
                                 void *stream);

/*
 * Latent up-projection after attention (Show HN page "Chay GLM 5.2 tren may tinh cham",
 * main-features section, MLA weight absorption: the query absorbs kv_b and the context is
 * projected after attention).  The attention output of dsa_sparse_mla_decode is still in the
 * 512-wide latent space; per head it is projected by that head's value block of kv_b, then all
 * heads by o_proj:
 *   v[r,h,j] = sum_d w_uv[h,j,d] * attn_out[r,h,d]        (d < 512)
 *   y[r,m]   = sum_{h,j} w_o[m, h*v_dim + j] * v[r,h,j]
 *   attn_out  [rows, n_heads, 512] f32 (r = b*Q + i, as dsa_sparse_mla_decode writes it)
 *   w_uv      [n_heads, v_dim, 512] bf16;  w_o [d_model, n_heads*v_dim] bf16
 *   y         [rows, d_model] f32
 * The f32 activations enter the bf16 matrix cores as two bf16 parts (hi + lo, 2^-18 relative),
 * so y is an fp32-accurate product.  The workspace (dsa_latent_up_projection_workspace_size
 * bytes, 256-byte aligned, no initial contents) holds v and, when the K dimension is split over
 * workgroups, the partial sums, which are added in a fixed order (deterministic results).
 * Supported: n_heads <= 128, v_dim a multiple of 32 (<= 1024), d_model a multiple of 16
 * (<= 65536), rows <= 1000000.
 */
dsa_status_t dsa_latent_up_projection(int32_t rows, int32_t n_heads, int32_t v_dim, int32_t d_model,
                                      const float *attn_out, const void *w_uv, const void *w_o, float *y,
                                      void *workspace, size_t workspace_bytes, void *stream);
size_t dsa_latent_up_projection_workspace_size(int32_t rows, int32_t n_heads, int32_t v_dim, int32_t d_model);

/*
 * Opt-in checks of the data preconditions (the library built with DSA_DEBUG: libdsa_debug.so).
 * Its kernels test every sequence length, page-table entry, MLA slot, top-k score and page-map
 * index they read against the preconditions above.  A violation sets its bit in an error word
 * that the library keeps on each device, and the kernel clamps the value into range (a slot or
 * index out of range is skipped like -1; the cache append writes nothing for that token), so no
 * access leaves its buffer; the results are then unspecified but the GPU keeps running.
 * dsa_debug_check synchronises `stream`, stores the word in *flags (if flags is not NULL),
 * clears it, and returns DSA_OK when it was 0, otherwise DSA_ERR_INVALID_ARGUMENT with the
 * violated preconditions in dsa_last_error().  It is not capturable (it reads device memory).
 * libdsa.so returns DSA_ERR_UNSUPPORTED with *flags = 0.  The word is shared by every call on
 * one device, so calls that overlap there report together.
 */
#define DSA_DEBUG_SEQ_LEN     1u    /* seq_lens[b] outside [q_per_seq, max_seq_len] */
#define DSA_DEBUG_PAGE_ID     2u    /* a page-table entry outside [0, num_slots / page_size) */
#define DSA_DEBUG_SLOT        4u    /* a slot of dsa_sparse_mla_decode outside [-1, num_slots) */
#define DSA_DEBUG_NAN_SCORE   8u    /* a NaN among the scores a top-k ranks */
#define DSA_DEBUG_TOPK_INDEX 16u    /* an index of dsa_page_map outside [-1, seq_lens[b]) */
dsa_status_t dsa_debug_check(uint32_t *flags, void *stream);
int32_t dsa_debug_enabled(void);    /* 1 for libdsa_debug.so, 0 for libdsa.so */

const char *dsa_status_string(dsa_status_t status);
const char *dsa_last_error(void);   /* thread-local detail for the last non-OK status */
int32_t dsa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H_ */
