"""fp64 CPU oracle of the DSA decode path.

TEST INFRASTRUCTURE ONLY.  This module is the plain, slow definition of what the
HIP path computes.  It may be imported or executed only by ``tests/``, by
``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of ``bench.py``.
The product path (``sparse_attention_10_amd``) never imports it, and it never
imports the product path: the two share no code.  Only the seeded input
generator (``dsa_inputs``), which holds none of the method's arithmetic, feeds
both.

What is computed, stage by stage (the three ported kernel groups named in
"GLM-52 Runs on RTX 4090", section "how did he do it", and in the
renning22/glm-5.2-4090 README, section "how it works": lightning-indexer GEMM,
top-k + page-mapping transform, MLA sparse decode):

  1. indexer_scores   s[b,i,t] = sum_h w[b,i,h] * max(0, q[b,i,h,:] . k[slot(b,t),:])
                      for every visible token t <= pos(b,i); -inf elsewhere.
  2. topk_select      the min(k, pos+1) visible tokens with the largest s; equal
                      scores go to the lower token index; returned in ascending
                      token order, padded with -1.
  3. page_map         slot = page_table[b][t // P] * P + t % P; -1 stays -1
                      (the fused page-mapping transform of the README's usage
                      section, SGLANG_NSA_FUSE_TOPK).
  4. sparse_mla       per (b,i,h): z_t = sm_scale * (q_h . c_t) over the 576
                      values of each selected latent row, o = softmax(z) . c[:, :512],
                      lse = log sum exp(z).  Weight-absorbed MLA, 64 heads with no
                      GQA, one 576-wide compressed row per token (Show HN: "Chay
                      GLM 5.2 tren may tinh cham", main-features section: 576
                      values per token, 64 heads / no GQA, MLA weight absorption).
  5. combine_splits   the split-k merge of per-chunk softmax partials.
  6. dense_mla        an independent formulation of attention over every visible
                      token (library softmax / logsumexp), for pins only: with
                      k >= context the sparse path must equal it, as colibri's
                      attention is dense and exact up to 2048 tokens (same page,
                      main-features section, DSA bullet).
  7. cache_append     the write that precedes the path on every decode step: each
                      new token's latent row and indexer key go to slot(b, pos(b,i));
                      an fp8 cache stores per-token scale = max|row| / 448 and the
                      nearest-even e4m3fn codes of row / scale (README usage section:
                      fp8_e4m3 KV cache; one scale per token row is this library's
                      choice of granularity).
  8. latent_up_projection
                      the step after the path: with MLA weight absorption the query
                      has absorbed kv_b and the attention output is still in the
                      512-wide latent space, so it is projected afterwards, per head
                      by that head's value block of kv_b (W_UV), then by o_proj (W_O)
                      (Show HN main-features section, MLA weight absorption bullet).

Every array is decoded from its stored bits here (bf16 and fp8 e4m3fn decoders
written from the format definitions) and all arithmetic is float64.

Readings taken where the pages are silent (each is listed with its reason in
the design notes): w is per query and head; the indexer key cache is paged by
the same page table as the latent cache; pos(b,i) = L_b - Q + i; the fp8 scale
multiplies the decoded code (dequantize, then dot); -0.0 and +0.0 are equal
scores; an empty selection yields out = 0 and lse = -inf.

Parity pins: see tests/test_oracle_pins.py.  Every function here is pinned
(brute force, closed forms, invariants or a library routine); none is
"parity unpinned".
"""
from __future__ import annotations

import numpy as np

V_DIM = 512
ROW_DIM = 576


# ---------------------------------------------------------------------------
# 0. stored values -> float64

def decode_bf16(bits) -> np.ndarray:
    """bf16 bit patterns -> float64: the 16 bits are the upper half of an IEEE
    binary32 word whose lower half is zero."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def decode_e4m3fn(codes) -> np.ndarray:
    """OCP FP8 E4M3FN codes -> float64, from the format definition: sign bit,
    4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes the
    subnormals m/8 * 2^-6; there are no infinities; S.1111.111 is NaN; the
    largest finite magnitude is 1.75 * 2^8 = 448."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c & 0x80) != 0, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & ((c & 0x7) == 7), np.nan, mag)
    return sign * mag


def dequantize(x, dtype: str, scale=None) -> np.ndarray:
    """Stored array -> float64 values.  For 'fp8' the value of a code in row r
    is scale[r] * decode(code): one f32 scale per token row."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    if dtype == "bf16":
        return decode_bf16(x)
    if dtype == "fp8":
        if scale is None:
            raise ValueError("fp8 values need their per-row scale")
        v = decode_e4m3fn(x)
        return v * np.asarray(scale, dtype=np.float32).astype(np.float64).reshape(
            v.shape[:-1] + (1,))
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# positions and paging

def query_positions(seq_lens, q_per_seq: int) -> np.ndarray:
    """pos(b, i) = L_b - Q + i: L_b counts the Q new tokens, query i sits at
    the i-th of them and sees every token up to and including itself."""
    L = np.asarray(seq_lens, dtype=np.int64)
    return L[:, None] - q_per_seq + np.arange(q_per_seq)[None, :]


def token_slots(page_table_row, tokens, page_size: int) -> np.ndarray:
    """Physical cache slot of logical token t of one sequence:
    page_table[t // P] * P + t % P."""
    t = np.asarray(tokens, dtype=np.int64)
    pt = np.asarray(page_table_row, dtype=np.int64)
    return pt[t // page_size] * page_size + t % page_size


# ---------------------------------------------------------------------------
# 1. lightning indexer

def indexer_scores(q, q_dtype, w, k_cache, k_dtype, k_scale, seq_lens, page_table,
                   q_per_seq: int, page_size: int, ld: int | None = None) -> np.ndarray:
    """Lightning-indexer scores [B, Q, ld] in float64.

    s[b,i,t] = sum_h w[b,i,h] * ReLU(q[b,i,h,:] . k~[slot(b,t),:]) for t <= pos(b,i),
    -inf for every other column.  k~ is the dequantized key row (f32, bf16, or
    fp8 code times its per-token scale)."""
    L = np.asarray(seq_lens)
    B = len(L)
    ld = int(L.max()) if ld is None else int(ld)
    qd = dequantize(q, q_dtype)                         # [B,Q,Hi,Di]
    wd = np.asarray(w, dtype=np.float32).astype(np.float64)   # [B,Q,Hi]
    pos = query_positions(L, q_per_seq)
    s = np.full((B, q_per_seq, ld), -np.inf)
    for b in range(B):
        n_max = int(pos[b].max()) + 1
        sl = token_slots(page_table[b], np.arange(n_max), page_size)
        kd = dequantize(k_cache[sl], k_dtype, None if k_scale is None else k_scale[sl])  # [n, Di]
        for i in range(q_per_seq):
            n = int(pos[b, i]) + 1
            logits = qd[b, i] @ kd[:n].T                # [Hi, n]
            s[b, i, :n] = wd[b, i] @ np.maximum(logits, 0.0)
    return s


# ---------------------------------------------------------------------------
# 2. top-k

def topk_select(scores_row, n_visible: int, k: int) -> np.ndarray:
    """Indices of the min(k, n_visible) largest of scores_row[:n_visible].

    Ranking key (-s_t, t): a larger score first, and among equal scores the lower
    token index first.  Scores compare as exact values (f32 inputs are widened
    exactly), so -0.0 and +0.0 are equal.  The chosen set is returned in
    ascending token order, padded to k with -1."""
    s = np.asarray(scores_row[:n_visible], dtype=np.float64)
    t = np.arange(n_visible)
    order = np.lexsort((t, -s))                         # last key is primary
    chosen = np.sort(order[:min(k, n_visible)])
    out = np.full(k, -1, dtype=np.int32)
    out[:chosen.size] = chosen
    return out


def topk(scores, seq_lens, q_per_seq: int, k: int) -> np.ndarray:
    """topk_select for every query row: row (b,i) sees pos(b,i)+1 tokens."""
    pos = query_positions(seq_lens, q_per_seq)
    B = len(seq_lens)
    out = np.empty((B, q_per_seq, k), dtype=np.int32)
    for b in range(B):
        for i in range(q_per_seq):
            out[b, i] = topk_select(scores[b, i], int(pos[b, i]) + 1, k)
    return out


# ---------------------------------------------------------------------------
# 3. page mapping

def page_map(idx, page_table, page_size: int) -> np.ndarray:
    """Selected logical token ids [B,Q,k] -> physical slots [B,Q,k]; -1 stays -1."""
    idx = np.asarray(idx, dtype=np.int64)
    out = np.full(idx.shape, -1, dtype=np.int64)
    for b in range(idx.shape[0]):
        valid = idx[b] >= 0
        out[b][valid] = token_slots(page_table[b], idx[b][valid], page_size)
    return out.astype(np.int32)


# ---------------------------------------------------------------------------
# 4./5. sparse MLA decode and the split-k merge

def mla_partial(qd, rows, sm_scale: float):
    """Softmax partial of one query over a set of dequantized latent rows.

    qd [H, 576], rows [n, 576] -> (m [H], l [H], o [H, 512]) with
    z = sm_scale * qd . rows^T, m = max_t z, l = sum_t exp(z - m),
    o = sum_t exp(z - m) * rows[t, :512] / l.  An empty set gives
    m = -inf, l = 0, o = 0."""
    H = qd.shape[0]
    if rows.shape[0] == 0:
        return np.full(H, -np.inf), np.zeros(H), np.zeros((H, V_DIM))
    z = sm_scale * (qd @ rows.T)                        # [H, n]
    m = z.max(axis=1)
    e = np.exp(z - m[:, None])
    l = e.sum(axis=1)
    o = (e @ rows[:, :V_DIM]) / l[:, None]
    return m, l, o


def combine_splits(m, l, o):
    """Merge per-chunk partials (m_j, l_j, o_j), j over chunks:
    M = max_j m_j, a_j = exp(m_j - M) * l_j, out = sum_j a_j o_j / sum_j a_j,
    lse = M + log sum_j a_j.  Chunks with l_j = 0 carry no weight; if every
    chunk is empty, out = 0 and lse = -inf."""
    m = np.asarray(m, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    M = m.max(axis=0)
    live = np.isfinite(M)
    Ms = np.where(live, M, 0.0)
    a = np.where(l > 0, np.exp(np.where(l > 0, m, 0.0) - Ms[None, :]) * l, 0.0)
    den = a.sum(axis=0)
    out = np.where(live[:, None], (a[:, :, None] * o).sum(axis=0) / np.where(live, den, 1.0)[:, None], 0.0)
    lse = np.where(live, Ms + np.log(np.where(live, den, 1.0)), -np.inf)
    return out, lse


def sparse_mla(q, q_dtype, kv_cache, kv_dtype, kv_scale, slots, sm_scale: float):
    """Sparse MLA decode: out [B,Q,H,512], lse [B,Q,H] in float64.

    For each (b,i) the selected rows are kv_cache[slots[b,i,j]] for every
    slots entry that is not -1 (their order does not matter)."""
    qd_all = dequantize(q, q_dtype)                     # [B,Q,H,576]
    B, Q, H, _ = qd_all.shape
    out = np.zeros((B, Q, H, V_DIM))
    lse = np.full((B, Q, H), -np.inf)
    for b in range(B):
        for i in range(Q):
            sel = np.asarray(slots[b, i], dtype=np.int64)
            sel = sel[sel >= 0]
            rows = dequantize(kv_cache[sel], kv_dtype, None if kv_scale is None else kv_scale[sel])
            m, l, o = mla_partial(qd_all[b, i], rows, sm_scale)
            out[b, i] = o
            lse[b, i] = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return out, lse


def dense_mla(q, q_dtype, kv_cache, kv_dtype, kv_scale, seq_lens, page_table,
              q_per_seq: int, page_size: int, sm_scale: float):
    """Dense MLA over every visible token (t <= pos(b,i)), written with the
    library's softmax and logsumexp: the logit matrix, a row softmax, then
    times V = the first 512 values of each row."""
    from scipy.special import logsumexp, softmax
    qd_all = dequantize(q, q_dtype)
    B, Q, H, _ = qd_all.shape
    pos = query_positions(seq_lens, q_per_seq)
    out = np.zeros((B, Q, H, V_DIM))
    lse = np.zeros((B, Q, H))
    for b in range(B):
        for i in range(Q):
            sl = token_slots(page_table[b], np.arange(int(pos[b, i]) + 1), page_size)
            rows = dequantize(kv_cache[sl], kv_dtype, None if kv_scale is None else kv_scale[sl])
            logits = sm_scale * (qd_all[b, i] @ rows.T)
            out[b, i] = softmax(logits, axis=1) @ rows[:, :V_DIM]
            lse[b, i] = logsumexp(logits, axis=1)
    return out, lse


# ---------------------------------------------------------------------------
# 6. the whole decode step

def decode_step(inp: dict, cfg) -> dict:
    """Stages 1 -> 2 -> 3 -> 4 in order, on the arrays of dsa_inputs.make_inputs."""
    s = indexer_scores(inp["q_idx"], cfg.q_idx_dtype, inp["w"], inp["k_cache"], cfg.key_dtype,
                       inp["k_scale"], inp["seq_lens"], inp["page_table"], cfg.q_per_seq,
                       cfg.page_size)
    idx = topk(s, inp["seq_lens"], cfg.q_per_seq, cfg.top_k)
    slots = page_map(idx, inp["page_table"], cfg.page_size)
    out, lse = sparse_mla(inp["q_mla"], cfg.q_mla_dtype, inp["kv_cache"], cfg.kv_dtype,
                          inp["kv_scale"], slots, cfg.sm_scale)
    return {"scores": s, "idx": idx, "slots": slots, "out": out, "lse": lse}


# ---------------------------------------------------------------------------
# 7. cache append: the write of the new tokens' rows before the path reads them

FP8_MAX = 448.0
# below this row maximum the per-token scale is 1 (the all-zero row's scale): every value
# then encodes to a signed zero, and no scale can underflow the binary32 range
SCALE_FLOOR = 2.0 ** -100


def encode_e4m3fn(y) -> np.ndarray:
    """binary32 values -> OCP FP8 E4M3FN codes, round to nearest with ties to the
    even code, from the format definition: the candidates are the finite
    non-negative magnitudes of codes 0x00..0x7E (decode_e4m3fn), a magnitude
    above 448 saturates to 448, and the sign bit is copied from y (so -0.0 and a
    negative value that rounds to zero give 0x80).  NaN inputs are not defined."""
    a = np.minimum(np.abs(np.asarray(y, dtype=np.float32).astype(np.float64)), FP8_MAX)
    neg = np.signbit(np.asarray(y, dtype=np.float32))
    vals = decode_e4m3fn(np.arange(0x7F, dtype=np.uint8))          # strictly increasing
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, 0x7E)    # vals[hi-1] < a <= vals[hi]
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - vals[lo], vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(neg, code | np.uint8(0x80), code).astype(np.uint8)


def quantize_row_fp8(x):
    """One token row (float64 holding exact binary32 or bf16 values) -> (codes uint8,
    scale float32).  scale = binary32(max|x| / 448), or 1 when max|x| < 2^-100 (the
    all-zero row included); y = binary32(x / scale) value by value; codes =
    encode_e4m3fn(y).  A binary64 quotient rounded to binary32 is the correctly
    rounded binary32 quotient (53 >= 2*24 + 2 bits), so both roundings are the
    IEEE single-precision divisions."""
    x = np.asarray(x, dtype=np.float64)
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    scale = np.float32(amax / FP8_MAX) if amax >= SCALE_FLOOR else np.float32(1.0)
    y = (x / np.float64(scale)).astype(np.float32)
    return encode_e4m3fn(y), scale


def cache_append(cache, cache_dtype: str, scale, new_rows, new_dtype: str, seq_lens, page_table,
                 q_per_seq: int, page_size: int):
    """Write the Q new tokens of each sequence into the paged cache: the row of
    query i of sequence b goes to slot(b, pos(b,i)), pos(b,i) = L_b - Q + i.
    cache [num_slots, D] in cache_dtype ('f32', 'bf16' or 'fp8'); scale [num_slots]
    f32 for 'fp8' (else None); new_rows [B, Q, D] in new_dtype ('f32' or 'bf16').
    A cache of the rows' own dtype receives their stored bits; an fp8 cache
    receives quantize_row_fp8 of each row and its scale.  Returns new arrays
    (cache, scale); every other slot keeps its contents."""
    cache = np.array(cache, copy=True)
    scale = None if scale is None else np.array(scale, dtype=np.float32, copy=True)
    x = dequantize(new_rows, new_dtype)
    pos = query_positions(seq_lens, q_per_seq)
    for b in range(pos.shape[0]):
        slots = token_slots(np.asarray(page_table)[b], pos[b], page_size)
        for i, s in enumerate(slots):
            if cache_dtype == "fp8":
                cache[s], scale[s] = quantize_row_fp8(x[b, i])
            elif cache_dtype == new_dtype:
                cache[s] = np.asarray(new_rows)[b, i]
            else:
                raise ValueError(f"no append from {new_dtype} rows into a {cache_dtype} cache")
    return cache, scale


# ---------------------------------------------------------------------------
# 8. latent up-projection: the projection after attention of the weight-absorbed MLA

def latent_up_projection(o, w_uv, w_o):
    """o [R, H, 512] float (the attention output in the latent space), w_uv [H, Dv, 512]
    bf16 bits (per head, the value block of kv_b), w_o [Dm, H*Dv] bf16 bits (o_proj):
        v[r, h, j] = sum_d w_uv[h, j, d] * o[r, h, d]
        y[r, m]    = sum_{h, j} w_o[m, h*Dv + j] * v[r, h, j]
    Returns (y [R, Dm], v [R, H, Dv]) in float64."""
    od = np.asarray(o, dtype=np.float64)
    w1 = decode_bf16(w_uv)
    w2 = decode_bf16(w_o)
    R, H, _ = od.shape
    v = np.einsum("rhd,hjd->rhj", od, w1)
    y = v.reshape(R, -1) @ w2.T
    return y, v
