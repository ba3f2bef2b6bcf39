"""Shared helpers of the GPU parity tests: run the C-ABI calls on seeded inputs and compare
with the fp64 oracle to the pass criteria of the path:
  * top-k indices and page-map slots: bit-exact on identical score arrays;
  * indexer scores: per query row, max_t |gpu - ref| <= 1e-5 * max_t |ref| over the visible
    columns, masked columns exactly -inf;
  * attention: max-abs <= 2e-3 over every output value, cosine >= 0.99999 for every
    (row, head) 512-vector, lse within 1e-4 absolute.
"""
from __future__ import annotations

import numpy as np
import torch

import dsa_inputs
import sparse_attention_10_amd as dsa
from oracle import dsa_oracle as O

INDEXER_RTOL = 1e-5
ATTN_MAX_ABS = 2e-3
ATTN_MIN_COS = 0.99999
LSE_ABS = 1e-4

DEV = "cuda:0"


def batch_of(cfg, t):
    return dsa.make_batch(t["seq_lens"], t["page_table"], cfg.q_per_seq, cfg.page_size,
                          cfg.max_seq_len, cfg.num_slots)


def gpu_scores(cfg, t, ld=None, fill=float("nan")):
    ld = cfg.max_seq_len if ld is None else ld
    scores = torch.full((cfg.batch, cfg.q_per_seq, ld), fill, dtype=torch.float32, device=DEV)
    dsa.dsa_indexer_scores(batch_of(cfg, t), t["q_idx"], t["w"], t["k_cache"], t["k_scale"], scores)
    torch.cuda.synchronize()
    return scores


def check_indexer(cfg, got: np.ndarray, ref: np.ndarray, seq_lens):
    pos = O.query_positions(seq_lens, cfg.q_per_seq)
    worst = 0.0
    for b in range(cfg.batch):
        L = int(seq_lens[b])
        for i in range(cfg.q_per_seq):
            n = int(pos[b, i]) + 1
            g, r = got[b, i, :n].astype(np.float64), ref[b, i, :n]
            scale = max(np.abs(r).max(), 1e-30)
            err = np.abs(g - r).max() / scale
            worst = max(worst, err)
            assert err <= INDEXER_RTOL, f"indexer row ({b},{i}) normwise error {err:.3e}"
            assert np.all(np.isneginf(got[b, i, n:L])), f"row ({b},{i}) masked columns are not -inf"
    return worst


def check_attention(out_g: np.ndarray, out_r: np.ndarray, lse_g=None, lse_r=None):
    out_g = out_g.astype(np.float64)
    err = np.abs(out_g - out_r).max()
    assert err <= ATTN_MAX_ABS, f"attention max-abs error {err:.3e}"
    g = out_g.reshape(-1, out_g.shape[-1])
    r = out_r.reshape(-1, out_r.shape[-1])
    ng, nr = np.linalg.norm(g, axis=1), np.linalg.norm(r, axis=1)
    live = nr > 0
    cos = (g[live] * r[live]).sum(1) / (ng[live] * nr[live])
    min_cos = cos.min() if cos.size else 1.0
    assert min_cos >= ATTN_MIN_COS, f"attention min cosine {min_cos:.8f}"
    assert np.all(g[~live] == 0), "rows with an empty selection must be 0"
    if lse_g is not None:
        lg, lr = lse_g.astype(np.float64).ravel(), lse_r.ravel()
        fin = np.isfinite(lr)
        assert np.array_equal(np.isneginf(lg), np.isneginf(lr)), "lse -inf pattern differs"
        lerr = np.abs(lg[fin] - lr[fin]).max() if fin.any() else 0.0
        assert lerr <= LSE_ABS, f"lse error {lerr:.3e}"
    return err, min_cos


def gpu_mla(cfg, t, slots_t, n_split=0, with_lse=True):
    B, Q, H = cfg.batch, cfg.q_per_seq, cfg.mla_heads
    out = torch.full((B, Q, H, 512), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((B, Q, H), float("nan"), dtype=torch.float32, device=DEV) if with_lse else None
    dsa.dsa_sparse_mla_decode(t["q_mla"], t["kv_cache"], t["kv_scale"], slots_t, cfg.sm_scale, out, lse,
                              n_split=n_split)
    torch.cuda.synchronize()
    return out, lse


def oracle_mla(cfg, inp, slots: np.ndarray):
    return O.sparse_mla(inp["q_mla"], cfg.q_mla_dtype, inp["kv_cache"], cfg.kv_dtype, inp["kv_scale"], slots,
                        cfg.sm_scale)


def run_step(cfg, t, n_split=0, debug=True):
    B, Q, H, k = cfg.batch, cfg.q_per_seq, cfg.mla_heads, cfg.top_k
    out = torch.full((B, Q, H, 512), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((B, Q, H), float("nan"), dtype=torch.float32, device=DEV)
    dbg_s = torch.full((B, Q, cfg.max_seq_len), float("nan"), dtype=torch.float32, device=DEV) if debug else None
    dbg_i = torch.full((B, Q, k), -7, dtype=torch.int32, device=DEV) if debug else None
    dbg_l = torch.full((B, Q, k), -7, dtype=torch.int32, device=DEV) if debug else None
    args = dsa.decode_step_args(batch_of(cfg, t), t["q_idx"], t["w"], t["k_cache"], t["k_scale"], k,
                                t["q_mla"], t["kv_cache"], t["kv_scale"], cfg.sm_scale, out, lse, n_split,
                                dbg_s, dbg_i, dbg_l)
    nbytes = dsa.decode_step_workspace_bytes(args)
    ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=DEV)
    dsa.dsa_decode_step(args, ws)
    torch.cuda.synchronize()
    return dict(out=out, lse=lse, scores=dbg_s, idx=dbg_i, slots=dbg_l)
