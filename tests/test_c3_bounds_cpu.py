"""Host emulation, at the exact batch-32 ragged decode workload (contexts 4K-128K drawn from
its seed, page tables dealt from one shuffled pool), of the index arithmetic of the fused step's
kernels as they stand: every global read and write must stay inside its buffer and every score
column must be written exactly once.  The emulation restates the launchers' and kernels'
integer arithmetic (sparse_attention_10_amd/csrc: indexer_reg_kernel's balanced key ranges and
per-wave block walk, the top-k two-pass plan, the sparse MLA chunking) and sizes the buffers
with the library's own size queries; it runs on the CPU only."""
import ctypes
import math

import numpy as np
import pytest

import dsa_inputs
import sparse_attention_10_amd as dsa

KRB = 16                 # indexer tokens per block
REG_MAX_PAGES = 1024     # page-table entries an indexer workgroup stages
NW, D = 8, 3             # waves and ring depth of the one-row, bf16-key register kernel


def _c3():
    cfg = dsa_inputs.base_config("c3")
    pt = dsa_inputs.page_table_for(cfg, np.random.default_rng([cfg.seed, dsa_inputs._T_PERM]))
    return cfg, pt


# a batch of 32 ragged sequences at parity-test lengths (the GPU parity case
# test_indexer_parity_batch32_ragged runs exactly this configuration)
SCALED32_LENS = [int(x) for x in np.random.default_rng(3232).integers(256, 12000, size=32, endpoint=True)]


def scaled32():
    cfg = dsa_inputs.scaled_config("c3", SCALED32_LENS, seed=3233)
    pt = dsa_inputs.page_table_for(cfg, np.random.default_rng([cfg.seed, dsa_inputs._T_PERM]))
    return cfg, pt


def _indexer_launch(cfg):
    """launch_indexer's host arithmetic for the register kernel (one query row per sequence)."""
    B, Q, P, maxL = cfg.batch, cfg.q_per_seq, cfg.page_size, cfg.max_seq_len
    QB = Q if Q <= 2 else 2
    ng = (Q + QB - 1) // QB
    blocks = (maxL + KRB - 1) // KRB
    tb_max = max(1, (REG_MAX_PAGES - 2) * P // KRB)
    R = max(1, 256 // ng)
    tb = min(max((blocks * B + R - 1) // R, 1), tb_max)
    groups = (blocks + tb - 1) // tb
    balanced, ranges = 0, B * groups
    if B >= 2 and 2 * B <= R and B <= 8 * 64 and (B * blocks + (R - B) - 1) // (R - B) <= tb_max:
        balanced, ranges = R - B, R
    return dict(QB=QB, ng=ng, tb=tb, groups=groups, balanced=balanced, grid=(ranges + 7) // 8 * 8 * ng)


def _partition(lens, maxL, balanced, B):
    """The balanced partition every indexer workgroup derives from seq_lens: (T, [ranges of b])."""
    ti = [(max(min(L, maxL), 0) + KRB - 1) // KRB for L in lens]
    total = sum(ti)
    R = balanced + B
    T = max(1, (total + R - 1) // R)
    T_safe = max(1, (total + balanced - 1) // balanced)
    for _ in range(4):
        if T >= T_safe:
            break
        cnt = sum((t + T - 1) // T for t in ti)
        if cnt <= R:
            break
        T = min(T_safe, max(T + 1, (T * cnt + R - 1) // R))
    if T < T_safe and sum((t + T - 1) // T for t in ti) > R:
        T = T_safe
    gi = [(t + T - 1) // T for t in ti]
    return T, gi


def test_c3_indexer_reads_and_writes_stay_in_bounds_and_cover_every_column_once():
    cfg, pt = _c3()
    assert min(cfg.seq_lens) >= 4096 and max(cfg.seq_lens) <= 131072 and cfg.batch == 32
    _emulate_indexer(cfg, pt)


def test_scaled_batch32_indexer_stays_in_bounds():
    cfg, pt = scaled32()
    assert cfg.batch == 32 and cfg.q_per_seq == 1
    _emulate_indexer(cfg, pt)


def _emulate_indexer(cfg, pt):
    B, Q, P, maxL = cfg.batch, cfg.q_per_seq, cfg.page_size, cfg.max_seq_len
    lens = cfg.seq_lens
    lp = _indexer_launch(cfg)
    assert lp["balanced"] > 0 and lp["grid"] == 256 and lp["QB"] == 1   # the balanced partition
    T, gi = _partition(lens, maxL, lp["balanced"], B)
    incl = np.cumsum(gi)
    assert incl[-1] <= lp["grid"], "every range gets a workgroup"
    written = [np.zeros(L, np.int32) for L in lens]
    p_shift = int(math.log2(P))
    for kr in range(lp["grid"]):
        if kr >= incl[-1]:
            continue                                    # the workgroup returns
        b = int(np.searchsorted(incl, kr, side="right"))
        first = int(incl[b] - gi[b])
        blk0, nblk = (kr - first) * T, T
        L = min(lens[b], maxL)
        t_begin = blk0 * KRB
        assert t_begin < L, "a listed range starts inside its sequence"
        t_end = min(L, (blk0 + nblk) * KRB)
        pos_last = L - Q + Q - 1
        t_stop = min(t_end, pos_last + 1)
        nb = (t_stop - t_begin + KRB - 1) // KRB if t_stop > t_begin else 0
        page0 = t_begin // P
        npg = (t_stop - 1) // P - page0 + 1 if nb > 0 else 0
        assert npg <= REG_MAX_PAGES, "the range's page-table entries fit the LDS copy"
        assert page0 + npg <= pt.shape[1] and np.all(pt[b, page0:page0 + npg] >= 0)
        for w in range(NW):
            nbw = (nb - w + NW - 1) // NW if nb > w else 0
            nbw_pad = (nbw + D - 1) // D * D
            # blocks requested: jj < nbw_pad + D (the ring refills past the last block read row 0)
            for jj in range(nbw_pad + D):
                tb = t_begin + (w + jj * NW) * KRB
                if tb < t_stop:
                    pg = tb >> p_shift
                    assert page0 <= pg < page0 + npg
                    row0 = int(pt[b, pg]) * P + (tb - pg * P)
                    assert 0 <= row0 and row0 + KRB <= cfg.num_slots, "key rows of a block lie in the cache"
                    assert (tb % P) + KRB <= P, "a block stays inside its page"
                if jj < nbw:
                    for t in range(tb, tb + KRB):
                        if t < t_end:
                            written[b][t] += 1
        for t in range(t_begin + nb * KRB, t_end):      # the tail loop (-inf past the last position)
            written[b][t] += 1
    for b, wb in enumerate(written):
        assert np.all(wb == 1), f"sequence {b}: columns written {wb.min()}..{wb.max()} times"


def test_c3_topk_two_pass_plan_and_candidates_fit_the_workspace():
    cfg, _ = _c3()
    rows, maxL, k = cfg.batch * cfg.q_per_seq, cfg.max_seq_len, cfg.top_k
    # topk_plan: rows of 64K+ columns, at most 128 rows, chunks of 16K-32K, one workgroup per CU
    plan = None
    if maxL >= 65536 and rows <= 128:
        for L in (16384, 32768):
            C = (maxL + L - 1) // L
            if L >= 4 * k and C >= 2 and rows * C <= 256:
                plan = (L, C)
                break
    assert plan is not None
    L, C = plan
    kc = min(k, L)
    cand_ld = C * kc
    batch = dsa.DsaBatch(cfg.batch, cfg.q_per_seq, maxL, cfg.page_size, cfg.max_pages, cfg.num_slots, 1 << 20, 1 << 20)
    ws = dsa.lib().dsa_topk_workspace_size(ctypes.byref(batch), k)
    score_bytes = (rows * cand_ld * 4 + 255) // 256 * 256
    assert ws >= score_bytes + rows * cand_ld * 4
    for L_b in cfg.seq_lens:
        n_row = min(L_b, C * L)
        assert n_row == L_b, "the chunks reach every visible column"
        # first pass: chunk c ranks columns [cL, cL + n) and writes at most kc candidates at c*kc
        covered = 0
        for c in range(C):
            n = min(max(n_row - c * L, 0), L)
            assert c * kc + min(n, kc) <= cand_ld
            covered += n
        assert covered == n_row
        # second pass: the candidates of the chunks that hold columns
        nch = (n_row + L - 1) // L
        n2 = (nch - 1) * kc + min(k, n_row - (nch - 1) * L)
        assert 0 < n2 <= cand_ld


def test_c3_step_workspace_and_mla_chunks():
    cfg, _ = _c3()
    rows, H, k = cfg.batch * cfg.q_per_seq, cfg.mla_heads, cfg.top_k
    ns = dsa.lib().dsa_sparse_mla_default_split(cfg.batch, cfg.q_per_seq, H, k, dsa.DSA_BF16)
    ns = min(ns, (k + 31) // 32)
    chunk = ((k + ns - 1) // ns + 31) // 32 * 32
    assert chunk <= 2048, "the bf16 ring kernel's staging limit"
    starts = [s * chunk for s in range(ns)]
    assert starts[-1] < k and sum(min(k, s + chunk) - s for s in starts) == k
    a = dsa.DsaDecodeStepArgs()
    a.batch = dsa.DsaBatch(cfg.batch, cfg.q_per_seq, cfg.max_seq_len, cfg.page_size, cfg.max_pages, cfg.num_slots,
                           1 << 20, 1 << 20)
    a.idx_heads, a.idx_dim, a.top_k, a.mla_heads = 64, 128, k, H
    a.q_idx_dtype = a.k_dtype = a.q_mla_dtype = a.kv_dtype = dsa.DSA_BF16
    need = dsa.lib().dsa_decode_step_workspace_size(ctypes.byref(a))
    scores = rows * cfg.max_seq_len * 4
    partials = rows * ns * H * 512 * 4 + 2 * rows * ns * H * 4
    assert need >= scores + 2 * rows * k * 4 + partials
