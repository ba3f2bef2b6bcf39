"""Host restatement, at the exact batch-32 ragged decode workload (contexts 4K-128K drawn from its
seed, page tables dealt from one shuffled pool), of the index arithmetic of the kernels that ran
when that workload's first benchmark faulted the GPU: git revision 8e5a3bf of
sparse_attention_10_amd/csrc (the 128-token-tile indexer with up to 8 tiles per workgroup, the
1024-thread top-k whose 64-keys-per-thread variant spilled to scratch, the 4-wave sparse MLA with
its split-k merge, and the fused step's workspace layout).  Every global read and write they make
for valid inputs must lie inside its buffer, every LDS index inside its array, and every score
column must be written exactly once.  Those kernels have since been replaced; this test only
records that their arithmetic at this workload was in bounds, so the fault's cause is not among
these accesses.  It runs on the CPU only."""
import numpy as np

import dsa_inputs

# constants of that revision
K_MAX_TOPK_SEQ = 262144
IDX_SUB, IDX_WAVES = 32, 4
IDX_TILE = IDX_SUB * IDX_WAVES                  # 128 tokens per workgroup tile
TOPK_THREADS, TOPK_WAVES = 1024, 16
TOPK_BINS = 1 << 11
TOPK_MAX_IT = K_MAX_TOPK_SEQ // TOPK_THREADS    # 256 rows of the ballot tables
MLA_TT, MLA_NT = 32, 256                        # tokens per tile, threads per workgroup
ROW_BF16 = 576 * 2


def _c3():
    cfg = dsa_inputs.base_config("c3")
    pt = dsa_inputs.page_table_for(cfg, np.random.default_rng([cfg.seed, dsa_inputs._T_PERM]))
    return cfg, pt


def test_fault_revision_indexer_at_c3():
    cfg, pt = _c3()
    B, Q, P, maxL = cfg.batch, cfg.q_per_seq, cfg.page_size, cfg.max_seq_len
    assert B == 32 and Q == 1
    # launch_indexer: one row per group (Q odd), tiles per workgroup from the work
    QB = 2 if Q % 2 == 0 else 1
    tiles = (maxL + IDX_TILE - 1) // IDX_TILE
    work = tiles * B * ((Q + QB - 1) // QB)
    tpw = min(max(work // 2048, 1), 8)
    assert tpw == 8, "the multi-tile path the tests had not run"
    gx = (tiles + tpw - 1) // tpw
    ld = maxL                                    # the fused step's score rows are max_seq_len long
    written = [np.zeros(L, np.int32) for L in cfg.seq_lens]
    for b in range(B):
        L = min(cfg.seq_lens[b], maxL)
        npages = (cfg.seq_lens[b] + P - 1) // P
        pos_last = L - Q + 0 + min(QB, Q) - 1
        for x in range(gx):
            base = x * tpw * IDX_TILE
            if base >= L:
                continue                          # uniform early exit
            end = min(L, base + tpw * IDX_TILE)
            for w in range(IDX_WAVES):
                t = np.arange(IDX_SUB)
                subs = np.arange(base + w * IDX_SUB, end, IDX_TILE)
                # current sub-tiles and the prefetch of the next one (read only when valid)
                for sub in np.concatenate([subs, subs[-1:] + IDX_TILE]) if len(subs) else [base + w * IDX_SUB]:
                    tok = sub + t
                    valid = (tok < end) & (tok <= pos_last)
                    pg = tok[valid] // P
                    assert np.all(pg < npages) and np.all(pg < pt.shape[1])
                    slot = pt[b, pg].astype(np.int64) * P + tok[valid] % P
                    assert np.all(slot >= 0) and np.all(slot < cfg.num_slots)
                for sub in subs:                  # score writes of the current sub-tile
                    tok = sub + t
                    tok = tok[tok < end]
                    assert np.all(tok < ld)
                    np.add.at(written[b], tok, 1)
    for b, wb in enumerate(written):
        assert np.all(wb == 1), f"sequence {b}: columns written {wb.min()}..{wb.max()} times"


def test_fault_revision_topk_at_c3():
    cfg, pt = _c3()
    B, Q, P, maxL, k = cfg.batch, cfg.q_per_seq, cfg.page_size, cfg.max_seq_len, cfg.top_k
    ld = maxL
    items = 8 if maxL <= 8 * TOPK_THREADS else 16 if maxL <= 16 * TOPK_THREADS else \
        32 if maxL <= 32 * TOPK_THREADS else 64
    assert items == 64, "the variant with the 416-byte-per-lane private segment"
    for b in range(B):
        for i in range(Q):
            n = max(cfg.seq_lens[b] - Q + i + 1, 0)
            n = min(n, ld, K_MAX_TOPK_SEQ)
            assert n > k                          # every c3 row ranks (contexts >= 4096)
            n_reg = min(n, items * TOPK_THREADS)
            assert n_reg <= ld and n <= ld        # register block and streamed tail stay in the row
            # radix rounds: at most 11 bits, bins < TOPK_BINS
            for plen in range(0, 32):
                D = min(11, 32 - plen)
                assert (1 << D) <= TOPK_BINS
                # thread t scans bins nb-1-2t and nb-2-2t: 1024 threads cover 2048 bins
                assert 2 * TOPK_THREADS >= (1 << D)
            nit = (n + TOPK_THREADS - 1) // TOPK_THREADS
            assert nit <= TOPK_MAX_IT
            ne = nit * TOPK_WAVES                  # ballot-table entries
            assert (nit - 1) * TOPK_WAVES + TOPK_WAVES - 1 < TOPK_MAX_IT * TOPK_WAVES
            per = (ne + TOPK_THREADS - 1) // TOPK_THREADS
            assert per <= 4, "the table scan holds at most 4 entries per thread"
            # winners: positions < k are written, columns t < n map through page t / P
            npages = (cfg.seq_lens[b] + P - 1) // P
            assert (n - 1) // P < npages
            assert np.all(pt[b, :npages] >= 0) and int(pt[b, :npages].max()) * P + P <= cfg.num_slots


def test_fault_revision_mla_and_step_workspace_at_c3():
    cfg, pt = _c3()
    B, Q, H, k, maxL = cfg.batch, cfg.q_per_seq, cfg.mla_heads, cfg.top_k, cfg.max_seq_len
    rows = B * Q
    # effective_split / mla_default_split of that revision
    ns = min(256 // rows, (k + 63) // 64)
    ns = max(1, min(ns, (k + 31) // 32))
    chunk = (k + ns - 1) // ns
    chunk = (chunk + MLA_TT - 1) // MLA_TT * MLA_TT
    assert (ns, chunk) == (8, 256)
    pieces = MLA_TT * (ROW_BF16 // 16)             # 2304 16-byte pieces per bf16 tile
    per = pieces // MLA_NT
    assert per * MLA_NT == pieces                  # every piece has one thread, none beyond
    for split in range(ns):
        j0, j1 = split * chunk, min(k, split * chunk + chunk)
        ntiles = (j1 - j0 + MLA_TT - 1) // MLA_TT if j1 > j0 else 0
        for it in range(ntiles):
            jb = j0 + it * MLA_TT
            g = np.arange(per)[:, None] * MLA_NT + np.arange(MLA_NT)[None, :]
            tk = g // (ROW_BF16 // 16)
            j = jb + tk
            assert np.all(j[j < j1] < k)           # slot-list reads inside the row's k entries
    # a selected slot is a page-mapped token of its sequence: inside the cache
    for b in range(B):
        npages = (cfg.seq_lens[b] + cfg.page_size - 1) // cfg.page_size
        top = int(pt[b, :npages].max()) * cfg.page_size + cfg.page_size - 1
        assert top < cfg.num_slots and (top + 1) * ROW_BF16 <= cfg.num_slots * ROW_BF16
    # partials [rows, ns, H, 512] and m, l [rows, ns, H]: the largest index each kernel forms
    o_elems, ml_elems = rows * ns * H * 512, rows * ns * H
    last_pr = ((rows - 1) * ns + ns - 1) * H + H - 1
    assert last_pr < ml_elems and last_pr * 512 + 511 < o_elems
    # the fused step's workspace: scores rows x ld, idx and slots rows x k, then the partials,
    # each region 256-byte aligned and disjoint
    def up(x):
        return (x + 255) // 256 * 256
    regions = [up(rows * maxL * 4), up(rows * k * 4), up(rows * k * 4), up(o_elems * 4), up(ml_elems * 4),
               up(ml_elems * 4)]
    offs = np.concatenate([[0], np.cumsum(regions)])
    assert np.all(np.diff(offs) >= [rows * maxL * 4, rows * k * 4, rows * k * 4, o_elems * 4, ml_elems * 4,
                                    ml_elems * 4])
