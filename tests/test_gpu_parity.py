"""GPU parity of every stage of the DSA decode path against the fp64 oracle, through the C ABI.

Sizes are chosen so the oracle finishes in seconds while the kernels still run several tiles
and a ragged tail; the workload-sized cases live in test_gpu_fullsize.py.
"""
import zlib

import numpy as np
import pytest
import torch

import dsa_inputs
import sparse_attention_10_amd as dsa
from oracle import dsa_oracle as O
from tests.gpu_helpers import (DEV, batch_of, check_attention, check_indexer, gpu_mla, gpu_scores,
                               oracle_mla, run_step)

pytestmark = pytest.mark.gpu


def _case(name, lens, seed, with_mla=True, with_indexer=True, **kw):
    cfg = dsa_inputs.scaled_config(name, lens, seed=seed, **kw)
    inp = dsa_inputs.make_inputs(cfg, with_mla=with_mla, with_indexer=with_indexer)
    return cfg, inp, dsa_inputs.to_torch(inp, cfg, DEV)


INDEXER_CASES = [
    ("c1", [4096], dict()),                                           # f32, vector path
    ("c2", [5000], dict()),                                           # bf16 matrix-core path, ragged tail
    ("c3", [4133, 300, 1, 8191, 2050], dict()),                       # ragged batch
    ("c5", [3000, 4097, 130], dict()),                                # fp8 keys, Q = 2
    ("c4", [64 + 1000], dict(q_per_seq=64)),                          # prefill-style causal block
    # the prefill path (16 rows per workgroup): a partial last block over two sequences, one
    # block over many key ranges, a page size that is not a power of two
    ("c4", [37 + 2000, 37 + 500], dict(q_per_seq=37)),
    ("c4", [16 + 70000], dict(q_per_seq=16)),
    ("c4", [48 + 3000], dict(q_per_seq=48, page_size=96)),
    ("c2", [777, 65], dict(q_per_seq=3)),                             # odd Q (one row per block)
    ("c2", [900], dict(idx_heads=8, idx_dim=32)),                     # vector path, bf16
    ("c5", [700], dict(idx_heads=8, idx_dim=32, q_per_seq=1)),        # vector path, fp8
    ("c2", [600], dict(page_size=16)),                                # another page size
    # long contexts: several 128-token tiles per workgroup (work >= 4096 tiles)
    ("c2", [131072, 131072, 60000, 60000, 60001, 59999, 4097, 77], dict()),
    ("c5", [131072, 100000, 70000, 9000], dict()),                    # fp8, Q = 2, two tiles per workgroup
    # more rows per sequence than one workgroup takes: rows in groups of two, a partial last group
    ("c2", [1000, 333], dict(q_per_seq=4)),
    ("c5", [2000, 515], dict(q_per_seq=4)),
    ("c2", [1500, 700], dict(q_per_seq=3)),
    # one row of one sequence: the key ring is 1, 2 or 4 blocks deep by the blocks per wave
    ("c2", [40000], dict()),
    ("c5", [3000], dict(q_per_seq=1)),
    ("c5", [40000], dict(q_per_seq=1)),
    ("c5", [1500], dict(q_per_seq=3)),
    ("c2", [700, 450], dict(q_per_seq=6)),
    ("c5", [300 + 20], dict(q_per_seq=20)),
    # page sizes that do not hold whole 16-token blocks
    ("c2", [1000, 37], dict(page_size=24)),
    ("c5", [500, 61], dict(page_size=1)),
]


@pytest.mark.parametrize("name,lens,kw", INDEXER_CASES, ids=[f"{c[0]}-{len(c[1])}x{max(c[1])}-{i}" for i, c in enumerate(INDEXER_CASES)])
def test_indexer_parity(name, lens, kw):
    cfg, inp, t = _case(name, lens, seed=101, with_mla=False, **kw)
    got = gpu_scores(cfg, t).cpu().numpy()
    ref = O.indexer_scores(inp["q_idx"], cfg.q_idx_dtype, inp["w"], inp["k_cache"], cfg.key_dtype,
                           inp["k_scale"], inp["seq_lens"], inp["page_table"], cfg.q_per_seq, cfg.page_size)
    check_indexer(cfg, got, ref, inp["seq_lens"])
    # columns at or past L_b are left untouched
    for b, L in enumerate(cfg.seq_lens):
        assert np.all(np.isnan(got[b, :, L:]))


def _topk_gpu(scores_np, seq_lens, Q, k, page_table=None, P=64, workspace=None):
    B = len(seq_lens)
    ld = scores_np.shape[-1]
    if page_table is None:
        page_table = np.arange((ld + P - 1) // P, dtype=np.int32)[None, :].repeat(B, 0)
    st = torch.from_numpy(np.ascontiguousarray(scores_np, dtype=np.float32)).to(DEV)
    sl = torch.tensor(seq_lens, dtype=torch.int32, device=DEV)
    pt = torch.from_numpy(np.ascontiguousarray(page_table)).to(DEV)
    batch = dsa.make_batch(sl, pt, Q, P, ld, int(page_table.max() + 1) * P)
    idx = torch.full((B, Q, k), -7, dtype=torch.int32, device=DEV)
    slots = torch.full((B, Q, k), -7, dtype=torch.int32, device=DEV)
    dsa.dsa_topk(batch, st, k, idx, slots, workspace=workspace)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), slots.cpu().numpy(), page_table


def _topk_ref(scores_np, seq_lens, Q, k, page_table, P=64):
    idx = O.topk(scores_np.astype(np.float64), seq_lens, Q, k)
    return idx, O.page_map(idx, page_table, P)


def _adversarial(kind, n, rng):
    if kind == "levels":
        return rng.choice(np.array([0.5, 0.25, 0.125, 1.0], np.float32), n)
    if kind == "allequal":
        return np.full(n, 0.375, np.float32)
    if kind == "zeros":
        return rng.choice(np.array([0.0, -0.0, 1e-30, -1e-30], np.float32), n)
    if kind == "neginf":
        x = rng.standard_normal(n).astype(np.float32)
        x[rng.random(n) < 0.7] = -np.inf
        return x
    if kind == "mixedsign":
        return (rng.standard_normal(n) * 1e3).astype(np.float32)
    if kind == "narrow":   # scores in a narrow positive band, like the indexer's
        return (0.0175 + 0.002 * rng.standard_normal(n)).astype(np.float32)
    if kind == "dupes":    # two values dominate so the k-th value is heavily tied
        x = np.full(n, 2.0, np.float32)
        x[rng.random(n) < 0.01] = 3.0
        return x
    raise ValueError(kind)


TOPK_CASES = [
    ("narrow", [32768], 1, 2048), ("narrow", [70000], 1, 2048), ("narrow", [131072], 1, 2048),
    ("levels", [5000, 3000], 1, 256), ("allequal", [4100], 1, 2048), ("zeros", [9000], 1, 1000),
    ("neginf", [20000], 1, 2048), ("mixedsign", [12345], 1, 1), ("dupes", [50000], 1, 2048),
    ("narrow", [2048, 2049, 10, 1], 1, 2048), ("narrow", [65536, 65536], 2, 2048),
    ("mixedsign", [40000], 1, 8192), ("levels", [1025], 3, 1024),
    # many long ragged rows at once: register part plus the streamed tail
    ("narrow", [131072, 100000, 70001, 65537, 40000, 32769, 5000, 2049], 1, 2048),
    ("dupes", [131072, 98304], 2, 2048),
    # two passes (rows of 64K+ columns in chunks of 16K): a last chunk of exactly k columns, one
    # of k + 1, a row inside the first chunk, rows that need no selection
    ("narrow", [65636, 18432, 18433, 3000, 2048, 50], 1, 2048),
    ("levels", [65536 + 17, 40000], 2, 2048),
]


@pytest.mark.parametrize("kind,lens,Q,k", TOPK_CASES, ids=[f"{c[0]}-{max(c[1])}-Q{c[2]}-k{c[3]}" for c in TOPK_CASES])
def test_topk_bit_exact(kind, lens, Q, k):
    rng = np.random.default_rng(zlib.crc32(f"{kind}-{lens}-{Q}-{k}".encode()))
    ld = max(lens)
    scores = np.stack([np.stack([_adversarial(kind, ld, rng) for _ in range(Q)]) for _ in lens])
    B = len(lens)
    pt = np.stack([rng.permutation((ld + 63) // 64).astype(np.int32) for _ in range(B)])
    idx_g, slots_g, _ = _topk_gpu(scores, lens, Q, k, pt)
    idx_r, slots_r = _topk_ref(scores, lens, Q, k, pt)
    assert np.array_equal(idx_g, idx_r)
    assert np.array_equal(slots_g, slots_r)


def test_topk_on_indexer_scores_bit_exact():
    cfg, inp, t = _case("c3", [9000, 4097, 70000], seed=102, with_mla=False)
    s = gpu_scores(cfg, t, fill=float("-inf"))
    sn = s.cpu().numpy()
    idx_g, slots_g, _ = _topk_gpu(sn, cfg.seq_lens, 1, cfg.top_k, inp["page_table"])
    idx_r, slots_r = _topk_ref(sn, cfg.seq_lens, 1, cfg.top_k, inp["page_table"])
    assert np.array_equal(idx_g, idx_r) and np.array_equal(slots_g, slots_r)


def test_page_map_bit_exact():
    rng = np.random.default_rng(5)
    B, Q, k, P, maxP = 4, 2, 300, 64, 40
    pt = rng.integers(0, 1000, (B, maxP)).astype(np.int32)
    idx = rng.integers(-1, maxP * P, (B, Q, k)).astype(np.int32)
    sl = torch.full((B,), maxP * P, dtype=torch.int32, device=DEV)
    pt_d, idx_d = torch.from_numpy(pt).to(DEV), torch.from_numpy(idx).to(DEV)
    batch = dsa.make_batch(sl, pt_d, Q, P, maxP * P, 1000 * P)
    out = torch.full((B, Q, k), -7, dtype=torch.int32, device=DEV)
    dsa.dsa_page_map(batch, idx_d, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), O.page_map(idx, pt, P))


def _random_slots(cfg, rng, k, frac_invalid=0.0):
    slots = np.stack([np.stack([rng.choice(cfg.num_slots, k, replace=False) for _ in range(cfg.q_per_seq)])
                      for _ in range(cfg.batch)]).astype(np.int32)
    if frac_invalid:
        slots[rng.random(slots.shape) < frac_invalid] = -1
    return slots


MLA_CASES = [
    # name, lens, k, H, n_split, invalid fraction
    ("c2", [3000], 2048, 64, 1, 0.0),
    ("c2", [3000], 2048, 64, 0, 0.0),
    ("c2", [3000], 2048, 64, 7, 0.0),
    ("c2", [3000], 2048, 64, 64, 0.0),
    ("c2", [3000], 100, 64, 3, 0.1),
    ("c3", [2500, 700, 4000], 512, 64, 0, 0.3),
    ("c5", [3000, 2000], 2048, 64, 0, 0.0),
    ("c5", [3000], 333, 64, 2, 0.05),
    ("c2", [1500], 256, 16, 0, 0.0),
    ("c2", [1500], 256, 32, 2, 0.0),
    ("c2", [1500], 256, 48, 1, 0.0),
    ("c1", [4096], 256, 16, 0, 0.0),
    ("c1", [900], 300, 16, 0, 0.2),
    # many query rows at once (32 rows x 8 chunks; 64 sequences x 2 fp8 rows x 2 chunks)
    ("c3", [200] * 32, 2048, 64, 0, 0.0),
    ("c5", [300] * 64, 512, 64, 2, 0.0),
    # chunks above the wide fp8 kernel's 1024-row and the bf16 ring kernel's 2048-row staging
    # limits take the 8-wave kernels with register-staged (bf16) or narrower (fp8) tiles
    ("c5", [5000], 4096, 64, 1, 0.02),
    ("c2", [5000], 4096, 64, 1, 0.02),
    ("c2", [5000], 4096, 32, 2, 0.0),
    # fp8 with fewer heads than the wide kernel's four groups, partial last tiles
    ("c5", [1500], 200, 32, 3, 0.1),
    ("c5", [1500], 200, 48, 0, 0.0),
]


@pytest.mark.parametrize("name,lens,k,H,ns,inv", MLA_CASES, ids=[f"{c[0]}-k{c[2]}-H{c[3]}-s{c[4]}-inv{c[5]}" for c in MLA_CASES])
def test_sparse_mla_parity(name, lens, k, H, ns, inv):
    Q = 2 if name == "c5" else 1
    cfg, inp, t = _case(name, lens, seed=103, mla_heads=H, top_k=k, q_per_seq=Q)
    rng = np.random.default_rng(7)
    slots = _random_slots(cfg, rng, k, inv)
    out, lse = gpu_mla(cfg, t, torch.from_numpy(slots).to(DEV), n_split=ns)
    ro, rl = oracle_mla(cfg, inp, slots)
    check_attention(out.cpu().numpy(), ro, lse.cpu().numpy(), rl)


def test_sparse_mla_empty_selection_and_single_row():
    cfg, inp, t = _case("c2", [500], seed=104, top_k=64)
    slots = np.full((1, 1, 64), -1, np.int32)
    out, lse = gpu_mla(cfg, t, torch.from_numpy(slots).to(DEV), n_split=2)
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))
    slots[0, 0, 37] = 123
    out, lse = gpu_mla(cfg, t, torch.from_numpy(slots).to(DEV), n_split=2)
    ro, rl = oracle_mla(cfg, inp, slots)
    check_attention(out.cpu().numpy(), ro, lse.cpu().numpy(), rl)
    # one selected row: the output is that row's V (up to the bf16 P weight of exactly 1)
    v = O.dequantize(inp["kv_cache"][123:124], "bf16")[0, :512]
    assert np.abs(out.cpu().numpy()[0, 0] - v[None, :]).max() < 1e-6


@pytest.mark.parametrize("name,ns,qps", [("c2", 1, 1), ("c2", 2, 1), ("c2", 1, 5), ("c2", 2, 5), ("c5", 1, 1),
                                         ("c5", 2, 1)])
def test_sparse_mla_wide_logit_range(name, ns, qps):
    """Heads whose largest logit lies far above or far below the kernels' first-tile reference.

    Head 3 meets one selected row, late in the chunk, whose logit lies more than 64 (log2
    units) above the rest; head 7 sees every logit near -200 and, in the second chunk, a first
    tile with no live slot.  Both need the second pass of the kernels; the expected values are
    the oracle's.  The logits are exact products accumulated in fp32 (e4m3 codes are widened to
    bf16), but P enters the P.V product as bf16 (fp8 rows: with the token's scale folded in), so
    a token's contribution carries a relative rounding of up to 2^-9; the boosted row's large
    norm makes that visible in every head of row 0, so the output bound there is relative to
    each head's output scale (2^-8), while the direction (cosine) and lse keep the strict bar.
    One bf16 query row runs on the 16-head kernel, five on the 64-head one."""
    cfg, inp, _ = _case(name, [3000], seed=106, top_k=512, q_per_seq=qps)
    rng = np.random.default_rng(12)
    slots = _random_slots(cfg, rng, 512)
    slots[0, 0, 256:384] = -1                                    # chunk 1 (ns=2) starts with a dead tile
    q = O.dequantize(inp["q_mla"], "bf16").copy()
    kv = O.dequantize(inp["kv_cache"], cfg.kv_dtype, inp["kv_scale"]).copy()
    boost = int(slots[0, 0, 200])
    rest = slots[0, 1:]
    rest[rest == boost] = -1                                     # only row 0 meets the boosted row
    fp8 = cfg.kv_dtype == "fp8"
    kv[boost] = q[0, 0, 3] * (1300.0 if fp8 else 3000.0)        # head 3: one dominant logit
    kv[:, 575] = 30.0                                            # a shared RoPE component ...
    q[0, 0, 7, 575] = -110.0                                     # ... that pushes head 7's logits to about -200
    inp["q_mla"] = dsa_inputs.encode_bf16(q)
    if fp8:
        inp["kv_cache"], inp["kv_scale"] = dsa_inputs.encode_fp8_rows(kv)
    else:
        inp["kv_cache"] = dsa_inputs.encode_bf16(kv)
    t = dsa_inputs.to_torch(inp, cfg, DEV)
    out, lse = gpu_mla(cfg, t, torch.from_numpy(slots).to(DEV), n_split=ns)
    ro, rl = oracle_mla(cfg, inp, slots)
    og, lg = out.cpu().numpy().astype(np.float64), lse.cpu().numpy()
    assert np.isfinite(og).all() and np.isfinite(lg).all()
    # Row 0 meets the boosted row, whose V values reach a few hundred.  P enters P.V rounded to
    # bf16 (fp8 rows: P * scale), which moves each token's weight by at most 2^-9 of itself; the
    # output (normalised by the rounded weights, an exact convex combination) then moves by at
    # most 2^-9 of its own scale and keeps its direction.  Where the kernel's reference is the
    # head's maximum (after a second pass) the dominant weight is exactly 1 and this rounding
    # vanishes, but which heads get a second pass depends on the kernel's grouping of heads.
    g0, r0 = og[0, 0], ro[0, 0]
    scale = np.maximum(1.0, np.abs(r0).max(axis=-1, keepdims=True))
    err = (np.abs(g0 - r0) / scale).max()
    assert err <= 2.0 ** -8, f"scaled max-abs error {err:.3e}"
    cos = (g0 * r0).sum(1) / (np.linalg.norm(g0, axis=1) * np.linalg.norm(r0, axis=1))
    assert cos.min() >= 0.99999, f"min cosine {cos.min():.8f}"
    assert (np.abs(lg[0, 0] - rl[0, 0]) / np.maximum(1.0, np.abs(rl[0, 0]))).max() <= 1e-4
    if qps > 1:   # the other rows never meet the boosted row: the plain bar
        check_attention(og[0, 1:], ro[0, 1:], lg[0, 1:], rl[0, 1:])
    if not fp8:
        # head 3 has one row far above the rest (a second pass in its workgroup): that row's V
        assert np.abs(og[0, 0, 3] - ro[0, 0, 3]).max() <= 1e-5 * np.abs(ro[0, 0, 3]).max()
        assert abs(lg[0, 0, 3] - rl[0, 0, 3]) <= 1e-4 * abs(rl[0, 0, 3])


@pytest.mark.parametrize("name", ["c5", "c2"])
def test_sparse_mla_tiny_query_heads(name):
    """Query heads far below the normal range: head 5's values are bf16 subnormals (about
    2^-130), head 6 is all zeros.  The fp8 kernel scales each head's q by a power of two before
    splitting it into e4m3 parts; that scale must stay finite for such heads.  Their logits are
    ~0, so their outputs are the mean of the selected V rows."""
    cfg, inp, _ = _case(name, [2000], seed=107, top_k=512, q_per_seq=1)
    q = O.dequantize(inp["q_mla"], "bf16").copy()
    q[0, 0, 5] *= 2.0 ** -125
    q[0, 0, 6] = 0.0
    inp["q_mla"] = dsa_inputs.encode_bf16(q)
    assert np.abs(O.dequantize(inp["q_mla"], "bf16")[0, 0, 5]).max() < 2.0 ** -119
    t = dsa_inputs.to_torch(inp, cfg, DEV)
    rng = np.random.default_rng(13)
    slots = _random_slots(cfg, rng, 512)
    for ns in (1, 2):
        out, lse = gpu_mla(cfg, t, torch.from_numpy(slots).to(DEV), n_split=ns)
        ro, rl = oracle_mla(cfg, inp, slots)
        check_attention(out.cpu().numpy(), ro, lse.cpu().numpy(), rl)


def test_split_combine_parity_direct():
    rng = np.random.default_rng(9)
    rows, ns, H = 3, 5, 64
    m = rng.standard_normal((rows, ns, H)).astype(np.float32) * 3
    l = (rng.random((rows, ns, H)) * 10).astype(np.float32)
    l[0, 2, :] = 0.0
    m[0, 2, :] = -np.inf
    l[1, :, 5] = 0.0
    m[1, :, 5] = -np.inf                      # (row 1, head 5) has no live chunk
    o = rng.standard_normal((rows, ns, H, 512)).astype(np.float32)
    out = torch.full((rows, H, 512), float("nan"), device=DEV)
    lse = torch.full((rows, H), float("nan"), device=DEV)
    dsa.dsa_mla_combine(torch.from_numpy(o).to(DEV), torch.from_numpy(m).to(DEV), torch.from_numpy(l).to(DEV),
                        out, lse)
    torch.cuda.synchronize()
    for r in range(rows):
        ro, rl = O.combine_splits(m[r].astype(np.float64), l[r].astype(np.float64), o[r].astype(np.float64))
        assert np.abs(out[r].cpu().numpy() - ro).max() < 1e-5
        lg = lse[r].cpu().numpy()
        assert np.array_equal(np.isneginf(lg), np.isneginf(rl))
        fin = np.isfinite(rl)
        assert np.abs(lg[fin] - rl[fin]).max() < 1e-5


@pytest.mark.parametrize("ns", [1, 2, 7, 32])
def test_split_invariance_gpu(ns):
    cfg, inp, t = _case("c2", [3000], seed=105)
    slots = _random_slots(cfg, np.random.default_rng(11), cfg.top_k)
    st = torch.from_numpy(slots).to(DEV)
    out1, lse1 = gpu_mla(cfg, t, st, n_split=1)
    outn, lsen = gpu_mla(cfg, t, st, n_split=ns)
    assert torch.allclose(out1, outn, rtol=0, atol=1e-5)
    assert torch.allclose(lse1, lsen, rtol=0, atol=1e-5)


STEP_CASES = [("c1", [4096], dict()), ("c2", [6000], dict()), ("c3", [4100, 2500, 9000], dict()),
              ("c5", [5000, 3000], dict()), ("c4", [64 + 3000], dict(q_per_seq=64, top_k=512)),
              # deeper speculative verify: draft depth 3 (4 rows per sequence, fp8 caches) and 2
              ("c5", [5000, 3000, 2100], dict(q_per_seq=4)), ("c2", [4500, 2600], dict(q_per_seq=3)),
              # the largest batch of the indexer's length-balanced key ranges (128 sequences, some
              # below k), and a batch beyond it (200 fp8 sequences: ranges per sequence)
              ("c3", [int(x) for x in np.random.default_rng(128).integers(100, 2600, size=128)], dict()),
              ("c5", [int(x) for x in np.random.default_rng(200).integers(2, 2600, size=200)], dict(q_per_seq=1)),
              # verify rows sharing their indexer query (nested, nearly equal selections) with the
              # MLA's rows of a sequence on one XCD: 16 fp8 sequences x 2 rows, 8 bf16 x 3 rows
              ("c5", [int(x) for x in np.random.default_rng(16).integers(2100, 3000, size=16)],
               dict(q_per_seq=2, shared_index_query=True)),
              ("c2", [int(x) for x in np.random.default_rng(8).integers(2100, 4000, size=8)],
               dict(q_per_seq=3, shared_index_query=True))]


@pytest.mark.parametrize("name,lens,kw", STEP_CASES, ids=[f"{c[0]}-B{len(c[1])}" + ("-shared" if c[2].get("shared_index_query") else "")
                              for c in STEP_CASES])
def test_decode_step_staged(name, lens, kw):
    """Staged protocol: (1) the step's scores against the oracle; (2) its selection against the
    oracle's top-k run on the step's own f32 scores (bit-exact) and its slots against the page
    map (bit-exact); (3) its attention output against the oracle on the step's own slots; and
    (4) its selection against the oracle's fp64 selection, where every disagreement must sit
    within 2e-5 * max|s| of the k-th score."""
    cfg, inp, t = _case(name, lens, seed=106, **kw)
    _check_staged(cfg, inp, t)


def test_decode_step_staged_batch32_ragged():
    """The staged protocol on a batch of 32 ragged sequences (contexts 515-11865): the indexer's
    balanced key-range partition at B = 32, its ranges crossing sequence boundaries, 32 top-k rows
    and 32 MLA rows.  tests/test_c3_bounds_cpu.py emulates this exact configuration's index
    arithmetic on the CPU."""
    from tests.test_c3_bounds_cpu import scaled32
    cfg, _ = scaled32()
    inp = dsa_inputs.make_inputs(cfg)
    _check_staged(cfg, inp, dsa_inputs.to_torch(inp, cfg, DEV))


def _check_staged(cfg, inp, t):
    r = run_step(cfg, t)
    s_g = r["scores"].cpu().numpy()
    s_ref = O.indexer_scores(inp["q_idx"], cfg.q_idx_dtype, inp["w"], inp["k_cache"], cfg.key_dtype,
                             inp["k_scale"], inp["seq_lens"], inp["page_table"], cfg.q_per_seq, cfg.page_size)
    check_indexer(cfg, s_g, s_ref, inp["seq_lens"])
    idx_g, slots_g = r["idx"].cpu().numpy(), r["slots"].cpu().numpy()
    idx_r = O.topk(np.where(np.isnan(s_g), -np.inf, s_g).astype(np.float64), inp["seq_lens"], cfg.q_per_seq,
                   cfg.top_k)
    assert np.array_equal(idx_g, idx_r)
    assert np.array_equal(slots_g, O.page_map(idx_g, inp["page_table"], cfg.page_size))
    ro, rl = oracle_mla(cfg, inp, slots_g)
    check_attention(r["out"].cpu().numpy(), ro, r["lse"].cpu().numpy(), rl)
    # (4) the fp64 selection differs only near the k-th score
    idx64 = O.topk(s_ref, inp["seq_lens"], cfg.q_per_seq, cfg.top_k)
    pos = O.query_positions(inp["seq_lens"], cfg.q_per_seq)
    for b in range(cfg.batch):
        for i in range(cfg.q_per_seq):
            a, c = set(idx_g[b, i][idx_g[b, i] >= 0]), set(idx64[b, i][idx64[b, i] >= 0])
            if a == c:
                continue
            row = s_ref[b, i, :pos[b, i] + 1]
            kth = np.sort(row)[::-1][cfg.top_k - 1]
            for tok in a ^ c:
                assert abs(row[tok] - kth) <= 2e-5 * np.abs(row).max()


@pytest.mark.parametrize("name,lens,Q", [("c2", [1500], 1), ("c5", [700, 1200], 2), ("c1", [300], 1),
                                         ("c5", [900, 1300, 260], 4)])
def test_decode_step_dense_when_k_covers_context(name, lens, Q):
    """k >= context: the step must equal dense attention whatever the indexer's numerics."""
    cfg, inp, t = _case(name, lens, seed=107, top_k=max(lens), q_per_seq=Q)
    r = run_step(cfg, t, debug=False)
    do, dl = O.dense_mla(inp["q_mla"], cfg.q_mla_dtype, inp["kv_cache"], cfg.kv_dtype, inp["kv_scale"],
                         inp["seq_lens"], inp["page_table"], Q, cfg.page_size, cfg.sm_scale)
    check_attention(r["out"].cpu().numpy(), do, r["lse"].cpu().numpy(), dl)


@pytest.mark.parametrize("lens,Q,block", [([64 + 1000], 48, 16), ([40 + 700, 40 + 2100], 40, 16),
                                           ([64 + 3000], 64, 32)])
def test_prefill_row_blocks_match_one_block(lens, Q, block):
    """Chunked prefill scored and ranked in row blocks that reuse one score buffer (ragged last
    block, two sequences) gives exactly the step of one block: every score element is the same
    matrix-core sum whatever the workgroup partition, so indices, slots and attention agree bit
    for bit; one block is itself checked against the oracle by the staged step tests."""
    cfg = dsa_inputs.scaled_config("c4", lens, seed=117, q_per_seq=Q, top_k=256)
    inp = dsa_inputs.make_inputs(cfg)
    t = dsa_inputs.to_torch(inp, cfg, DEV)

    def step(rows_per_block):
        B, H, k = cfg.batch, cfg.mla_heads, cfg.top_k
        out = torch.full((B, Q, H, 512), float("nan"), dtype=torch.float32, device=DEV)
        lse = torch.full((B, Q, H), float("nan"), dtype=torch.float32, device=DEV)
        idx = torch.full((B, Q, k), -7, dtype=torch.int32, device=DEV)
        slots = torch.full((B, Q, k), -7, dtype=torch.int32, device=DEV)
        args = dsa.decode_step_args(batch_of(cfg, t), t["q_idx"], t["w"], t["k_cache"], t["k_scale"], k,
                                    t["q_mla"], t["kv_cache"], t["kv_scale"], cfg.sm_scale, out, lse, 0,
                                    None, idx, slots, prefill_rows_per_block=rows_per_block)
        ws = torch.empty(max(1, dsa.decode_step_workspace_bytes(args)), dtype=torch.uint8, device=DEV)
        dsa.dsa_decode_step(args, ws)
        torch.cuda.synchronize()
        return out, lse, idx, slots

    whole = step(Q)
    blocked = step(block)
    for a, b in zip(blocked, whole):
        assert torch.equal(a, b)


def test_decode_step_deterministic():
    cfg, inp, t = _case("c3", [5000, 3000, 7000], seed=108)
    r1 = run_step(cfg, t)
    r2 = run_step(cfg, t)
    for key in ("out", "lse", "scores", "idx", "slots"):
        a, b = r1[key].cpu(), r2[key].cpu()
        assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                           b.view(torch.int32) if b.dtype == torch.float32 else b), key


# Long rows: the candidate path and the narrowing rounds (a bin of more than 4096 equal keys),
# rows that need no selection in the same launch, a page size that is not a power of two, a k
# above the candidate cap, and rows whose scores start off 16-byte alignment (Q = 2, odd ld).
LONG_CASES = [
    ("narrow", [40000, 1000, 23456], 1, 2048, 64),
    ("zeros", [40000], 1, 2048, 64),
    ("levels", [33000, 17000], 1, 3000, 48),
    ("allequal", [65536], 1, 8192, 64),
    ("mixedsign", [16384, 16385], 2, 1, 64),
    ("narrow", [262144], 1, 2048, 64),
    ("narrow", [30001, 29999, 777], 3, 2048, 64),
    ("dupes", [70001, 5], 1, 100, 16),
]


@pytest.mark.parametrize("kind,lens,Q,k,P", LONG_CASES, ids=[f"{c[0]}-{len(c[1])}x{max(c[1])}-Q{c[2]}-k{c[3]}-P{c[4]}" for c in LONG_CASES])
def test_topk_long_rows(kind, lens, Q, k, P):
    rng = np.random.default_rng(zlib.crc32(f"coop-{kind}-{lens}-{Q}-{k}-{P}".encode()))
    ld = max(lens)
    scores = np.stack([np.stack([_adversarial(kind, ld, rng) for _ in range(Q)]) for _ in lens])
    B = len(lens)
    pt = np.stack([rng.permutation((ld + P - 1) // P).astype(np.int32) for _ in range(B)])
    idx_g, slots_g, _ = _topk_gpu(scores, lens, Q, k, pt, P=P)
    idx_r, slots_r = _topk_ref(scores, lens, Q, k, pt, P=P)
    assert np.array_equal(idx_g, idx_r)
    assert np.array_equal(slots_g, slots_r)


def test_decode_step_hip_graph_replay():
    """The step captured in a HIP graph replays to the eager result, every replay."""
    cfg, inp, t = _case("c2", [40000], seed=109)
    B, Q, H, k = cfg.batch, cfg.q_per_seq, cfg.mla_heads, cfg.top_k
    out = torch.zeros((B, Q, H, 512), dtype=torch.float32, device=DEV)
    lse = torch.zeros((B, Q, H), dtype=torch.float32, device=DEV)
    args = dsa.decode_step_args(batch_of(cfg, t), t["q_idx"], t["w"], t["k_cache"], t["k_scale"], k,
                                t["q_mla"], t["kv_cache"], t["kv_scale"], cfg.sm_scale, out, lse)
    ws = torch.zeros(dsa.decode_step_workspace_bytes(args), dtype=torch.uint8, device=DEV)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        dsa.dsa_decode_step(args, ws, stream=s)
    torch.cuda.synchronize()
    eager_o, eager_l = out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        dsa.dsa_decode_step(args, ws, stream=s)
    for rep in range(4):
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_o), f"replay {rep}"
        assert torch.equal(lse, eager_l), f"replay {rep}"


def test_multi_layer_graph_replay_matches_oracle():
    """Several layers' decode steps (each with its own caches, one shared workspace) captured in
    one HIP graph, the way a model's per-token forward replays them.  The first replay is checked
    layer by layer against the oracle with the staged protocol; every later replay, with eager
    work between replays, must reproduce it bit for bit."""
    layers = [("c2", [3000], dict()), ("c5", [2500, 1800], dict()), ("c2", [900], dict(q_per_seq=3)),
              ("c5", [4100], dict())]
    cases, args, bufs = [], [], []
    for n, (name, lens, kw) in enumerate(layers):
        cfg, inp, t = _case(name, lens, seed=120 + n, **kw)
        B, Q, H, k = cfg.batch, cfg.q_per_seq, cfg.mla_heads, cfg.top_k
        b = dict(out=torch.zeros((B, Q, H, 512), device=DEV), lse=torch.zeros((B, Q, H), device=DEV),
                 scores=torch.zeros((B, Q, cfg.max_seq_len), device=DEV),
                 idx=torch.zeros((B, Q, k), dtype=torch.int32, device=DEV),
                 slots=torch.zeros((B, Q, k), dtype=torch.int32, device=DEV))
        args.append(dsa.decode_step_args(batch_of(cfg, t), t["q_idx"], t["w"], t["k_cache"], t["k_scale"], k,
                                         t["q_mla"], t["kv_cache"], t["kv_scale"], cfg.sm_scale, b["out"],
                                         b["lse"], 0, b["scores"], b["idx"], b["slots"]))
        cases.append((cfg, inp, t))
        bufs.append(b)
    ws = torch.zeros(max(dsa.decode_step_workspace_bytes(a) for a in args), dtype=torch.uint8, device=DEV)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for a in args:
            dsa.dsa_decode_step(a, ws, stream=s)
    first = None
    for rep in range(3):
        for b in bufs:                      # eager work between replays
            for v in b.values():
                v.fill_(-3)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        got = [{k: v.cpu() for k, v in b.items()} for b in bufs]
        if first is None:
            first = got
            for (cfg, inp, _), r in zip(cases, got):
                s_g = r["scores"].numpy()
                s_ref = O.indexer_scores(inp["q_idx"], cfg.q_idx_dtype, inp["w"], inp["k_cache"], cfg.key_dtype,
                                         inp["k_scale"], inp["seq_lens"], inp["page_table"], cfg.q_per_seq,
                                         cfg.page_size)
                check_indexer(cfg, s_g, s_ref, inp["seq_lens"])
                idx_g, slots_g = r["idx"].numpy(), r["slots"].numpy()
                assert np.array_equal(idx_g, O.topk(np.where(np.isnan(s_g), -np.inf, s_g).astype(np.float64),
                                                    inp["seq_lens"], cfg.q_per_seq, cfg.top_k))
                assert np.array_equal(slots_g, O.page_map(idx_g, inp["page_table"], cfg.page_size))
                ro, rl = oracle_mla(cfg, inp, slots_g)
                check_attention(r["out"].numpy(), ro, r["lse"].numpy(), rl)
        else:
            for n, (r0, r) in enumerate(zip(first, got)):
                for key in r:
                    assert torch.equal(r0[key].view(torch.int32) if r0[key].dtype == torch.float32 else r0[key],
                                       r[key].view(torch.int32) if r[key].dtype == torch.float32 else r[key]), \
                        f"replay {rep}, layer {n}, {key}"


def test_abi_errors_leave_outputs_untouched():
    cfg, inp, t = _case("c2", [600], seed=110)
    out = torch.full((1, 1, 64, 512), 3.0, device=DEV)
    slots = torch.zeros((1, 1, 64), dtype=torch.int32, device=DEV)
    with pytest.raises(dsa.DsaError) as e:
        dsa.dsa_sparse_mla_decode(t["q_mla"][:, :, :8].contiguous(), t["kv_cache"], None, slots, 0.1,
                                  out[:, :, :8].contiguous())
    assert e.value.status == dsa.DSA_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
