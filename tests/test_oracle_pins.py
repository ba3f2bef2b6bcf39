"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test checks the oracle against a brute-force loop written separately, a
closed form, an invariant the mathematics fixes, a hand-derived example
(tests/golden/tiny_hand.json) or an external library routine.  They are chosen
so that a dropped term, a wrong sign or index, or a transposed operand in the
oracle fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import dsa_inputs
from oracle import dsa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tiny_hand.json")


def _f(x):
    if isinstance(x, str):
        return float(x)
    if isinstance(x, list):
        return [_f(v) for v in x]
    return x


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as fh:
        return json.load(fh)


# ---------------------------------------------------------------------------
# dtype decoders against torch's own conversions (an external routine)

def test_e4m3fn_all_codes_match_torch():
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.decode_e4m3fn(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))
    assert np.nanmax(np.abs(got)) == 448.0
    assert int(np.isnan(got).sum()) == 2          # S.1111.111 for both signs only


def test_bf16_all_codes_match_torch():
    import torch
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = O.decode_bf16(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])


def test_fp8_hand_values(golden):
    g = golden["fp8_e4m3fn"]
    got = O.decode_e4m3fn(np.array(g["codes"], dtype=np.uint8))
    exp = np.array(_f(g["values"]))
    assert np.array_equal(got, exp)
    assert np.signbit(got[-1])


def test_dequantize_fp8_applies_row_scale():
    codes = np.array([[0x38, 0x40], [0x38, 0xB8]], dtype=np.uint8)   # [1, 2], [1, -1]
    scale = np.array([0.5, 3.0], dtype=np.float32)
    assert np.array_equal(O.dequantize(codes, "fp8", scale), np.array([[0.5, 1.0], [3.0, -3.0]]))


# ---------------------------------------------------------------------------
# positions and cache format

def test_query_positions_workload_shapes():
    # chunked prefill: 4096 queries appended to a 65536-token prefix
    pos = O.query_positions([65536 + 4096], 4096)
    assert pos[0, 0] == 65536 and pos[0, -1] == 65536 + 4095
    # speculative verify: two rows at the end of a 65536-token context
    assert O.query_positions([65536], 2).tolist() == [[65534, 65535]]
    assert O.query_positions([7, 9], 1).tolist() == [[6], [8]]


def test_cache_row_format():
    # one compressed row of 576 values per token, V = the first 512; the pages'
    # "57x smaller than 32,768 floats per token" is 32768 / 576
    assert O.ROW_DIM == 576 and O.V_DIM == 512 and O.ROW_DIM - O.V_DIM == 64
    assert round(32768 / O.ROW_DIM) == 57
    cfg = dsa_inputs.scaled_config("c2", [100], seed=5)
    inp = dsa_inputs.make_inputs(cfg, with_indexer=False)
    assert inp["kv_cache"].shape == (cfg.num_slots, 576)
    assert inp["q_mla"].shape[-1] == 576


# ---------------------------------------------------------------------------
# indexer

def _brute_indexer(q, w, k, page_table, seq_lens, Q, P):
    """Pure-Python loops over (b, i, t, h, d)."""
    B = len(seq_lens)
    out = {}
    for b in range(B):
        for i in range(Q):
            pos = seq_lens[b] - Q + i
            for t in range(seq_lens[b]):
                if t > pos:
                    out[(b, i, t)] = -math.inf
                    continue
                slot = int(page_table[b][t // P]) * P + t % P
                acc = 0.0
                for h in range(len(w[b][i])):
                    dot = 0.0
                    for d in range(len(q[b][i][h])):
                        dot += float(q[b][i][h][d]) * float(k[slot][d])
                    acc += float(w[b][i][h]) * (dot if dot > 0 else 0.0)
                out[(b, i, t)] = acc
    return out


def test_indexer_hand_example(golden):
    g = golden["indexer"]
    q = np.array(g["q"], dtype=np.float32)
    w = np.array(g["w"], dtype=np.float32)
    k = np.array(g["k_cache"], dtype=np.float32)
    pt = np.array(g["page_table"], dtype=np.int32)
    s = O.indexer_scores(q, "f32", w, k, "f32", None, g["seq_lens"], pt, 2, g["page_size"])
    assert np.array_equal(s, np.array(_f(g["expected_scores"])))
    idx = O.topk(s, g["seq_lens"], 2, g["top_k"])
    assert idx.tolist() == g["expected_idx"]
    assert O.page_map(idx, pt, g["page_size"]).tolist() == g["expected_slots"]


def test_indexer_brute_force_tiny():
    rng = np.random.default_rng(7)
    P, Q, Hi, Di = 64, 2, 3, 5
    lens = [130, 77]
    npages = [3, 2]
    perm = rng.permutation(sum(npages)).astype(np.int32)
    pt = np.full((2, 3), -1, np.int32)
    pt[0, :3] = perm[:3]
    pt[1, :2] = perm[3:]
    q = rng.standard_normal((2, Q, Hi, Di)).astype(np.float32)
    w = rng.random((2, Q, Hi)).astype(np.float32)
    k = rng.standard_normal((sum(npages) * P, Di)).astype(np.float32)
    s = O.indexer_scores(q, "f32", w, k, "f32", None, lens, pt, Q, P)
    ref = _brute_indexer(q.tolist(), w.tolist(), k.tolist(), pt.tolist(), lens, Q, P)
    for (b, i, t), v in ref.items():
        if math.isinf(v):
            assert s[b, i, t] == -math.inf
        else:
            assert abs(s[b, i, t] - v) <= 1e-14 * max(1.0, abs(v))
    # columns past L_b of the shorter sequence are -inf as well
    assert np.all(np.isneginf(s[1, :, 77:]))


def test_indexer_gemv_special_case():
    # one head, w = 1, non-negative q and keys: ReLU is the identity and the
    # score row is the matrix-vector product K q (textbook GEMV)
    rng = np.random.default_rng(3)
    P, L, Di = 64, 200, 16
    pt = rng.permutation(4).astype(np.int32)[None, :]
    k = rng.random((256, Di)).astype(np.float32)
    q = rng.random((1, 1, 1, Di)).astype(np.float32)
    w = np.ones((1, 1, 1), np.float32)
    s = O.indexer_scores(q, "f32", w, k, "f32", None, [L], pt, 1, P)
    slots = np.array([pt[0, t // P] * P + t % P for t in range(L)])
    gemv = k[slots].astype(np.float64).dot(q[0, 0, 0].astype(np.float64))
    assert np.allclose(s[0, 0, :L], gemv, rtol=1e-15, atol=0)


def _small_indexer_case(seed, key_dtype="bf16", Q=2):
    cfg = dsa_inputs.scaled_config("c2", [150, 64 * 3], seed=seed, q_per_seq=Q, idx_heads=8,
                                   idx_dim=32, key_dtype=key_dtype)
    return cfg, dsa_inputs.make_inputs(cfg, with_mla=False)


def _scores(cfg, inp, **kw):
    a = dict(q=inp["q_idx"], q_dtype=cfg.q_idx_dtype, w=inp["w"], k_cache=inp["k_cache"],
             k_dtype=cfg.key_dtype, k_scale=inp["k_scale"], seq_lens=inp["seq_lens"],
             page_table=inp["page_table"], q_per_seq=cfg.q_per_seq, page_size=cfg.page_size)
    a.update(kw)
    return O.indexer_scores(**a)


def test_indexer_invariants():
    cfg, inp = _small_indexer_case(11)
    s = _scores(cfg, inp)
    fin = np.isfinite(s)
    assert np.all(s[fin] >= 0)                                  # w >= 0 => s >= 0
    # linear in w
    # (dyadic weights keep w1 + 2 w2 exact in f32)
    r = np.random.default_rng(5)
    w1 = (r.integers(0, 64, inp["w"].shape) / 64.0).astype(np.float32)
    w2 = (r.integers(0, 64, inp["w"].shape) / 128.0).astype(np.float32)
    s1 = _scores(cfg, inp, w=w1)
    s2 = _scores(cfg, inp, w=w2)
    s12 = _scores(cfg, inp, w=(w1 + 2.0 * w2).astype(np.float32))
    assert np.allclose(s12[fin], s1[fin] + 2.0 * s2[fin], rtol=1e-13, atol=1e-15)
    # positive homogeneity in q (alpha = 2 keeps bf16 values exact)
    qd = O.dequantize(inp["q_idx"], "bf16") * 2.0
    s3 = _scores(cfg, inp, q=qd, q_dtype="f64")
    assert np.array_equal(s3[fin], 2.0 * s[fin])
    # causal mask: row i sees pos(b,i) + 1 tokens
    pos = O.query_positions(inp["seq_lens"], cfg.q_per_seq)
    for b in range(cfg.batch):
        for i in range(cfg.q_per_seq):
            assert np.all(np.isfinite(s[b, i, :pos[b, i] + 1]))
            assert np.all(np.isneginf(s[b, i, pos[b, i] + 1:]))


def test_indexer_fp8_equals_predequantized():
    cfg, inp = _small_indexer_case(12, key_dtype="fp8")
    s = _scores(cfg, inp)
    kd = O.decode_e4m3fn(inp["k_cache"]) * inp["k_scale"].astype(np.float64)[:, None]
    s2 = _scores(cfg, inp, k_cache=kd, k_dtype="f64", k_scale=None)
    assert np.array_equal(s, s2)


def test_indexer_page_relabel_invariance():
    cfg, inp = _small_indexer_case(13)
    s = _scores(cfg, inp)
    P = cfg.page_size
    npg = cfg.num_pages
    relabel = np.random.default_rng(99).permutation(npg)       # old page p -> new page relabel[p]
    k_new = np.empty_like(inp["k_cache"])
    for p in range(npg):
        k_new[relabel[p] * P:(relabel[p] + 1) * P] = inp["k_cache"][p * P:(p + 1) * P]
    pt_new = np.where(inp["page_table"] >= 0, relabel[np.maximum(inp["page_table"], 0)], -1).astype(np.int32)
    s2 = _scores(cfg, inp, k_cache=k_new, page_table=pt_new)
    assert np.array_equal(s, s2)


# ---------------------------------------------------------------------------
# top-k

def _threshold_topk(s, k):
    """Second formulation: T = the k-th largest value; keep every s > T and then
    the lowest-index ties s == T until k are kept."""
    n = len(s)
    if k >= n:
        return list(range(n)) + [-1] * (k - n)
    T = sorted(s, reverse=True)[k - 1]
    keep = [t for t in range(n) if s[t] > T]
    for t in range(n):
        if len(keep) == k:
            break
        if s[t] == T:
            keep.append(t)
    return sorted(keep)


def test_topk_hand_ties(golden):
    g = golden["topk_ties"]
    s = np.array(_f(g["scores"]))
    assert np.signbit(s[3])
    for k, exp in g["cases"]:
        assert O.topk_select(s, len(s), k).tolist() == exp


_levels = st.sampled_from([-math.inf, -1.5, -0.0, 0.0, 0.25, 1.0, 3.0e-5, 7.0])


@settings(max_examples=300, deadline=None)
@given(vals=st.lists(_levels, min_size=1, max_size=200), k=st.integers(1, 260))
def test_topk_matches_threshold_formulation_tie_heavy(vals, k):
    s = np.array(vals)
    assert O.topk_select(s, len(s), k).tolist() == _threshold_topk(vals, k)


@settings(max_examples=200, deadline=None)
@given(vals=st.lists(st.floats(-1e6, 1e6, width=32), min_size=1, max_size=300), k=st.integers(1, 300))
def test_topk_matches_threshold_formulation_f32(vals, k):
    s = np.array(vals, dtype=np.float32)
    assert O.topk_select(s, len(s), k).tolist() == _threshold_topk([float(v) for v in s], k)


def test_topk_closed_forms():
    n, k = 1000, 64
    assert O.topk_select(np.full(n, 0.5), n, k).tolist() == list(range(k))
    assert O.topk_select(-np.arange(n, dtype=float), n, k).tolist() == list(range(k))
    assert O.topk_select(np.arange(n, dtype=float), n, k).tolist() == list(range(n - k, n))
    assert O.topk_select(np.arange(n, dtype=float), 10, k).tolist() == list(range(10)) + [-1] * (k - 10)
    # only the visible prefix counts
    s = np.arange(n, dtype=float)
    assert O.topk_select(s, 100, 5).tolist() == [95, 96, 97, 98, 99]


# ---------------------------------------------------------------------------
# page map

def test_page_map_identity_table():
    pt = np.arange(10, dtype=np.int32)[None, :]
    idx = np.array([[[0, 5, 63, 64, 65, 639, -1]]], dtype=np.int32)
    assert O.page_map(idx, pt, 64).tolist() == [[[0, 5, 63, 64, 65, 639, -1]]]


def test_page_map_bijection_onto_allocated_slots():
    cfg = dsa_inputs.scaled_config("c3", [300, 64, 1, 129, 1000], seed=21)
    pt = dsa_inputs.page_table_for(cfg, np.random.default_rng(21))
    P = cfg.page_size
    images = []
    for b, L in enumerate(cfg.seq_lens):
        idx = np.arange(L, dtype=np.int32)[None, None, :]
        ptb = pt[b:b + 1]
        sl = O.page_map(idx, ptb, P)[0, 0]
        assert len(set(sl.tolist())) == L                          # injective
        npg = (L + P - 1) // P
        expect = np.concatenate([np.arange(p * P, p * P + P) for p in pt[b, :npg]])[:L]
        assert np.array_equal(sl, expect)                          # first L slots of its pages, in order
        inv = {int(v): t for t, v in enumerate(sl)}
        assert [inv[int(v)] for v in sl] == list(range(L))         # the inverse recovers t
        images.append(set(sl.tolist()))
    allu = set().union(*images)
    assert sum(len(x) for x in images) == len(allu)                # disjoint across sequences
    in_use = set()
    for b, L in enumerate(cfg.seq_lens):
        for t in range(L):
            in_use.add(int(pt[b, t // P]) * P + t % P)
    assert allu == in_use
    assert max(allu) < cfg.num_slots


# ---------------------------------------------------------------------------
# sparse MLA

def _mla_case(seed, n_slots=300, H=4):
    rng = np.random.default_rng(seed)
    kv = (rng.standard_normal((n_slots, 576)) / 24).astype(np.float32)
    q = (rng.standard_normal((1, 1, H, 576)) / 24).astype(np.float32)
    return q, kv


def test_mla_hand_example(golden):
    g = golden["mla"]
    kv = np.zeros((2, 576), np.float64)
    kv[0, 512] = math.log(3.0)
    kv[0, 0] = 1.0
    kv[1, 1] = 2.0
    q = np.zeros((1, 1, 1, 576))
    q[0, 0, 0, 512] = 1.0
    out, lse = O.sparse_mla(q, "f64", kv, "f64", None, np.array([[[0, 1]]]), 1.0)
    assert abs(out[0, 0, 0, 0] - g["expected_out_0"]) < 1e-15
    assert abs(out[0, 0, 0, 1] - g["expected_out_1"]) < 1e-15
    assert np.all(out[0, 0, 0, 2:] == 0)
    assert abs(lse[0, 0, 0] - g["expected_lse"]) < 1e-15


def test_mla_single_token_and_zero_query():
    q, kv = _mla_case(1)
    out, lse = O.sparse_mla(q, "f32", kv, "f32", None, np.array([[[17, -1, -1]]]), 1 / 24)
    assert np.array_equal(out[0, 0], np.broadcast_to(kv[17, :512].astype(np.float64), (4, 512)))
    z = (q[0, 0].astype(np.float64) @ kv[17].astype(np.float64)) / 24
    assert np.allclose(lse[0, 0], z, rtol=0, atol=1e-15)
    sel = np.array([3, 9, 100, 250, 4])
    q0 = np.zeros_like(q)
    out, lse = O.sparse_mla(q0, "f32", kv, "f32", None, sel[None, None, :], 1 / 24)
    assert np.allclose(out[0, 0], kv[sel, :512].astype(np.float64).mean(axis=0)[None, :], rtol=0, atol=1e-16)
    assert np.allclose(lse[0, 0], math.log(5), rtol=0, atol=1e-15)


def test_mla_permutation_and_padding_invariance():
    q, kv = _mla_case(2)
    sel = np.random.default_rng(5).choice(300, 40, replace=False)
    o1, l1 = O.sparse_mla(q, "f32", kv, "f32", None, sel[None, None, :], 0.1)
    perm = np.random.default_rng(6).permutation(40)
    padded = np.concatenate([sel[perm][:20], [-1, -1], sel[perm][20:], [-1]])
    o2, l2 = O.sparse_mla(q, "f32", kv, "f32", None, padded[None, None, :], 0.1)
    assert np.allclose(o1, o2, rtol=0, atol=1e-15) and np.allclose(l1, l2, rtol=0, atol=1e-14)


def test_mla_brute_force_tiny():
    rng = np.random.default_rng(8)
    kv = rng.standard_normal((20, 576))
    q = rng.standard_normal((1, 1, 2, 576))
    sel = [4, 0, 13, 7]
    out, lse = O.sparse_mla(q, "f64", kv, "f64", None, np.array([[sel]]), 0.05)
    for h in range(2):
        z = [0.05 * sum(q[0, 0, h, d] * kv[t, d] for d in range(576)) for t in sel]
        den = sum(math.exp(v) for v in z)
        assert abs(lse[0, 0, h] - math.log(den)) < 1e-12
        for d in (0, 1, 255, 511):
            num = sum(math.exp(z[j]) * kv[t, d] for j, t in enumerate(sel))
            assert abs(out[0, 0, h, d] - num / den) < 1e-12


@pytest.mark.parametrize("n_split", [1, 2, 7, 40])
def test_split_combine_invariance(n_split):
    q, kv = _mla_case(3)
    sel = np.random.default_rng(9).choice(300, 40, replace=False)
    full, full_lse = O.sparse_mla(q, "f32", kv, "f32", None, sel[None, None, :], 1 / 24)
    qd = q[0, 0].astype(np.float64)
    ms, ls, os_ = [], [], []
    for chunk in np.array_split(sel, n_split):
        m, l, o = O.mla_partial(qd, kv[chunk].astype(np.float64), 1 / 24)
        ms.append(m), ls.append(l), os_.append(o)
    # an empty chunk carries no weight
    m, l, o = O.mla_partial(qd, kv[:0].astype(np.float64), 1 / 24)
    ms.append(m), ls.append(l), os_.append(o)
    out, lse = O.combine_splits(ms, ls, os_)
    assert np.allclose(out, full[0, 0], rtol=0, atol=1e-13)
    assert np.allclose(lse, full_lse[0, 0], rtol=0, atol=1e-13)


def test_combine_all_empty():
    out, lse = O.combine_splits([np.full(2, -np.inf)], [np.zeros(2)], [np.zeros((2, 512))])
    assert np.all(out == 0) and np.all(np.isneginf(lse))


@pytest.mark.parametrize("name,lens,Q", [("c1", [300], 1), ("c2", [200, 77], 2), ("c5", [130], 2)])
def test_topk_ge_context_gives_dense_attention(name, lens, Q):
    cfg = dsa_inputs.scaled_config(name, lens, seed=31, q_per_seq=Q, top_k=max(lens) + 5,
                                   mla_heads=8, idx_heads=4, idx_dim=32)
    inp = dsa_inputs.make_inputs(cfg)
    step = O.decode_step(inp, cfg)
    dense, dlse = O.dense_mla(inp["q_mla"], cfg.q_mla_dtype, inp["kv_cache"], cfg.kv_dtype,
                              inp["kv_scale"], inp["seq_lens"], inp["page_table"], Q,
                              cfg.page_size, cfg.sm_scale)
    assert np.allclose(step["out"], dense, rtol=0, atol=1e-12)
    assert np.allclose(step["lse"], dlse, rtol=0, atol=1e-12)
    # and every visible token was selected, in order
    pos = O.query_positions(cfg.seq_lens, Q)
    for b in range(cfg.batch):
        for i in range(Q):
            n = pos[b, i] + 1
            assert step["idx"][b, i, :n].tolist() == list(range(n))
            assert np.all(step["idx"][b, i, n:] == -1)


def test_decode_step_sparse_differs_from_dense_when_k_small():
    # with k < context the selection matters: sanity that the pin above is not vacuous
    cfg = dsa_inputs.scaled_config("c1", [600], seed=32, top_k=64)
    inp = dsa_inputs.make_inputs(cfg)
    step = O.decode_step(inp, cfg)
    dense, _ = O.dense_mla(inp["q_mla"], cfg.q_mla_dtype, inp["kv_cache"], cfg.kv_dtype,
                           inp["kv_scale"], inp["seq_lens"], inp["page_table"], 1,
                           cfg.page_size, cfg.sm_scale)
    assert np.abs(step["out"] - dense).max() > 1e-4
    assert (step["idx"] >= 0).sum() == 64


# ---------------------------------------------------------------------------
# cache append (the write of new tokens before the path reads them)

def _e4m3_probe_values():
    """Every finite e4m3fn magnitude, every midpoint between neighbours, one binary32
    step either side of each midpoint, values above 448, signed zeros and a
    log-uniform sweep, with both signs."""
    import torch
    mags = O.decode_e4m3fn(np.arange(0x7F, dtype=np.uint8))
    mids = (mags[:-1] + mags[1:]) / 2                      # exact in binary32
    m32 = mids.astype(np.float32)
    near = np.concatenate([np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(1e9))])
    big = np.array([448.0, 448.5, 455.0, 463.9], dtype=np.float32)
    r = np.random.default_rng(7)
    sweep = np.exp2(r.uniform(-14, 8.8, 4000)).astype(np.float32)
    v = np.concatenate([mags.astype(np.float32), m32, near, big, sweep, np.float32([0.0])])
    return np.concatenate([v, -v]).astype(np.float32), torch


def test_encode_e4m3fn_matches_torch():
    """The nearest-even encoder written from the format definition against torch's CPU
    float8_e4m3fn conversion, an independent routine, on every code, every tie and its
    binary32 neighbours (magnitudes below 464 so torch's conversion does not overflow)."""
    v, torch = _e4m3_probe_values()
    got = O.encode_e4m3fn(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)
    assert O.encode_e4m3fn(np.float32([-0.0]))[0] == 0x80
    assert O.encode_e4m3fn(np.float32([1e6, -1e6])).tolist() == [0x7E, 0xFE]    # saturates


def test_encode_e4m3fn_round_trip_and_ties():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(O.encode_e4m3fn(O.decode_e4m3fn(codes).astype(np.float32)), codes)
    # ties go to the even code: 1.0625 lies halfway between 1.0 (0x38) and 1.125 (0x39)
    assert O.encode_e4m3fn(np.float32([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10])).tolist() == \
        [0x38, 0x3A, 0x00, 0x02]


def test_quantize_row_fp8_bounds_and_special_rows():
    r = np.random.default_rng(11)
    for _ in range(50):
        x = (r.standard_normal(576) * np.exp2(r.uniform(-20, 20))).astype(np.float32).astype(np.float64)
        codes, sc = O.quantize_row_fp8(x)
        back = O.decode_e4m3fn(codes) * np.float64(sc)
        # half a unit in the last place: 2^-4 relative for normal codes, 2^-10 * scale below 2^-6
        assert np.all(np.abs(back - x) <= np.abs(x) * 2.0 ** -4 * (1 + 1e-6) + float(sc) * 2.0 ** -10)
        j = int(np.argmax(np.abs(x)))
        assert codes[j] == (0xFE if x[j] < 0 else 0x7E)           # the row maximum maps to 448
        # power-of-two rescaling moves only the scale
        c2, s2 = O.quantize_row_fp8(x * 2.0 ** 7)
        assert np.array_equal(c2, codes) and s2 == np.float32(sc * 2.0 ** 7)
    codes, sc = O.quantize_row_fp8(np.zeros(128))
    assert sc == 1.0 and not codes.any()
    codes, sc = O.quantize_row_fp8(np.full(8, -2.0 ** -110))
    assert sc == 1.0 and np.all(codes == 0x80)


def test_quantize_row_fp8_matches_the_input_generator():
    """The seeded generator quantizes binary32 rows with torch's conversion; on rows that
    are exact binary32 values both give the same codes and scales."""
    r = np.random.default_rng(12)
    x = (r.standard_normal((40, 576)) / 24).astype(np.float32).astype(np.float64)
    x[3] = 0.0
    gc, gs = dsa_inputs.encode_fp8_rows(x)
    for i in range(x.shape[0]):
        c, s = O.quantize_row_fp8(x[i])
        assert np.array_equal(c, gc[i]) and s == gs[i]


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "f32"])
def test_cache_append_places_rows_and_leaves_the_rest(dtype):
    r = np.random.default_rng(13)
    P, B, Q, D = 4, 3, 3, 24
    lens = np.array([3, 9, 14], dtype=np.int32)
    pages = r.permutation(12).astype(np.int32)
    pt = pages.reshape(B, 4)
    n_slots = 12 * P
    src_dtype = "f32" if dtype == "f32" else "bf16"
    x = r.standard_normal((B, Q, D)).astype(np.float32)
    new = x if src_dtype == "f32" else (x.view(np.uint32) >> 16).astype(np.uint16)
    old = (r.integers(0, 255, (n_slots, D), dtype=np.uint8) if dtype == "fp8" else
           r.standard_normal((n_slots, D)).astype(np.float32) if dtype == "f32" else
           r.integers(0, 2 ** 15, (n_slots, D), dtype=np.uint16))
    old_sc = r.random(n_slots).astype(np.float32) + 1 if dtype == "fp8" else None
    cache, sc = O.cache_append(old, dtype, old_sc, new, src_dtype, lens, pt, Q, P)
    written = set()
    for b in range(B):
        for i in range(Q):
            t = lens[b] - Q + i
            s = pt[b, t // P] * P + t % P                     # slot(b, t) written out by hand
            written.add(s)
            got = O.dequantize(cache[s:s + 1], dtype, None if sc is None else sc[s:s + 1])[0]
            want = O.dequantize(new[b, i], src_dtype)
            if dtype == "fp8":
                assert np.all(np.abs(got - want) <= np.abs(want) * 2.0 ** -4 * (1 + 1e-6) + sc[s] * 2.0 ** -10)
            else:
                assert np.array_equal(got, want)
    rest = np.array(sorted(set(range(n_slots)) - written))
    assert len(written) == B * Q
    assert np.array_equal(cache[rest], old[rest])
    if sc is not None:
        assert np.array_equal(sc[rest], old_sc[rest])


# ---------------------------------------------------------------------------
# latent up-projection (the projection after attention of the weight-absorbed MLA)

def _bits(x):
    return dsa_inputs.encode_bf16(np.asarray(x, dtype=np.float64))


def test_up_projection_hand_example(golden):
    g = golden["up_projection"]
    o = np.zeros((1, 2, 512))
    for r, h, d, v in g["o_nonzero"]:
        o[r, h, d] = v
    w_uv = np.zeros((2, 2, 512))
    for h, j, d, v in g["w_uv_nonzero"]:
        w_uv[h, j, d] = v
    y, v = O.latent_up_projection(o, _bits(w_uv), _bits(g["w_o"]))
    assert np.array_equal(v, np.array(g["expected_v"]))
    assert np.array_equal(y, np.array(g["expected_y"]))


def test_up_projection_brute_force_tiny():
    """Pure-Python loops over (r, h, j, d) and (m, h, j)."""
    rng = np.random.default_rng(41)
    R, H, Dv, Dm = 2, 3, 4, 5
    o = rng.standard_normal((R, H, 512))
    w_uv = _bits(rng.standard_normal((H, Dv, 512)) / 8)
    w_o = _bits(rng.standard_normal((Dm, H * Dv)) / 2)
    y, v = O.latent_up_projection(o, w_uv, w_o)
    W1, W2 = O.decode_bf16(w_uv), O.decode_bf16(w_o)
    for r in range(R):
        vv = [[sum(float(W1[h][j][d]) * float(o[r][h][d]) for d in range(512)) for j in range(Dv)] for h in range(H)]
        for h in range(H):
            for j in range(Dv):
                assert abs(v[r, h, j] - vv[h][j]) <= 1e-12 * (1 + abs(vv[h][j]))
        for m in range(Dm):
            ym = sum(float(W2[m][h * Dv + j]) * vv[h][j] for h in range(H) for j in range(Dv))
            assert abs(y[r, m] - ym) <= 1e-12 * (1 + abs(ym))


def test_up_projection_identity_and_permutation():
    """Identity weights return the latent output itself; permutation weights permute it (head
    blocks of o_proj are contiguous and in head order)."""
    rng = np.random.default_rng(42)
    R, H = 3, 2
    o = rng.standard_normal((R, H, 512))
    eye = np.eye(512)
    y, v = O.latent_up_projection(o, _bits(np.stack([eye] * H)), _bits(np.eye(H * 512)))
    assert np.array_equal(y, o.reshape(R, H * 512)) and np.array_equal(v, o)
    p0, p1 = rng.permutation(512), rng.permutation(512)
    w_uv = np.stack([eye[p0], eye[p1]])                 # row j picks latent p_h[j]
    pm = rng.permutation(H * 512)
    y, v = O.latent_up_projection(o, _bits(w_uv), _bits(np.eye(H * 512)[pm]))
    assert np.array_equal(v[:, 0], o[:, 0, p0]) and np.array_equal(v[:, 1], o[:, 1, p1])
    assert np.array_equal(y, v.reshape(R, -1)[:, pm])


def test_up_projection_after_attention_equals_attention_over_projected_values():
    """Weight absorption: projecting the latent attention output afterwards equals attending over
    each token's value reconstructed per head (W_UV c_t[:512]) and projecting those; the softmax
    weights are recomputed here with scipy from the logits, independently of the oracle."""
    from scipy.special import softmax
    rng = np.random.default_rng(43)
    cfg = dsa_inputs.scaled_config("c2", [300], seed=44, mla_heads=4, top_k=40)
    inp = dsa_inputs.make_inputs(cfg, with_indexer=False)
    slots = rng.choice(cfg.num_slots, (1, 1, 40), replace=False).astype(np.int32)
    o, _ = O.sparse_mla(inp["q_mla"], "bf16", inp["kv_cache"], "bf16", None, slots, cfg.sm_scale)
    Dv, Dm = 16, 24
    w_uv = _bits(rng.standard_normal((4, Dv, 512)) / 16)
    w_o = _bits(rng.standard_normal((Dm, 4 * Dv)) / 8)
    y_abs, _ = O.latent_up_projection(o[0], w_uv, w_o)
    q = O.decode_bf16(inp["q_mla"])[0, 0]                     # [H, 576]
    c = O.decode_bf16(inp["kv_cache"])[slots[0, 0]]          # [40, 576]
    W1, W2 = O.decode_bf16(w_uv), O.decode_bf16(w_o)
    v = np.zeros((4, Dv))
    for h in range(4):
        p = softmax(cfg.sm_scale * (c @ q[h]))
        vals = c[:, :512] @ W1[h].T                          # [40, Dv]: each token's value of head h
        v[h] = p @ vals
    y_direct = W2 @ v.reshape(-1)
    assert np.allclose(y_abs[0], y_direct, rtol=1e-11, atol=1e-14)


def test_up_projection_is_linear_in_o():
    rng = np.random.default_rng(45)
    w_uv = _bits(rng.standard_normal((2, 8, 512)) / 16)
    w_o = _bits(rng.standard_normal((6, 16)))
    o1, o2 = rng.standard_normal((2, 3, 2, 512))
    y1, _ = O.latent_up_projection(o1, w_uv, w_o)
    y2, _ = O.latent_up_projection(o2, w_uv, w_o)
    y3, _ = O.latent_up_projection(2.5 * o1 - o2, w_uv, w_o)
    assert np.allclose(y3, 2.5 * y1 - y2, rtol=1e-12, atol=1e-12)
    assert not np.allclose(y1, 0)
    yz, _ = O.latent_up_projection(np.zeros((1, 2, 512)), w_uv, w_o)
    assert np.array_equal(yz, np.zeros((1, 6)))


def test_shared_index_query_selections_nest():
    """Verify rows that share one indexer query see nested prefixes of the same scores (row i
    one token more than row i - 1, position L - Q + i), so the top-k of row i is that of row
    i - 1 with at most one token exchanged for the newly visible one; and the inputs repeat the
    first row's query and head weights."""
    cfg = dsa_inputs.scaled_config("c5", [700, 420, 90], seed=33, q_per_seq=4, top_k=64, idx_heads=8,
                                   shared_index_query=True)
    inp = dsa_inputs.make_inputs(cfg, with_mla=False)
    assert np.array_equal(inp["q_idx"], np.repeat(inp["q_idx"][:, :1], 4, axis=1))
    assert np.array_equal(inp["w"], np.repeat(inp["w"][:, :1], 4, axis=1))
    s = O.indexer_scores(inp["q_idx"], cfg.q_idx_dtype, inp["w"], inp["k_cache"], cfg.key_dtype,
                         inp["k_scale"], inp["seq_lens"], inp["page_table"], cfg.q_per_seq, cfg.page_size)
    idx = O.topk(s, inp["seq_lens"], cfg.q_per_seq, cfg.top_k)
    changed = 0
    for b, L in enumerate(cfg.seq_lens):
        for i in range(1, 4):
            a, c = set(idx[b, i - 1][idx[b, i - 1] >= 0]), set(idx[b, i][idx[b, i] >= 0])
            new = L - 4 + i
            assert c - a <= {new} and len(a - c) <= 1 and len(a) <= len(c)
            changed += len(c - a)
    assert changed > 0      # the new token enters some selection (not a vacuous comparison)
