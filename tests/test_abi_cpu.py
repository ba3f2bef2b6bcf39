"""The C ABI without a GPU: the library loads, exports every entry point include/dsa.h
declares, and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

import sparse_attention_10_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(dsa.LIB_PATH):
        from sparse_attention_10_amd import build
        build.build()
    return dsa.lib()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(dsa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_path(L):
    names = _declared()
    for n in ("dsa_indexer_scores", "dsa_topk", "dsa_page_map", "dsa_sparse_mla_decode", "dsa_decode_step",
              "dsa_mla_combine"):
        assert n in names
    assert set(names) == set(dsa.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    for n in _declared():
        assert hasattr(L, n), n
    assert L.dsa_abi_version() == 1
    assert L.dsa_status_string(0) == b"DSA_OK"
    assert L.dsa_status_string(3) == b"DSA_ERR_WORKSPACE_TOO_SMALL"


def test_debug_build_exports_every_symbol_and_release_reports_unsupported(L):
    if not os.path.exists(dsa.DEBUG_LIB_PATH):
        from sparse_attention_10_amd import build
        build.build(debug=True)
    D = dsa.load_library(dsa.DEBUG_LIB_PATH)
    for n in _declared():
        assert hasattr(D, n), n
    assert D.dsa_debug_enabled() == 1 and L.dsa_debug_enabled() == 0
    # the release build has no error word: dsa_debug_check says so without touching a device
    flags = ctypes.c_uint32(7)
    assert L.dsa_debug_check(ctypes.byref(flags), None) == dsa.DSA_ERR_UNSUPPORTED
    assert flags.value == 0
    assert b"DSA_DEBUG" in L.dsa_last_error()


def _batch(**kw):
    b = dict(batch=1, q_per_seq=1, max_seq_len=4096, page_size=64, max_pages_per_seq=64, num_slots=4096,
             seq_lens=256, page_table=512)
    b.update(kw)
    return dsa.DsaBatch(b["batch"], b["q_per_seq"], b["max_seq_len"], b["page_size"], b["max_pages_per_seq"],
                        b["num_slots"], b["seq_lens"], b["page_table"])


FAKE = 1 << 20   # an aligned non-NULL address; validation failures never dereference it


def _indexer(L, batch, **kw):
    a = dict(q=FAKE, qd=dsa.DSA_BF16, w=FAKE, k=FAKE, kd=dsa.DSA_BF16, ks=None, Hi=64, Di=128, s=FAKE, ld=4096)
    a.update(kw)
    return L.dsa_indexer_scores(ctypes.byref(batch), a["q"], a["qd"], a["w"], a["k"], a["kd"], a["ks"], a["Hi"],
                                a["Di"], a["s"], a["ld"], None)


@pytest.mark.parametrize("kw,bkw,status", [
    (dict(q=None), {}, 1),
    (dict(), dict(batch=0), 1),
    (dict(), dict(q_per_seq=5000), 1),
    (dict(), dict(page_size=0), 1),
    (dict(), dict(max_pages_per_seq=10), 1),
    (dict(), dict(seq_lens=None), 1),
    (dict(kd=dsa.DSA_FP8_E4M3FN), {}, 1),            # fp8 keys without scales
    (dict(qd=dsa.DSA_FP8_E4M3FN), {}, 1),            # fp8 q is not accepted
    (dict(kd=7), {}, 1),
    (dict(ld=100), {}, 1),
    (dict(Hi=0), {}, 1),
    (dict(Hi=200), {}, 2),
    (dict(q=FAKE + 2), {}, 1),                        # matrix-core path needs 16-byte alignment
])
def test_indexer_rejects(L, kw, bkw, status):
    assert _indexer(L, _batch(**bkw), **kw) == status
    assert len(L.dsa_last_error()) > 0


def test_topk_rejects(L):
    b = _batch()
    assert L.dsa_topk(ctypes.byref(b), FAKE, 4096, 0, FAKE, None, None, 0, None) == 1
    assert L.dsa_topk(ctypes.byref(b), FAKE, 4096, 9000, FAKE, None, None, 0, None) == 2
    assert L.dsa_topk(ctypes.byref(b), None, 4096, 16, FAKE, None, None, 0, None) == 1
    assert L.dsa_topk(ctypes.byref(b), FAKE, 10, 16, FAKE, None, None, 0, None) == 1
    big = _batch(max_seq_len=300000, max_pages_per_seq=5000)
    assert L.dsa_topk(ctypes.byref(big), FAKE, 300000, 16, FAKE, None, None, 0, None) == 2
    assert L.dsa_topk_workspace_size(ctypes.byref(b), 2048) == 0


def test_topk_workspace_long_rows(L):
    # a few rows of 64K+ columns are ranked in two passes whose candidates need a workspace:
    # 32 rows x 8 chunks of 16K keep 8 x 2048 (score, column) pairs each
    long = _batch(batch=32, q_per_seq=1, max_seq_len=131072, max_pages_per_seq=2048, num_slots=32 * 131072)
    need = L.dsa_topk_workspace_size(ctypes.byref(long), 2048)
    assert need >= 32 * 8 * 2048 * 8
    assert L.dsa_topk(ctypes.byref(long), FAKE, 131072, 2048, FAKE, None, None, 0, None) == 3
    assert L.dsa_topk(ctypes.byref(long), FAKE, 131072, 2048, FAKE, None, FAKE, need - 1, None) == 3
    # 128 rows of 64K columns: chunks of 32K, two per row
    verify = _batch(batch=64, q_per_seq=2, max_seq_len=65536, max_pages_per_seq=1024, num_slots=64 * 65536)
    assert L.dsa_topk_workspace_size(ctypes.byref(verify), 2048) >= 128 * 2 * 2048 * 8
    # below 64K columns, or more rows than half the compute units: one pass
    assert L.dsa_topk_workspace_size(ctypes.byref(_batch(max_seq_len=65535, max_pages_per_seq=1024)), 2048) == 0
    many = _batch(batch=65, q_per_seq=2, max_seq_len=65536, max_pages_per_seq=1024, num_slots=65 * 65536)
    assert L.dsa_topk_workspace_size(ctypes.byref(many), 2048) == 0


def _mla(L, **kw):
    a = dict(B=1, Q=1, q=FAKE, qd=dsa.DSA_BF16, kv=FAKE, kvd=dsa.DSA_BF16, ks=None, ns_=4096, sl=FAKE, k=2048,
             H=64, scale=0.04, out=FAKE, lse=None, split=0, ws=None, wsb=0)
    a.update(kw)
    return L.dsa_sparse_mla_decode(a["B"], a["Q"], a["q"], a["qd"], a["kv"], a["kvd"], a["ks"], a["ns_"], a["sl"],
                                   a["k"], a["H"], a["scale"], a["out"], a["lse"], a["split"], a["ws"], a["wsb"],
                                   None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(H=8), 2), (dict(H=100), 2), (dict(kvd=dsa.DSA_F32), 2),
    (dict(kvd=dsa.DSA_FP8_E4M3FN), 1), (dict(k=0), 1), (dict(k=10000), 2), (dict(scale=float("nan")), 1),
    (dict(split=-1), 1), (dict(out=FAKE + 4), 1), (dict(split=4), 3),
])
def test_mla_rejects(L, kw, status):
    assert _mla(L, **kw) == status


def test_mla_workspace_sizes(L):
    # one chunk needs no workspace; k chunks need partial o, m and l per head
    assert L.dsa_sparse_mla_workspace_size(1, 1, 64, 2048, 1, dsa.DSA_BF16, dsa.DSA_BF16) == 0
    ns = L.dsa_sparse_mla_default_split(1, 1, 64, 2048, dsa.DSA_BF16)
    assert ns == 16          # few bf16 rows: one 128-row tile per chunk (16-head workgroups)
    assert L.dsa_sparse_mla_default_split(4, 1, 64, 2048, dsa.DSA_BF16) == 16
    need = L.dsa_sparse_mla_workspace_size(1, 1, 64, 2048, 4, dsa.DSA_BF16, dsa.DSA_BF16)
    assert need >= 4 * 64 * 512 * 4 + 2 * 4 * 64 * 4
    assert L.dsa_sparse_mla_workspace_size(1, 1, 16, 2048, 4, dsa.DSA_F32, dsa.DSA_BF16) == 0   # vector path: no split
    # many rows fill the GPU with one chunk each; fp8 rows keep chunks of at most 2048 rows
    assert L.dsa_sparse_mla_default_split(4096, 1, 64, 2048, dsa.DSA_BF16) == 1
    assert L.dsa_sparse_mla_default_split(4096, 1, 64, 2048, dsa.DSA_FP8_E4M3FN) == 1
    assert L.dsa_sparse_mla_default_split(4096, 1, 64, 4096, dsa.DSA_FP8_E4M3FN) == 2
    assert L.dsa_sparse_mla_default_split(64, 2, 64, 2048, dsa.DSA_FP8_E4M3FN) == 2


def test_decode_step_workspace_and_rejects(L):
    a = dsa.DsaDecodeStepArgs()
    a.batch = _batch()
    a.q_idx, a.q_idx_dtype, a.w, a.k_cache, a.k_dtype = FAKE, dsa.DSA_BF16, FAKE, FAKE, dsa.DSA_BF16
    a.idx_heads, a.idx_dim, a.top_k = 64, 128, 2048
    a.q_mla, a.q_mla_dtype, a.kv_cache, a.kv_dtype = FAKE, dsa.DSA_BF16, FAKE, dsa.DSA_BF16
    a.mla_heads, a.sm_scale, a.out = 64, 1 / 24, FAKE
    need = L.dsa_decode_step_workspace_size(ctypes.byref(a))
    assert need >= 4096 * 4 + 2 * 2048 * 4
    assert L.dsa_decode_step(ctypes.byref(a), FAKE, need - 1, None) == 3
    a.top_k = 0
    assert L.dsa_decode_step(ctypes.byref(a), FAKE, need, None) == 1
    assert L.dsa_decode_step(None, FAKE, need, None) == 1


def test_valid_call_without_gpu_reports_instead_of_crashing(L):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st = _indexer(L, _batch())
    assert st in (dsa.DSA_ERR_HIP, dsa.DSA_ERR_UNSUPPORTED)


def _append(L, batch, **kw):
    a = dict(kv=FAKE, kvd=dsa.DSA_BF16, kc=FAKE, kcd=dsa.DSA_BF16, ks=None,
             k=FAKE, kd=dsa.DSA_BF16, Di=128, kk=FAKE, kkd=dsa.DSA_FP8_E4M3FN, kks=FAKE)
    a.update(kw)
    return L.dsa_kv_cache_append(ctypes.byref(batch), a["kv"], a["kvd"], a["kc"], a["kcd"], a["ks"],
                                 a["k"], a["kd"], a["Di"], a["kk"], a["kkd"], a["kks"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(kv=None, k=None), 1),                       # nothing to append
    (dict(kc=None), 1),                               # rows without a cache
    (dict(kvd=dsa.DSA_F32), 2),                       # f32 rows into a bf16 cache
    (dict(kvd=dsa.DSA_FP8_E4M3FN, kcd=dsa.DSA_FP8_E4M3FN, ks=FAKE), 2),   # fp8 rows
    (dict(kks=None), 1),                              # fp8 key cache without scales
    (dict(Di=100), 2),
    (dict(Di=2048), 2),
    (dict(k=FAKE + 8), 1),                            # misaligned rows
    (dict(kvd=9), 1),
])
def test_cache_append_rejects(L, kw, status):
    assert _append(L, _batch(), **kw) == status
    assert len(L.dsa_last_error()) > 0


def test_noalloc_step_rejects_oversized_steps_before_the_device(L):
    """A 4096-row prefill chunk over 69632 tokens needs over 1 GiB of scores: beyond the fixed
    scratch of the no-allocation step, which refuses it before any device call."""
    a = dsa.DsaDecodeStepArgs()
    a.batch = _batch(q_per_seq=4096, max_seq_len=69632, max_pages_per_seq=1088, num_slots=69632)
    a.q_idx, a.q_idx_dtype, a.w = FAKE, dsa.DSA_BF16, FAKE
    a.k_cache, a.k_dtype, a.k_scale = FAKE, dsa.DSA_BF16, None
    a.idx_heads, a.idx_dim, a.top_k = 64, 128, 2048
    a.q_mla, a.q_mla_dtype, a.kv_cache, a.kv_dtype, a.kv_scale = FAKE, dsa.DSA_BF16, FAKE, dsa.DSA_BF16, None
    a.mla_heads, a.sm_scale, a.n_split, a.out, a.lse = 64, 1.0 / 24, 0, FAKE, None
    assert L.dsa_decode_step_workspace_size(ctypes.byref(a)) > L.dsa_decode_step_noalloc_max_bytes()
    assert L.dsa_decode_step_noalloc_max_bytes() == 128 << 20
    assert L.dsa_decode_step_noalloc(ctypes.byref(a), None) == dsa.DSA_ERR_WORKSPACE_TOO_SMALL
    assert b"scratch" in L.dsa_last_error()
    assert L.dsa_decode_step_noalloc(None, None) == dsa.DSA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("R,H,Dv,Dm,ptrs,ws,status", [
    (0, 64, 128, 256, True, 1 << 30, 1),
    (4, 64, 100, 256, True, 1 << 30, 2),       # value dim not a multiple of 32
    (4, 64, 128, 250, True, 1 << 30, 2),       # model width not a multiple of 16
    (4, 200, 128, 256, True, 1 << 30, 2),
    (4, 64, 128, 256, False, 1 << 30, 1),      # NULL arrays
    (4, 64, 128, 256, True, 16, 3),            # workspace too small
])
def test_up_projection_rejects(L, R, H, Dv, Dm, ptrs, ws, status):
    p = FAKE if ptrs else None
    assert L.dsa_latent_up_projection(R, H, Dv, Dm, p, p, p, p, FAKE, ws, None) == status
    assert len(L.dsa_last_error()) > 0


def test_up_projection_workspace_size(L):
    # v [R, H, Dv] f32, plus K-split partials [ksplit, R, Dm] f32 when the rows leave the GPU idle
    # (one or two rows take the vector path, whose columns are whole sums: no partials)
    assert L.dsa_latent_up_projection_workspace_size(128, 64, 128, 6144) >= 128 * 64 * 128 * 4
    assert L.dsa_latent_up_projection_workspace_size(4, 64, 128, 6144) > 4 * 64 * 128 * 4
    assert L.dsa_latent_up_projection_workspace_size(1, 64, 128, 6144) == 64 * 128 * 4
    assert L.dsa_latent_up_projection_workspace_size(2, 16, 128, 6144) == 2 * 16 * 128 * 4
    assert L.dsa_latent_up_projection_workspace_size(0, 64, 128, 6144) == 0
