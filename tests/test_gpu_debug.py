"""The opt-in DSA_DEBUG build (libdsa_debug.so) on the GPU, through the C ABI.

* On valid inputs it computes exactly what libdsa.so computes (the checks touch no arithmetic)
  and reports no violation.
* Each data precondition that libdsa.so leaves unchecked is broken once, on the debug build
  only: its kernels flag the violation in the error word and clamp the value into range, so the
  call completes; dsa_debug_check returns the flag and clears it.  (These inputs never reach
  libdsa.so, whose kernels assume the preconditions.)
"""
import numpy as np
import pytest
import torch

import dsa_inputs
import sparse_attention_10_amd as dsa
from tests.gpu_helpers import DEV, batch_of, run_step

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dbg_lib():
    L = dsa.load_library(dsa.DEBUG_LIB_PATH)
    assert L.dsa_debug_enabled() == 1
    with dsa.using_library(L):
        assert dsa.debug_check() == 0          # (clears anything an earlier process state left)
    return L


def _case(name, lens, seed, **kw):
    cfg = dsa_inputs.scaled_config(name, lens, seed=seed, **kw)
    inp = dsa_inputs.make_inputs(cfg)
    return cfg, inp, dsa_inputs.to_torch(inp, cfg, DEV)


@pytest.mark.parametrize("name,lens", [("c2", [5000]), ("c5", [3000, 1200])])
def test_debug_build_matches_release_on_valid_inputs(dbg_lib, name, lens):
    cfg, _, t = _case(name, lens, seed=401)
    ref = run_step(cfg, t)
    with dsa.using_library(dbg_lib):
        got = run_step(cfg, t)
        assert dsa.debug_check() == 0
    for key in ("out", "lse", "scores", "idx", "slots"):
        assert torch.equal(got[key], ref[key]) or (key == "scores" and np.array_equal(
            got[key].cpu().numpy(), ref[key].cpu().numpy(), equal_nan=True)), key


@pytest.mark.parametrize("i", range(24))
def test_debug_build_matches_release_on_random_steps(dbg_lib, i):
    """The first 24 configurations of the seeded step sweep (tests/test_gpu_random.py): every
    dtype family, ragged lengths below k, page sizes 1-128, verify and chunk rows."""
    from tests.test_gpu_random import draw_case
    name, lens, kw = draw_case(i)
    cfg, _, t = _case(name, lens, seed=3000 + i, **kw)
    ref = run_step(cfg, t)
    with dsa.using_library(dbg_lib):
        got = run_step(cfg, t)
        assert dsa.debug_check() == 0
    for key in ("out", "lse", "idx", "slots"):
        assert torch.equal(got[key], ref[key]), key
    assert np.array_equal(got["scores"].cpu().numpy(), ref["scores"].cpu().numpy(), equal_nan=True)


@pytest.mark.parametrize("i", range(8))
def test_debug_build_matches_release_on_grouped_steps(dbg_lib, i):
    """The first 8 grouped verify batches of the seeded sweep (8 or 16 sequences x 2-4 rows):
    the debug build's checks find nothing and change nothing."""
    from tests.test_gpu_random import draw_grouped_case
    name, lens, kw = draw_grouped_case(i)
    cfg, _, t = _case(name, lens, seed=4000 + i, **kw)
    ref = run_step(cfg, t)
    with dsa.using_library(dbg_lib):
        got = run_step(cfg, t)
        assert dsa.debug_check() == 0
    for key in ("out", "lse", "idx", "slots"):
        assert torch.equal(got[key], ref[key]), key
    assert np.array_equal(got["scores"].cpu().numpy(), ref["scores"].cpu().numpy(), equal_nan=True)


def test_debug_flags_page_id_out_of_range(dbg_lib):
    cfg, _, t = _case("c2", [5000], seed=402)
    pages = cfg.num_slots // cfg.page_size
    t["page_table"][0, 3] = pages + 7             # past the pool
    t["page_table"][0, 9] = -2
    with dsa.using_library(dbg_lib):
        r = run_step(cfg, t)
        flags = dsa.debug_check()
    assert flags & dsa.DSA_DEBUG_PAGE_ID
    slots = r["slots"].cpu().numpy()
    assert slots.min() >= -1 and slots.max() < cfg.num_slots   # clamped entries map into the pool


def test_debug_flags_seq_len_past_max(dbg_lib):
    cfg, _, t = _case("c2", [3000], seed=403)
    t["seq_lens"][0] = cfg.max_seq_len + 100
    with dsa.using_library(dbg_lib):
        r = run_step(cfg, t)
        flags = dsa.debug_check()
    assert flags & dsa.DSA_DEBUG_SEQ_LEN
    assert torch.isfinite(r["out"]).all()


@pytest.mark.parametrize("name", ["c2", "c5"])
def test_debug_flags_mla_slot_out_of_range(dbg_lib, name):
    cfg, _, t = _case(name, [3000], seed=404, top_k=512, q_per_seq=1)
    rng = np.random.default_rng(404)
    slots = rng.choice(cfg.num_slots, (1, 1, 512), replace=False).astype(np.int32)
    bad = slots.copy()
    bad[0, 0, 5] = cfg.num_slots + 3
    bad[0, 0, 300] = -7
    good = slots.copy()
    good[0, 0, 5] = -1
    good[0, 0, 300] = -1

    def mla(sl):
        out = torch.empty((1, 1, cfg.mla_heads, 512), dtype=torch.float32, device=DEV)
        lse = torch.empty((1, 1, cfg.mla_heads), dtype=torch.float32, device=DEV)
        dsa.dsa_sparse_mla_decode(t["q_mla"], t["kv_cache"], t["kv_scale"], torch.from_numpy(sl).to(DEV),
                                  cfg.sm_scale, out, lse)
        torch.cuda.synchronize()
        return out, lse

    ref_out, ref_lse = mla(good)                  # release build, valid slots
    with dsa.using_library(dbg_lib):
        out, lse = mla(bad)
        flags = dsa.debug_check()
    assert flags & dsa.DSA_DEBUG_SLOT
    # an out-of-range slot is skipped exactly like -1
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)


def test_debug_flags_nan_score(dbg_lib):
    cfg, _, t = _case("c2", [3000], seed=405, top_k=256)
    scores = torch.randn((1, 1, cfg.max_seq_len), device=DEV)
    scores[0, 0, 1234] = float("nan")
    idx = torch.empty((1, 1, 256), dtype=torch.int32, device=DEV)
    with dsa.using_library(dbg_lib):
        dsa.dsa_topk(batch_of(cfg, t), scores, 256, idx)
        flags = dsa.debug_check()
    assert flags & dsa.DSA_DEBUG_NAN_SCORE


def test_debug_flags_page_map_index(dbg_lib):
    cfg, inp, t = _case("c2", [3000], seed=406, top_k=16)
    idx = torch.arange(16, dtype=torch.int32, device=DEV).view(1, 1, 16).contiguous()
    idx[0, 0, 2] = 3000 + 5                        # past the sequence
    idx[0, 0, 7] = -3
    slots = torch.empty_like(idx)
    with dsa.using_library(dbg_lib):
        dsa.dsa_page_map(batch_of(cfg, t), idx, slots)
        flags = dsa.debug_check()
    assert flags & dsa.DSA_DEBUG_TOPK_INDEX
    s = slots.cpu().numpy()[0, 0]
    assert s[2] == -1 and s[7] == -1
    pt = inp["page_table"][0]
    for j in (0, 1, 3, 15):
        assert s[j] == pt[j // cfg.page_size] * cfg.page_size + j % cfg.page_size


def test_debug_flags_append_page_id(dbg_lib):
    cfg, _, t = _case("c2", [3000], seed=407)
    pages = cfg.num_slots // cfg.page_size
    t["page_table"][0, (3000 - 1) // cfg.page_size] = pages + 1   # the new token's page
    kv_new = torch.randn((1, 1, 576), device=DEV).to(torch.bfloat16)
    before = t["kv_cache"].clone()
    with dsa.using_library(dbg_lib):
        dsa.dsa_kv_cache_append(batch_of(cfg, t), kv_new, t["kv_cache"], t["kv_scale"])
        flags = dsa.debug_check()
    assert flags & dsa.DSA_DEBUG_PAGE_ID
    assert torch.equal(t["kv_cache"], before)       # nothing written for that token
