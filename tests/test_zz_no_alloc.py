"""The no-allocation step (dsa_decode_step_noalloc) against the workspace step (dsa_decode_step)
on the same inputs: two calls in a row through the C ABI, the second on a smaller input, each
compared with the workspace path's output to the attention bar (and bit for bit: both run the
same deterministic kernels)."""
import ctypes

import numpy as np
import pytest
import torch

import dsa_inputs
import sparse_attention_10_amd as dsa
from tests.gpu_helpers import DEV, batch_of, check_attention

pytestmark = pytest.mark.gpu


def _step_pair(name, lens, seed, **kw):
    cfg = dsa_inputs.scaled_config(name, lens, seed=seed, **kw)
    inp = dsa_inputs.make_inputs(cfg)
    t = dsa_inputs.to_torch(inp, cfg, DEV)
    B, Q, H, k = cfg.batch, cfg.q_per_seq, cfg.mla_heads, cfg.top_k
    outs = []
    for noalloc in (False, True):
        out = torch.full((B, Q, H, 512), float("nan"), dtype=torch.float32, device=DEV)
        lse = torch.full((B, Q, H), float("nan"), dtype=torch.float32, device=DEV)
        args = dsa.decode_step_args(batch_of(cfg, t), t["q_idx"], t["w"], t["k_cache"], t["k_scale"], k,
                                    t["q_mla"], t["kv_cache"], t["kv_scale"], cfg.sm_scale, out, lse)
        if noalloc:
            assert dsa.decode_step_workspace_bytes(args) <= dsa.decode_step_noalloc_max_bytes()
            st = dsa.lib().dsa_decode_step_noalloc(ctypes.byref(args), None)
            assert st == dsa.DSA_OK, dsa.lib().dsa_last_error().decode()
        else:
            ws = torch.zeros(max(1, dsa.decode_step_workspace_bytes(args)), dtype=torch.uint8, device=DEV)
            dsa.dsa_decode_step(args, ws)
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy(), lse.cpu().numpy()))
    (o_ws, l_ws), (o_na, l_na) = outs
    check_attention(o_na, o_ws.astype(np.float64), l_na, l_ws.astype(np.float64))
    assert np.array_equal(o_na, o_ws) and np.array_equal(l_na, l_ws)


def test_noalloc_step_matches_workspace_step_twice():
    # first call: fp8 caches, two verify rows per sequence, long rows ranked in two passes and
    # split-k partials in the scratch buffer; second call: a smaller bf16 single-row step
    _step_pair("c5", [70000, 3000, 700], seed=31)
    _step_pair("c2", [1500], seed=32)


def test_noalloc_rejects_a_step_beyond_the_scratch_size():
    cfg = dsa_inputs.scaled_config("c4", [65536 + 4096], seed=33, q_per_seq=4096, top_k=2048)
    t = {n: torch.zeros(1, dtype=torch.uint8, device=DEV) for n in ("x",)}
    sl = torch.tensor(cfg.seq_lens, dtype=torch.int32, device=DEV)
    pt = torch.zeros((1, cfg.max_pages), dtype=torch.int32, device=DEV)
    batch = dsa.make_batch(sl, pt, cfg.q_per_seq, cfg.page_size, cfg.max_seq_len, cfg.num_slots)
    q_idx = torch.zeros((1, cfg.q_per_seq, 64, 128), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((1, cfg.q_per_seq, 64), dtype=torch.float32, device=DEV)
    keys = torch.zeros((64, 128), dtype=torch.bfloat16, device=DEV)
    q_mla = torch.zeros((1, cfg.q_per_seq, 64, 576), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((64, 576), dtype=torch.bfloat16, device=DEV)
    out = torch.zeros((1, cfg.q_per_seq, 64, 512), dtype=torch.float32, device=DEV)
    # (the whole chunk's scores in one block: 1.14 GB)
    args = dsa.decode_step_args(batch, q_idx, w, keys, None, 2048, q_mla, kv, None, cfg.sm_scale, out,
                                prefill_rows_per_block=4096)
    assert dsa.decode_step_workspace_bytes(args) > dsa.decode_step_noalloc_max_bytes()
    st = dsa.lib().dsa_decode_step_noalloc(ctypes.byref(args), None)
    assert st == dsa.DSA_ERR_WORKSPACE_TOO_SMALL
    assert b"scratch" in dsa.lib().dsa_last_error()
    del t
