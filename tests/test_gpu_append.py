"""GPU parity of the cache append (dsa_kv_cache_append) against the fp64 oracle, through the C ABI.

Both sides start from the same random cache contents; after the append every byte of both
caches and every scale must equal the oracle's (bit-exact: copies, codes and scales are integer
or exactly-rounded results).  Rows include the special cases of the fp8 encoding: all-zero and
negative-zero rows, rows below the scale floor, exact ties between two codes, and magnitudes
from 2^-30 to 2^100.
"""
import zlib

import numpy as np
import pytest
import torch

import sparse_attention_10_amd as dsa
from oracle import dsa_oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """binary32 values -> bf16 bit patterns (upper half: any bf16 value serves as an input)."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _dev(a: np.ndarray, kind: str):
    if kind == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    elif kind == "fp8":
        t = torch.from_numpy(np.ascontiguousarray(a)).view(torch.float8_e4m3fn)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(DEV)


def _host(t) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def _rows(r, n, D, special: bool) -> np.ndarray:
    x = (r.standard_normal((n, D)) * np.exp2(r.uniform(-30, 30, (n, 1)))).astype(np.float32)
    if special and n >= 5:
        x[0] = 0.0
        x[0, ::3] = -0.0
        x[1] = np.float32(2.0 ** -110) * np.sign(r.standard_normal(D)).astype(np.float32)
        x[2] = r.choice(np.float32([1.0625, 1.1875, -3 * 2.0 ** -10, 2.0 ** -10, 0.5]), D)
        x[2, 0] = 448.0                                   # scale exactly 1: every tie is exact
        x[3] *= np.float32(2.0 ** 70)
        x[4, 1:] = np.float32(1e-6) * x[4, 1:]            # one large value, the rest tiny
    return x


def _old_cache(r, n_slots, D, kind):
    if kind == "fp8":
        c = r.integers(0, 256, (n_slots, D), dtype=np.uint8)
        c[(c & 0x7F) == 0x7F] = 0                         # no NaN codes in the initial contents
        return c, (r.random(n_slots) + 0.5).astype(np.float32)
    if kind == "bf16":
        return _bf16_bits(r.standard_normal((n_slots, D)).astype(np.float32)), None
    return r.standard_normal((n_slots, D)).astype(np.float32), None


CASES = [
    # (name, seq_lens, Q, page size, rows dtype, latent cache dtype, key cache dtype, key dim)
    ("bf16 decode", [130, 64, 2000], 1, 64, "bf16", "bf16", "bf16", 128),
    ("fp8 verify rows", [66, 4097, 2, 700], 2, 64, "bf16", "fp8", "fp8", 128),
    ("f32 tiny decode", [4096], 1, 64, "f32", "f32", "f32", 64),
    ("f32 rows into fp8", [300, 129], 3, 64, "f32", "fp8", "fp8", 64),
    ("prefill chunk", [1000], 300, 64, "bf16", "fp8", "bf16", 128),
    ("odd page size, wide key", [500, 97], 5, 48, "bf16", "bf16", "fp8", 1024),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_cache_append_matches_oracle(case):
    name, lens, Q, P, src, kv_kind, k_kind, Di = case
    r = np.random.default_rng(zlib.crc32(name.encode()))
    B = len(lens)
    lens = np.array(lens, dtype=np.int32)
    pages_per = [(L + P - 1) // P for L in lens]
    n_pages = sum(pages_per) + 3                          # a few pages nobody owns
    perm = r.permutation(n_pages).astype(np.int32)
    maxP = max(pages_per)
    pt = np.zeros((B, maxP), dtype=np.int32)
    o = 0
    for b, n in enumerate(pages_per):
        pt[b, :n] = perm[o:o + n]
        o += n
    n_slots = n_pages * P
    kv_x = _rows(r, B * Q, O.ROW_DIM, special=True).reshape(B, Q, O.ROW_DIM)
    k_x = _rows(r, B * Q, Di, special=True).reshape(B, Q, Di)
    kv_new = kv_x if src == "f32" else _bf16_bits(kv_x)
    k_new = k_x if src == "f32" else _bf16_bits(k_x)
    kv_old, kv_sc_old = _old_cache(r, n_slots, O.ROW_DIM, kv_kind)
    k_old, k_sc_old = _old_cache(r, n_slots, Di, k_kind)

    kv_ref, kv_sc_ref = O.cache_append(kv_old, kv_kind, kv_sc_old, kv_new, src, lens, pt, Q, P)
    k_ref, k_sc_ref = O.cache_append(k_old, k_kind, k_sc_old, k_new, src, lens, pt, Q, P)

    print(f"cache append case {name}: B={B} Q={Q} P={P} {src}->{kv_kind}/{k_kind} Di={Di}", flush=True)
    seq_t = torch.from_numpy(lens).to(DEV)
    pt_t = torch.from_numpy(pt).to(DEV)
    batch = dsa.make_batch(seq_t, pt_t, Q, P, int(lens.max()), n_slots)
    kv_c, k_c = _dev(kv_old, kv_kind), _dev(k_old, k_kind)
    kv_s = None if kv_sc_old is None else torch.from_numpy(kv_sc_old).to(DEV)
    k_s = None if k_sc_old is None else torch.from_numpy(k_sc_old).to(DEV)
    dsa.dsa_kv_cache_append(batch, _dev(kv_new, src), kv_c, kv_s, _dev(k_new, src), k_c, k_s)
    torch.cuda.synchronize()

    assert np.array_equal(_host(kv_c), kv_ref), "latent cache differs"
    assert np.array_equal(_host(k_c), k_ref), "key cache differs"
    if kv_s is not None:
        assert np.array_equal(_host(kv_s), kv_sc_ref)
    if k_s is not None:
        assert np.array_equal(_host(k_s), k_sc_ref)


def test_cache_append_one_side_only_and_rejects():
    """Only the key cache is written when the latent rows are None; an unsupported pair is
    rejected before anything runs and the cache is unchanged."""
    r = np.random.default_rng(5)
    lens = np.array([70], dtype=np.int32)
    pt = np.array([[1, 0]], dtype=np.int32)
    seq_t, pt_t = torch.from_numpy(lens).to(DEV), torch.from_numpy(pt).to(DEV)
    batch = dsa.make_batch(seq_t, pt_t, 1, 64, 70, 128)
    k_old, k_sc_old = _old_cache(r, 128, 128, "fp8")
    k_new = _bf16_bits(r.standard_normal((1, 1, 128)).astype(np.float32))
    k_c, k_s = _dev(k_old, "fp8"), torch.from_numpy(k_sc_old).to(DEV)
    dsa.dsa_kv_cache_append(batch, None, None, None, _dev(k_new, "bf16"), k_c, k_s)
    torch.cuda.synchronize()
    k_ref, k_sc_ref = O.cache_append(k_old, "fp8", k_sc_old, k_new, "bf16", lens, pt, 1, 64)
    assert np.array_equal(_host(k_c), k_ref) and np.array_equal(_host(k_s), k_sc_ref)

    kv_c = _dev(_bf16_bits(np.zeros((128, 576), np.float32)), "bf16")
    with pytest.raises(dsa.DsaError) as e:
        dsa.dsa_kv_cache_append(batch, torch.ones((1, 1, 576), dtype=torch.float32, device=DEV), kv_c, None)
    assert e.value.status == dsa.DSA_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert not _host(kv_c).any()


@pytest.mark.parametrize("name,lens,Q", [("c5", [700, 1200], 4), ("c2", [1500, 333], 1)])
def test_append_then_decode_step_equals_dense_attention(name, lens, Q):
    """The decode of a verify block: the Q new tokens are appended (bf16 rows into the
    workload's caches), then the fused step runs on the updated caches with k >= context, so
    its output must equal dense attention over the oracle's own appended caches."""
    import dsa_inputs
    from tests.gpu_helpers import batch_of, check_attention, run_step
    cfg = dsa_inputs.scaled_config(name, lens, seed=301, q_per_seq=Q, top_k=max(lens))
    inp = dsa_inputs.make_inputs(cfg)
    t = dsa_inputs.to_torch(inp, cfg, DEV)
    r = np.random.default_rng(302)
    B = len(lens)
    kv_new = _bf16_bits((r.standard_normal((B, Q, O.ROW_DIM)) / 24).astype(np.float32))
    k_new = _bf16_bits((r.standard_normal((B, Q, cfg.idx_dim)) / np.sqrt(cfg.idx_dim)).astype(np.float32))
    print(f"append + step {name}: lens {lens} Q={Q} caches {cfg.kv_dtype}/{cfg.key_dtype}", flush=True)
    dsa.dsa_kv_cache_append(batch_of(cfg, t), _dev(kv_new, "bf16"), t["kv_cache"], t["kv_scale"],
                            _dev(k_new, "bf16"), t["k_cache"], t["k_scale"])
    res = run_step(cfg, t, debug=False)
    kv_ref, kv_sc = O.cache_append(inp["kv_cache"], cfg.kv_dtype, inp["kv_scale"], kv_new, "bf16",
                                   inp["seq_lens"], inp["page_table"], Q, cfg.page_size)
    assert np.array_equal(_host(t["kv_cache"]), kv_ref)
    do, dl = O.dense_mla(inp["q_mla"], cfg.q_mla_dtype, kv_ref, cfg.kv_dtype, kv_sc, inp["seq_lens"],
                         inp["page_table"], Q, cfg.page_size, cfg.sm_scale)
    check_attention(res["out"].cpu().numpy(), do, res["lse"].cpu().numpy(), dl)
