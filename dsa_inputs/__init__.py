"""Seeded synthetic inputs for the DSA decode path.

This module only draws random numbers and stores them in the dtypes the path
reads (f32, bf16 bit patterns, fp8 e4m3fn codes with a per-token f32 scale).
It holds none of the method's arithmetic: no indexer, no selection, no page
mapping, no attention.  Both the fp64 oracle (``oracle/``) and the HIP path
(``sparse_attention_10_amd``) are fed from the arrays it returns, so that the
two sides read identical bits.

Shapes and distributions follow the DSA workloads the library is built for:
64 indexer heads x 128 dims, top-k 2048, 64 MLA heads over 576-wide compressed
latent rows (512 latent + 64 RoPE), page size 64, fp8 e4m3 caches for the
speculative-verify shape (Show HN: "Chay GLM 5.2 tren may tinh cham", section
on the main implemented features: 576 values per token, 64 heads, no GQA;
renning22/glm-5.2-4090 README, usage section: fp8_e4m3 KV cache).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np

PAGE_SIZE = 64
MLA_DIM = 576          # 512 latent + 64 RoPE values per cached token
V_DIM = 512            # V is the first 512 values of the latent row
FP8_MAX = 448.0        # largest finite e4m3fn magnitude

# tensor ids for independent random streams: default_rng([seed, TENSOR_ID])
_T_LENS, _T_PERM, _T_QIDX, _T_W, _T_KEYS, _T_QMLA, _T_KV = range(7)


@dataclasses.dataclass
class DsaConfig:
    name: str
    batch: int
    q_per_seq: int
    seq_lens: List[int]            # L_b, counting the Q new tokens
    idx_heads: int                 # Hi
    idx_dim: int                   # Di
    q_idx_dtype: str               # 'f32' | 'bf16'
    key_dtype: str                 # 'f32' | 'bf16' | 'fp8'
    top_k: int
    mla_heads: int                 # H
    q_mla_dtype: str               # 'f32' | 'bf16'
    kv_dtype: str                  # 'f32' | 'bf16' | 'fp8'
    q_idx_std: float
    key_std: float
    w_scale: float
    mla_std: float
    sm_scale: float
    page_size: int = PAGE_SIZE
    seed: int = 0
    # the verify rows of a sequence share the indexer query and head weights of its first row
    # (their selections then nest: row i sees one more token than row i - 1)
    shared_index_query: bool = False

    @property
    def max_seq_len(self) -> int:
        return max(self.seq_lens)

    @property
    def pages_per_seq(self) -> List[int]:
        return [(L + self.page_size - 1) // self.page_size for L in self.seq_lens]

    @property
    def max_pages(self) -> int:
        return max(self.pages_per_seq)

    @property
    def num_pages(self) -> int:
        return sum(self.pages_per_seq)

    @property
    def num_slots(self) -> int:
        return self.num_pages * self.page_size


def _std(d: int) -> float:
    return 1.0 / math.sqrt(d)


def base_config(name: str, seed: Optional[int] = None) -> DsaConfig:
    """The workloads, by name: c1 (tiny fp32), c2 (32K single stream), c2_128k (the
    same layer at 128K), c3 (batch 32, ragged 4K-128K), c4 (4096-token chunked prefill
    over a 64K prefix), c5 (fp8 caches, batch 64 x 2 speculative-verify rows at 64K),
    c5_q4 (the same with 4 verify rows per sequence: a draft depth of 3), c5_shared (c5
    whose two verify rows per sequence share one indexer query, so that they select nearly the
    same tokens)."""
    name = name.lower()
    s = 1000 + int(name[1]) if seed is None else seed
    if name == "c1":
        return DsaConfig("c1", 1, 1, [4096], 4, 64, "f32", "f32", 256, 16, "f32", "f32",
                         _std(64), _std(64), 1.0, _std(576), 1.0 / math.sqrt(576), seed=s)
    common = dict(idx_heads=64, idx_dim=128, q_idx_dtype="bf16", key_dtype="bf16", top_k=2048,
                  mla_heads=64, q_mla_dtype="bf16", kv_dtype="bf16", q_idx_std=_std(128),
                  key_std=_std(128), w_scale=1.0 / 64, mla_std=_std(576),
                  sm_scale=1.0 / math.sqrt(576), seed=s)
    if name == "c2":
        return DsaConfig("c2", 1, 1, [32768], **common)
    if name == "c2_128k":      # the single-stream decode layer at a 128K context
        common["seed"] = 1006 if seed is None else seed
        return DsaConfig("c2_128k", 1, 1, [131072], **common)
    if name == "c3":
        rng = np.random.default_rng([s, _T_LENS])
        lens = rng.integers(4096, 131072, size=32, endpoint=True).tolist()
        return DsaConfig("c3", 32, 1, [int(x) for x in lens], **common)
    if name == "c4":
        return DsaConfig("c4", 1, 4096, [65536 + 4096], **common)
    if name == "c5":
        c = dict(common)
        c.update(key_dtype="fp8", kv_dtype="fp8")
        return DsaConfig("c5", 64, 2, [65536] * 64, **c)
    if name == "c5_shared":    # c5 with a sequence's verify rows selecting nearly the same tokens
        c = dict(common)
        c.update(key_dtype="fp8", kv_dtype="fp8")
        return DsaConfig("c5_shared", 64, 2, [65536] * 64, shared_index_query=True, **c)
    if name == "c5_q4":        # deeper speculative verify: 4 rows per sequence
        c = dict(common)
        c.update(key_dtype="fp8", kv_dtype="fp8", seed=1007 if seed is None else seed)
        return DsaConfig("c5_q4", 64, 4, [65536] * 64, **c)
    raise ValueError(f"unknown config {name!r}")


def scaled_config(name: str, seq_lens: Sequence[int], seed: int, **overrides) -> DsaConfig:
    """A workload with the dtypes and distributions of ``name`` but other
    sequence lengths (and any other field overridden), for parity tests at
    sizes the oracle finishes in seconds."""
    c = base_config(name, seed)
    c = dataclasses.replace(c, seq_lens=[int(x) for x in seq_lens], batch=len(seq_lens), seed=seed)
    return dataclasses.replace(c, **overrides) if overrides else c


# ---------------------------------------------------------------------------
# dtype encodings (torch's CPU conversions round to nearest even)

def encode_bf16(x: np.ndarray) -> np.ndarray:
    """float array -> uint16 bf16 bit patterns (round to nearest even)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def encode_fp8_rows(x: np.ndarray):
    """Per-row (per-token) fp8 e4m3fn quantization of a [N, D] array.

    scale = max|row| / 448 (1 for an all-zero row), stored as f32; codes are the
    nearest-even e4m3fn codes of row / scale.  Returns (codes uint8 [N, D],
    scale f32 [N])."""
    import torch
    x = np.asarray(x, dtype=np.float64)
    amax = np.abs(x).max(axis=1)
    scale = np.where(amax > 0, amax / FP8_MAX, 1.0).astype(np.float32)
    y = (x / scale.astype(np.float64)[:, None]).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def _encode(x: np.ndarray, dtype: str):
    if dtype == "f32":
        return x.astype(np.float32), None
    if dtype == "bf16":
        return encode_bf16(x), None
    if dtype == "fp8":
        shp = x.shape
        codes, scale = encode_fp8_rows(x.reshape(-1, shp[-1]))
        return codes.reshape(shp), scale
    raise ValueError(dtype)


def page_table_for(cfg: DsaConfig, rng: np.random.Generator) -> np.ndarray:
    """Ragged page tables dealt from one shuffled pool of physical pages.
    Unused entries are -1 (never read)."""
    perm = rng.permutation(cfg.num_pages).astype(np.int32)
    pt = np.full((cfg.batch, cfg.max_pages), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(cfg.pages_per_seq):
        pt[b, :n] = perm[off:off + n]
        off += n
    return pt


def make_inputs(cfg: DsaConfig, with_mla: bool = True, with_indexer: bool = True) -> Dict[str, np.ndarray]:
    """Draw every input of the decode step for ``cfg`` on the host.

    Returned arrays (numpy; bf16 as uint16 bits, fp8 as uint8 codes):
      seq_lens [B] i32, page_table [B, max_pages] i32,
      q_idx [B,Q,Hi,Di], w [B,Q,Hi] f32, k_cache [num_slots,Di], k_scale [num_slots] f32|None,
      q_mla [B,Q,H,576], kv_cache [num_slots,576], kv_scale [num_slots] f32|None.
    """
    s = cfg.seed
    out: Dict[str, np.ndarray] = {}
    out["seq_lens"] = np.asarray(cfg.seq_lens, dtype=np.int32)
    out["page_table"] = page_table_for(cfg, np.random.default_rng([s, _T_PERM]))
    B, Q, N = cfg.batch, cfg.q_per_seq, cfg.num_slots
    if with_indexer:
        r = np.random.default_rng([s, _T_QIDX])
        out["q_idx"], _ = _encode(r.standard_normal((B, Q, cfg.idx_heads, cfg.idx_dim)) * cfg.q_idx_std,
                                  cfg.q_idx_dtype)
        r = np.random.default_rng([s, _T_W])
        out["w"] = (r.random((B, Q, cfg.idx_heads)) * cfg.w_scale).astype(np.float32)
        if cfg.shared_index_query:
            out["q_idx"] = np.ascontiguousarray(np.broadcast_to(out["q_idx"][:, :1], out["q_idx"].shape))
            out["w"] = np.ascontiguousarray(np.broadcast_to(out["w"][:, :1], out["w"].shape))
        r = np.random.default_rng([s, _T_KEYS])
        out["k_cache"], out["k_scale"] = _encode(r.standard_normal((N, cfg.idx_dim)) * cfg.key_std,
                                                 cfg.key_dtype)
    if with_mla:
        r = np.random.default_rng([s, _T_QMLA])
        out["q_mla"], _ = _encode(r.standard_normal((B, Q, cfg.mla_heads, MLA_DIM)) * cfg.mla_std,
                                  cfg.q_mla_dtype)
        r = np.random.default_rng([s, _T_KV])
        out["kv_cache"], out["kv_scale"] = _encode(r.standard_normal((N, MLA_DIM)) * cfg.mla_std,
                                                   cfg.kv_dtype)
    return out


# tensor ids of the projection weights after attention (their own random streams)
_T_WUV, _T_WO = 20, 21


def make_up_projection_weights(n_heads: int, v_dim: int, d_model: int, seed: int):
    """Synthetic weights of the projection after attention, as bf16 bit patterns:
    w_uv [H, Dv, 512] ~ N(0,1)/sqrt(512) (per head, the value block of kv_b) and
    w_o [Dm, H*Dv] ~ N(0,1)/sqrt(H*Dv) (o_proj)."""
    r = np.random.default_rng([seed, _T_WUV])
    w_uv = encode_bf16(r.standard_normal((n_heads, v_dim, V_DIM)) / math.sqrt(V_DIM))
    r = np.random.default_rng([seed, _T_WO])
    w_o = encode_bf16(r.standard_normal((d_model, n_heads * v_dim)) / math.sqrt(n_heads * v_dim))
    return w_uv, w_o


def make_up_projection_weights_torch(n_heads: int, v_dim: int, d_model: int, seed: int, device):
    """The same kind of weights drawn in device memory (torch.bfloat16 tensors)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed + 7919)
    w_uv = (torch.randn((n_heads, v_dim, V_DIM), generator=g, device=device) / math.sqrt(V_DIM)).to(torch.bfloat16)
    w_o = (torch.randn((d_model, n_heads * v_dim), generator=g, device=device) /
           math.sqrt(n_heads * v_dim)).to(torch.bfloat16)
    return w_uv, w_o


def make_inputs_torch(cfg: DsaConfig, device, with_mla: bool = True, with_indexer: bool = True):
    """Draw the same kind of inputs directly in device memory with a seeded
    torch generator (for the full-size workloads, whose caches run to GBs).

    The values differ from ``make_inputs`` (another generator) but the shapes,
    dtypes, distributions and page-table structure are the same.  Returns a
    dict of torch tensors; bf16 tensors are torch.bfloat16, fp8 codes are
    torch.float8_e4m3fn, scales f32."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(cfg.seed)
    out = {}
    out["seq_lens"] = torch.tensor(cfg.seq_lens, dtype=torch.int32, device=device)
    pt = page_table_for(cfg, np.random.default_rng([cfg.seed, _T_PERM]))
    out["page_table"] = torch.from_numpy(pt).to(device)
    B, Q, N = cfg.batch, cfg.q_per_seq, cfg.num_slots
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}

    def draw(shape, std, dtype):
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        x.mul_(std)
        if dtype == "fp8":
            amax = x.abs().amax(dim=-1)
            scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
            codes = (x / scale.unsqueeze(-1)).to(torch.float8_e4m3fn)
            return codes, scale.float()
        return x.to(tdt[dtype]), None

    if with_indexer:
        out["q_idx"], _ = draw((B, Q, cfg.idx_heads, cfg.idx_dim), cfg.q_idx_std, cfg.q_idx_dtype)
        out["w"] = torch.rand((B, Q, cfg.idx_heads), generator=g, device=device) * cfg.w_scale
        if cfg.shared_index_query:
            out["q_idx"] = out["q_idx"][:, :1].expand_as(out["q_idx"]).contiguous()
            out["w"] = out["w"][:, :1].expand_as(out["w"]).contiguous()
        # the caches are drawn in slabs to bound the f32 temporary
        out["k_cache"], out["k_scale"] = _draw_cache(draw, N, cfg.idx_dim, cfg.key_std, cfg.key_dtype, device)
    if with_mla:
        out["q_mla"], _ = draw((B, Q, cfg.mla_heads, MLA_DIM), cfg.mla_std, cfg.q_mla_dtype)
        out["kv_cache"], out["kv_scale"] = _draw_cache(draw, N, MLA_DIM, cfg.mla_std, cfg.kv_dtype, device)
    return out


def _draw_cache(draw, n, d, std, dtype, device, slab=1 << 20):
    import torch
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}[dtype]
    cache = torch.empty((n, d), dtype=tdt, device=device)
    scale = torch.empty((n,), dtype=torch.float32, device=device) if dtype == "fp8" else None
    for a in range(0, n, slab):
        b = min(n, a + slab)
        x, s = draw((b - a, d), std, dtype)
        cache[a:b] = x
        if scale is not None:
            scale[a:b] = s
    return cache, scale


def to_torch(inp: Dict[str, np.ndarray], cfg: DsaConfig, device) -> Dict[str, "object"]:
    """Move make_inputs() arrays to ``device`` as torch tensors of the stored dtypes
    (bf16 bit patterns -> torch.bfloat16, fp8 codes -> torch.float8_e4m3fn), bit for bit."""
    import torch
    out = {}
    dt = {"q_idx": cfg.q_idx_dtype, "k_cache": cfg.key_dtype, "q_mla": cfg.q_mla_dtype,
          "kv_cache": cfg.kv_dtype}
    for name, arr in inp.items():
        if arr is None:
            out[name] = None
            continue
        kind = dt.get(name)
        if kind == "bf16":
            t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
        elif kind == "fp8":
            t = torch.from_numpy(np.ascontiguousarray(arr)).view(torch.float8_e4m3fn)
        else:
            t = torch.from_numpy(np.ascontiguousarray(arr))
        out[name] = t.to(device)
    return out


def from_torch(t) -> np.ndarray:
    """Device tensor -> numpy array of the stored bits (bf16 -> uint16, fp8 -> uint8)."""
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()
