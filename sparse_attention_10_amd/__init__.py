"""MI355X (gfx950) DSA decode path: thin Python binding over the C ABI in include/dsa.h.

Every function here only marshals arguments (torch device tensors -> raw pointers, the current
HIP stream) and calls the same-named C entry point of libdsa.so; all computation runs in the
library's HIP kernels.  If the library is not built the import still works but every call
raises: there is no fallback implementation.  With DSA_DEBUG=1 in the environment the binding
loads libdsa_debug.so instead, the build whose kernels check the data preconditions on the
device (read with debug_check()).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
RELEASE_LIB_PATH = os.path.join(_HERE, "libdsa.so")
DEBUG_LIB_PATH = os.path.join(_HERE, "libdsa_debug.so")
LIB_PATH = DEBUG_LIB_PATH if os.environ.get("DSA_DEBUG", "") not in ("", "0") else RELEASE_LIB_PATH

# error-word bits of the DSA_DEBUG build (dsa.h)
DSA_DEBUG_SEQ_LEN, DSA_DEBUG_PAGE_ID, DSA_DEBUG_SLOT, DSA_DEBUG_NAN_SCORE, DSA_DEBUG_TOPK_INDEX = 1, 2, 4, 8, 16

DSA_OK, DSA_ERR_INVALID_ARGUMENT, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE_TOO_SMALL, DSA_ERR_HIP = range(5)
DSA_F32, DSA_BF16, DSA_FP8_E4M3FN = range(3)

ROW_DIM = 576
V_DIM = 512

EXPORTS = ("dsa_indexer_scores", "dsa_topk", "dsa_topk_workspace_size", "dsa_page_map",
           "dsa_sparse_mla_decode", "dsa_sparse_mla_workspace_size", "dsa_sparse_mla_default_split",
           "dsa_mla_combine", "dsa_decode_step", "dsa_decode_step_workspace_size", "dsa_kv_cache_append",
           "dsa_decode_step_noalloc", "dsa_decode_step_noalloc_max_bytes",
           "dsa_latent_up_projection", "dsa_latent_up_projection_workspace_size",
           "dsa_debug_check", "dsa_debug_enabled",
           "dsa_status_string", "dsa_last_error", "dsa_abi_version")


class DsaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_status_name(status)}: {msg}")
        self.status = status


class DsaBatch(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("q_per_seq", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
                ("num_slots", ctypes.c_int64), ("seq_lens", ctypes.c_void_p), ("page_table", ctypes.c_void_p)]


class DsaDecodeStepArgs(ctypes.Structure):
    _fields_ = [("batch", DsaBatch),
                ("q_idx", ctypes.c_void_p), ("q_idx_dtype", ctypes.c_int), ("w", ctypes.c_void_p),
                ("k_cache", ctypes.c_void_p), ("k_dtype", ctypes.c_int), ("k_scale", ctypes.c_void_p),
                ("idx_heads", ctypes.c_int32), ("idx_dim", ctypes.c_int32),
                ("top_k", ctypes.c_int32),
                ("q_mla", ctypes.c_void_p), ("q_mla_dtype", ctypes.c_int),
                ("kv_cache", ctypes.c_void_p), ("kv_dtype", ctypes.c_int), ("kv_scale", ctypes.c_void_p),
                ("mla_heads", ctypes.c_int32), ("sm_scale", ctypes.c_float), ("n_split", ctypes.c_int32),
                ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("debug_scores", ctypes.c_void_p), ("debug_idx", ctypes.c_void_p),
                ("debug_slots", ctypes.c_void_p), ("prefill_rows_per_block", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """The library every call goes to: LIB_PATH (built in-tree by sparse_attention_10_amd.build),
    loaded once."""
    global _lib
    if _lib is None:
        _lib = load_library(LIB_PATH)
    return _lib


def load_library(path: str) -> ctypes.CDLL:
    """Load one build of the library (libdsa.so or libdsa_debug.so) with its signatures set."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m sparse_attention_10_amd.build`")
    L = ctypes.CDLL(path)
    vp, i32, i64, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    bp = ctypes.POINTER(DsaBatch)
    e = ctypes.c_int
    sig = {
        "dsa_indexer_scores": (e, [bp, vp, e, vp, vp, e, vp, i32, i32, vp, i64, vp]),
        "dsa_topk": (e, [bp, vp, i64, i32, vp, vp, vp, sz, vp]),
        "dsa_topk_workspace_size": (sz, [bp, i32]),
        "dsa_page_map": (e, [bp, vp, i32, vp, vp]),
        "dsa_sparse_mla_decode": (e, [i32, i32, vp, e, vp, e, vp, i64, vp, i32, i32, f32, vp, vp, i32, vp, sz, vp]),
        "dsa_sparse_mla_workspace_size": (sz, [i32, i32, i32, i32, i32, e, e]),
        "dsa_sparse_mla_default_split": (i32, [i32, i32, i32, i32, e]),
        "dsa_mla_combine": (e, [i32, i32, i32, vp, vp, vp, vp, vp, vp]),
        "dsa_decode_step": (e, [ctypes.POINTER(DsaDecodeStepArgs), vp, sz, vp]),
        "dsa_decode_step_workspace_size": (sz, [ctypes.POINTER(DsaDecodeStepArgs)]),
        "dsa_decode_step_noalloc": (e, [ctypes.POINTER(DsaDecodeStepArgs), vp]),
        "dsa_latent_up_projection": (e, [i32, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]),
        "dsa_latent_up_projection_workspace_size": (sz, [i32, i32, i32, i32]),
        "dsa_decode_step_noalloc_max_bytes": (sz, []),
        "dsa_kv_cache_append": (e, [bp, vp, e, vp, e, vp, vp, e, i32, vp, e, vp, vp]),
        "dsa_debug_check": (e, [ctypes.POINTER(ctypes.c_uint32), vp]),
        "dsa_debug_enabled": (i32, []),
        "dsa_status_string": (ctypes.c_char_p, [e]),
        "dsa_last_error": (ctypes.c_char_p, []),
        "dsa_abi_version": (i32, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype, fn.argtypes = res, args
    return L


class using_library:
    """Context manager that routes this module's calls to another loaded build (for example the
    DSA_DEBUG one) and restores the previous one afterwards."""

    def __init__(self, L: ctypes.CDLL):
        self._L, self._prev = L, None

    def __enter__(self):
        global _lib
        self._prev, _lib = _lib, self._L
        return self._L

    def __exit__(self, *exc):
        global _lib
        _lib = self._prev
        return False


def _status_name(s: int) -> str:
    try:
        return lib().dsa_status_string(s).decode()
    except Exception:  # the library may be what failed to load
        return f"status {s}"


def _check(status: int):
    if status != DSA_OK:
        raise DsaError(status, lib().dsa_last_error().decode())


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DSA_F32
    if t.dtype == torch.bfloat16:
        return DSA_BF16
    if t.dtype == torch.float8_e4m3fn:
        return DSA_FP8_E4M3FN
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("DSA tensors must live in GPU memory")
    if not t.is_contiguous():
        raise ValueError("DSA tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def make_batch(seq_lens: torch.Tensor, page_table: torch.Tensor, q_per_seq: int, page_size: int,
               max_seq_len: int, num_slots: int) -> DsaBatch:
    """Host descriptor of a ragged paged batch (seq_lens [B] i32, page_table [B, maxP] i32 on the GPU)."""
    if seq_lens.dtype != torch.int32 or page_table.dtype != torch.int32:
        raise TypeError("seq_lens and page_table must be int32")
    b = DsaBatch(seq_lens.numel(), q_per_seq, max_seq_len, page_size, page_table.shape[1], num_slots,
                 _ptr(seq_lens), _ptr(page_table))
    b._keep = (seq_lens, page_table)   # the descriptor holds raw pointers: keep the tensors alive
    return b


def dsa_indexer_scores(batch: DsaBatch, q: torch.Tensor, w: torch.Tensor, k_cache: torch.Tensor,
                       k_scale: Optional[torch.Tensor], scores: torch.Tensor, stream=None) -> torch.Tensor:
    """scores[b,i,t] for t < L_b (see dsa.h); q [B,Q,Hi,Di], w [B,Q,Hi], k_cache [slots,Di]."""
    Hi, Di = q.shape[-2], q.shape[-1]
    _check(lib().dsa_indexer_scores(ctypes.byref(batch), _ptr(q), dtype_code(q), _ptr(w), _ptr(k_cache),
                                    dtype_code(k_cache), _ptr(k_scale), Hi, Di, _ptr(scores),
                                    scores.shape[-1], _stream(stream)))
    return scores


def topk_workspace_bytes(batch: DsaBatch, k: int) -> int:
    return lib().dsa_topk_workspace_size(ctypes.byref(batch), k)


def dsa_topk(batch: DsaBatch, scores: torch.Tensor, k: int, topk_idx: torch.Tensor,
             topk_slots: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
             stream=None) -> torch.Tensor:
    """Top-k with the fused page map (see dsa.h).  Long rows use a workspace of
    topk_workspace_bytes(batch, k) bytes (no initial contents); without one a buffer is made."""
    need = topk_workspace_bytes(batch, k)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=scores.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().dsa_topk(ctypes.byref(batch), _ptr(scores), scores.shape[-1], k, _ptr(topk_idx),
                          _ptr(topk_slots), _ptr(workspace), nbytes, _stream(stream)))
    return topk_idx


def dsa_page_map(batch: DsaBatch, topk_idx: torch.Tensor, slots: torch.Tensor, stream=None) -> torch.Tensor:
    _check(lib().dsa_page_map(ctypes.byref(batch), _ptr(topk_idx), topk_idx.shape[-1], _ptr(slots),
                              _stream(stream)))
    return slots


def mla_workspace_bytes(batch: int, q_per_seq: int, n_heads: int, k: int, n_split: int, q_dtype: int,
                        kv_dtype: int) -> int:
    return lib().dsa_sparse_mla_workspace_size(batch, q_per_seq, n_heads, k, n_split, q_dtype, kv_dtype)


def dsa_sparse_mla_decode(q: torch.Tensor, kv_cache: torch.Tensor, kv_scale: Optional[torch.Tensor],
                          slots: torch.Tensor, sm_scale: float, out: torch.Tensor,
                          lse: Optional[torch.Tensor] = None, n_split: int = 0,
                          workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """q [B,Q,H,576], kv_cache [slots,576], slots [B,Q,k] -> out [B,Q,H,512] (+ lse [B,Q,H])."""
    B, Q, H = q.shape[0], q.shape[1], q.shape[2]
    k = slots.shape[-1]
    need = mla_workspace_bytes(B, Q, H, k, n_split, dtype_code(q), dtype_code(kv_cache))
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check(lib().dsa_sparse_mla_decode(B, Q, _ptr(q), dtype_code(q), _ptr(kv_cache), dtype_code(kv_cache),
                                       _ptr(kv_scale), kv_cache.shape[0], _ptr(slots), k, H, float(sm_scale),
                                       _ptr(out), _ptr(lse), n_split, _ptr(workspace),
                                       0 if workspace is None else workspace.numel(), _stream(stream)))
    return out


def dsa_mla_combine(part_o: torch.Tensor, part_m: torch.Tensor, part_l: torch.Tensor, out: torch.Tensor,
                    lse: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """part_o [rows, n_split, H, 512], part_m / part_l [rows, n_split, H] -> out [rows, H, 512]."""
    rows, ns, H = part_m.shape
    _check(lib().dsa_mla_combine(rows, H, ns, _ptr(part_o), _ptr(part_m), _ptr(part_l), _ptr(out), _ptr(lse),
                                 _stream(stream)))
    return out


def decode_step_args(batch: DsaBatch, q_idx, w, k_cache, k_scale, top_k: int, q_mla, kv_cache, kv_scale,
                     sm_scale: float, out, lse=None, n_split: int = 0, debug_scores=None, debug_idx=None,
                     debug_slots=None, prefill_rows_per_block: int = 0) -> DsaDecodeStepArgs:
    a = DsaDecodeStepArgs()
    a.batch = batch
    a.q_idx, a.q_idx_dtype, a.w = _ptr(q_idx), dtype_code(q_idx), _ptr(w)
    a.k_cache, a.k_dtype, a.k_scale = _ptr(k_cache), dtype_code(k_cache), _ptr(k_scale)
    a.idx_heads, a.idx_dim = q_idx.shape[-2], q_idx.shape[-1]
    a.top_k = top_k
    a.q_mla, a.q_mla_dtype = _ptr(q_mla), dtype_code(q_mla)
    a.kv_cache, a.kv_dtype, a.kv_scale = _ptr(kv_cache), dtype_code(kv_cache), _ptr(kv_scale)
    a.mla_heads, a.sm_scale, a.n_split = q_mla.shape[2], float(sm_scale), n_split
    a.out, a.lse = _ptr(out), _ptr(lse)
    a.debug_scores, a.debug_idx, a.debug_slots = _ptr(debug_scores), _ptr(debug_idx), _ptr(debug_slots)
    a.prefill_rows_per_block = prefill_rows_per_block
    a._keep = (batch, q_idx, w, k_cache, k_scale, q_mla, kv_cache, kv_scale, out, lse, debug_scores, debug_idx,
               debug_slots)
    return a


def decode_step_workspace_bytes(args: DsaDecodeStepArgs) -> int:
    return lib().dsa_decode_step_workspace_size(ctypes.byref(args))


def dsa_decode_step(args: DsaDecodeStepArgs, workspace: Optional[torch.Tensor], stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().dsa_decode_step(ctypes.byref(args), _ptr(workspace), nbytes, _stream(stream)))


def dsa_decode_step_noalloc(args: DsaDecodeStepArgs, stream=None):
    """The fused step on the library's fixed per-device scratch buffer (no workspace argument)."""
    _check(lib().dsa_decode_step_noalloc(ctypes.byref(args), _stream(stream)))


def decode_step_noalloc_max_bytes() -> int:
    return lib().dsa_decode_step_noalloc_max_bytes()


def up_projection_workspace_bytes(rows: int, n_heads: int, v_dim: int, d_model: int) -> int:
    return lib().dsa_latent_up_projection_workspace_size(rows, n_heads, v_dim, d_model)


def dsa_latent_up_projection(attn_out: torch.Tensor, w_uv: torch.Tensor, w_o: torch.Tensor, y: torch.Tensor,
                             workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """attn_out [..., H, 512] f32 (rows flattened), w_uv [H, Dv, 512] bf16, w_o [Dm, H*Dv] bf16
    -> y [rows, Dm] f32 (see dsa.h)."""
    H, Dv, Dm = w_uv.shape[0], w_uv.shape[1], w_o.shape[0]
    rows = attn_out.numel() // (H * 512)
    need = up_projection_workspace_bytes(rows, H, Dv, Dm)
    if workspace is None:
        workspace = torch.empty(max(1, need), dtype=torch.uint8, device=attn_out.device)
    _check(lib().dsa_latent_up_projection(rows, H, Dv, Dm, _ptr(attn_out), _ptr(w_uv), _ptr(w_o), _ptr(y),
                                          _ptr(workspace), workspace.numel(), _stream(stream)))
    return y


def dsa_kv_cache_append(batch: DsaBatch, kv_new: Optional[torch.Tensor], kv_cache: Optional[torch.Tensor],
                        kv_scale: Optional[torch.Tensor], k_new: Optional[torch.Tensor] = None,
                        k_cache: Optional[torch.Tensor] = None, k_scale: Optional[torch.Tensor] = None,
                        stream=None):
    """Write the new tokens' rows into their paged slots (see dsa.h): kv_new [B,Q,576] into
    kv_cache [slots,576] (+ kv_scale for fp8), k_new [B,Q,Di] into k_cache [slots,Di] (+ k_scale).
    Either pair may be None."""
    def code(t):
        return DSA_F32 if t is None else dtype_code(t)
    head_dim = 0 if k_new is None else k_new.shape[-1]
    _check(lib().dsa_kv_cache_append(ctypes.byref(batch), _ptr(kv_new), code(kv_new),
                                     _ptr(kv_cache if kv_new is not None else None), code(kv_cache), _ptr(kv_scale),
                                     _ptr(k_new), code(k_new), head_dim,
                                     _ptr(k_cache if k_new is not None else None), code(k_cache), _ptr(k_scale),
                                     _stream(stream)))


def debug_enabled() -> bool:
    """True for the DSA_DEBUG build (libdsa_debug.so)."""
    return bool(lib().dsa_debug_enabled())


def debug_check(stream=None) -> int:
    """DSA_DEBUG build: wait for `stream`, return the data-precondition bits the kernels flagged
    since the last check (DSA_DEBUG_* flags, 0 when none) and clear them.  The release build
    raises DsaError(DSA_ERR_UNSUPPORTED)."""
    flags = ctypes.c_uint32(0)
    st = lib().dsa_debug_check(ctypes.byref(flags), _stream(stream))
    if st not in (DSA_OK, DSA_ERR_INVALID_ARGUMENT):
        _check(st)
    return int(flags.value)
