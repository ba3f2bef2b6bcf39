"""The latent up-projection after attention (dsa_latent_up_projection) against the fp64 oracle.

Pass criterion (derived from the arithmetic, the pages state none for this step): on the matrix
cores the f32 activations enter as hi + lo bf16 parts (2^-18 relative) and every product is exact
in the fp32 accumulator; on the one- and two-row vector path every product is exact inside an
fp32 fma that rounds once.  Either way per row max_m |y - y_ref| <= 1e-5 * max_m |y_ref|.
"""
import numpy as np
import pytest
import torch

import dsa_inputs
import sparse_attention_10_amd as dsa
from oracle import dsa_oracle as O
from tests.gpu_helpers import DEV, run_step

pytestmark = pytest.mark.gpu

RTOL = 1e-5


def _gpu_proj(o_np, w_uv, w_o):
    R, H = o_np.shape[0], o_np.shape[1]
    o = torch.from_numpy(np.ascontiguousarray(o_np, dtype=np.float32)).to(DEV)
    wu = torch.from_numpy(w_uv.view(np.int16)).view(torch.bfloat16).to(DEV)
    wo = torch.from_numpy(w_o.view(np.int16)).view(torch.bfloat16).to(DEV)
    y = torch.full((R, w_o.shape[0]), float("nan"), dtype=torch.float32, device=DEV)
    dsa.dsa_latent_up_projection(o, wu, wo, y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _check(y, y_ref):
    for r in range(y_ref.shape[0]):
        scale = max(np.abs(y_ref[r]).max(), 1e-30)
        err = np.abs(y[r].astype(np.float64) - y_ref[r]).max() / scale
        assert err <= RTOL, f"row {r}: normwise error {err:.3e}"


CASES = [  # rows, heads, value dim, model width
    (1, 64, 128, 6144),      # one decode row at the measured width
    (128, 64, 128, 6144),    # the fp8 verify workload's 64 x 2 rows
    (3, 16, 32, 48),
    (37, 64, 64, 96),        # a partial 16-row block
    (20, 8, 96, 160),        # a value dim that leaves a wave of the 128-column tile idle
    (1, 1, 32, 16),
    (1, 20, 96, 160),        # K = 1920 over three splits whose last 128-chunk is partial
    (50, 4, 32, 144),        # 64-row tiles, a ragged second column tile
    (300, 8, 64, 272),       # three 128-row tiles with a ragged tail, three column tiles
    # the vector path for one and two rows (K = 512 times a power of two)
    (2, 16, 128, 6144),      # two rows, K = 2048
    (2, 64, 128, 1008),      # two rows, K = 8192: the matrix cores (the vector path holds up to 4096)
    (1, 16, 64, 1008),       # one row, K = 1024
    (2, 8, 64, 80),          # two rows, K = 512
]


@pytest.mark.parametrize("R,H,Dv,Dm", CASES, ids=[f"R{c[0]}-H{c[1]}-Dv{c[2]}-Dm{c[3]}" for c in CASES])
def test_up_projection_parity(R, H, Dv, Dm):
    rng = np.random.default_rng(R * 1000 + Dv)
    o = (rng.standard_normal((R, H, 512)) / 24).astype(np.float32)
    w_uv, w_o = dsa_inputs.make_up_projection_weights(H, Dv, Dm, seed=51)
    y = _gpu_proj(o, w_uv, w_o)
    y_ref, _ = O.latent_up_projection(o, w_uv, w_o)
    _check(y, y_ref)
    # deterministic: the K-split partial sums are added in a fixed order
    assert np.array_equal(y, _gpu_proj(o, w_uv, w_o))


def test_up_projection_of_a_decode_step():
    """The projection of a fused step's own attention output (fp8 caches, two verify rows)."""
    cfg = dsa_inputs.scaled_config("c5", [3000, 1200], seed=52)
    inp = dsa_inputs.make_inputs(cfg)
    r = run_step(cfg, dsa_inputs.to_torch(inp, cfg, DEV))
    o = r["out"].cpu().numpy().reshape(-1, cfg.mla_heads, 512)
    w_uv, w_o = dsa_inputs.make_up_projection_weights(cfg.mla_heads, 128, 256, seed=53)
    y = _gpu_proj(o, w_uv, w_o)
    y_ref, _ = O.latent_up_projection(o, w_uv, w_o)
    _check(y, y_ref)
