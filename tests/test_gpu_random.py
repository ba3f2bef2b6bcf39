"""A seeded sweep of fused-step configurations under the staged protocol (the same checks as
test_gpu_parity.test_decode_step_staged): the step's scores against the fp64 indexer, its
selection and slots bit-exact against the fp64 top-k and page map on its own scores, its
attention against fp64 sparse MLA on its own slots, and its selection against the fp64
selection up to ties at the k-th score.

Each configuration draws the dtype family (f32, bf16, fp8 caches), batch, rows per sequence
(decode, verify and a few many-row chunks), ragged lengths (some below k, so rows are padded
with -1), page size (powers of two, sizes that 16 does not divide, page size 1), k and the MLA
head count from a fixed seed, so every run checks the same cases (the first DSA_RANDOM_CASES of the
sequence, 96 by default).  A second sweep (DSA_RANDOM_GROUPED_CASES, 32 by default) draws 8 or 16
sequences of 2-4 verify rows, half of them sharing one indexer query per sequence, the batches
whose sparse MLA runs a sequence's rows on one XCD."""
import os

import numpy as np
import pytest

import dsa_inputs
from tests.gpu_helpers import DEV
from tests.test_gpu_parity import _check_staged

pytestmark = pytest.mark.gpu

N_CASES = int(os.environ.get("DSA_RANDOM_CASES", "96"))   # a longer sweep: set it higher


def draw_case(i):
    rng = np.random.default_rng([2024, i])
    name = ["c1", "c2", "c5"][i % 3]                   # f32 / bf16 / fp8 caches
    Q = int(rng.choice([1, 1, 2, 3, 4, 16, 20]))
    B = int(rng.integers(1, 7)) if Q < 16 else int(rng.integers(1, 3))
    P = int(rng.choice([1, 16, 24, 32, 48, 64, 128]))
    k = int(rng.choice([1, 64, 256, 1000, 2048]))
    H = int(rng.choice([1, 5, 16, 64])) if name == "c1" else int(rng.choice([16, 32, 48, 64]))
    lens = [int(x) for x in rng.integers(Q, 9000, size=B)]
    if rng.random() < 0.5:                             # one sequence shorter than k
        lens[int(rng.integers(0, B))] = int(rng.integers(Q, max(Q + 1, min(k, 9000))))
    return name, lens, dict(q_per_seq=Q, page_size=P, top_k=k, mla_heads=H)


@pytest.mark.parametrize("i", range(N_CASES))
def test_decode_step_staged_random(i):
    name, lens, kw = draw_case(i)
    print(f"case {i}: {name} lens={lens} {kw}", flush=True)
    cfg = dsa_inputs.scaled_config(name, lens, seed=3000 + i, **kw)
    inp = dsa_inputs.make_inputs(cfg)
    _check_staged(cfg, inp, dsa_inputs.to_torch(inp, cfg, DEV))


N_GROUPED = int(os.environ.get("DSA_RANDOM_GROUPED_CASES", "32"))


def draw_grouped_case(i):
    """8 or 16 sequences of 2-4 verify rows (bf16 or fp8 caches), with or without one indexer
    query per sequence: the sparse MLA then runs each sequence's rows on one XCD, chunk by
    chunk (nearly equal selections when the query is shared)."""
    rng = np.random.default_rng([2025, i])
    name = ["c2", "c5"][i % 2]
    B = int(rng.choice([8, 16]))
    Q = int(rng.integers(2, 5))
    P = int(rng.choice([16, 24, 32, 64, 128]))
    k = int(rng.choice([64, 256, 1000, 2048]))
    H = int(rng.choice([16, 32, 48, 64]))
    lens = [int(x) for x in rng.integers(Q, 3000, size=B)]
    if rng.random() < 0.5:
        lens[int(rng.integers(0, B))] = int(rng.integers(Q, max(Q + 1, min(k, 3000))))
    shared = bool(rng.random() < 0.5)
    return name, lens, dict(q_per_seq=Q, page_size=P, top_k=k, mla_heads=H, shared_index_query=shared)


@pytest.mark.parametrize("i", range(N_GROUPED))
def test_decode_step_staged_random_grouped(i):
    name, lens, kw = draw_grouped_case(i)
    print(f"grouped case {i}: {name} lens={lens} {kw}", flush=True)
    cfg = dsa_inputs.scaled_config(name, lens, seed=4000 + i, **kw)
    inp = dsa_inputs.make_inputs(cfg)
    _check_staged(cfg, inp, dsa_inputs.to_torch(inp, cfg, DEV))
