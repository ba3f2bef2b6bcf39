#!/usr/bin/env python3
"""Benchmark of the DSA decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c2|c3|c4|c5|c1] [--eager]

One step = one dsa_decode_step call: lightning indexer -> top-k with the fused page map ->
sparse MLA -> split-k merge, over one batch of synthetic input.  Default workload: one
decode layer of a 32K-token single stream (batch 1, 64 indexer heads x 128 dims bf16,
top-k 2048, 64 MLA heads over 576-wide bf16 latent rows).

Inputs are seeded and generated in device memory.  The step's inputs are replicated R times
over disjoint pages of one paged pool (R chosen so one cycle touches >= 512 MB), and step j
uses replica j mod R, so the 256 MB Infinity Cache cannot serve a step from the previous one.
The K timed steps are one HIP-graph replay (the launch overhead a serving loop would amortise),
bracketed by synchronisation; the eager rate is reported beside it.

Printed: ONE JSON line with the metric (algorithmic GB/s of the whole step), ms per step
(= microseconds per layer-step / 1000), a roofline object for the dominant kernel (timed
alone with HIP events on its own stream), per-stage timings, and the fp64 oracle timed on the
host's cores on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DSA decode-step µs/layer + achieved HBM GB/s (% of peak), 32K–128K ctx"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
MALL_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", default="c2")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a graph replay")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle time for the CPU baseline")
    ap.add_argument("--rotate", type=int, default=0, help="input replicas (0 = enough to exceed 512 MB)")
    ap.add_argument("--n-split", type=int, default=0, help="MLA split-k chunks (0 = library default)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 10 plain 1 GiB device copies (reference for the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


# ---------------------------------------------------------------------------------------------
# algorithmic bytes and flops of one step (each input read once, each output written once)

def step_bytes(cfg, lens, union_rows=None):
    """Bytes the method must move for one step of `cfg` with realised lengths `lens`:
    keys (+ per-token fp8 scale) of every visible token, q, w, the page-table entries in use,
    the selected latent rows (+ scale) counted once per sequence, q_mla, out and lse."""
    kb = {"f32": 4, "bf16": 2, "fp8": 1}
    B, Q = cfg.batch, cfg.q_per_seq
    key_row = cfg.idx_dim * kb[cfg.key_dtype] + (4 if cfg.key_dtype == "fp8" else 0)
    lat_row = 576 * kb[cfg.kv_dtype] + (4 if cfg.kv_dtype == "fp8" else 0)
    keys = sum(lens) * key_row
    q = B * Q * cfg.idx_heads * cfg.idx_dim * kb[cfg.q_idx_dtype] + B * Q * cfg.idx_heads * 4
    pt = sum((L + cfg.page_size - 1) // cfg.page_size for L in lens) * 4 + B * 4
    if union_rows is None:
        union_rows = sum(min(cfg.top_k * Q, L) for L in lens)
    rows = union_rows * lat_row
    qm = B * Q * cfg.mla_heads * 576 * kb[cfg.q_mla_dtype]
    out = B * Q * cfg.mla_heads * (512 + 1) * 4
    return dict(indexer=keys + q + pt, mla=rows + qm + out, total=keys + q + pt + rows + qm + out)


def step_flops(cfg, lens):
    Q = cfg.q_per_seq
    vis = sum(sum(L - Q + i + 1 for i in range(Q)) for L in lens)
    idx = 2.0 * vis * cfg.idx_heads * cfg.idx_dim
    sel = sum(sum(min(cfg.top_k, L - Q + i + 1) for i in range(Q)) for L in lens)
    mla = 2.0 * sel * cfg.mla_heads * (576 + 512)
    return dict(indexer=idx, mla=mla)


# ---------------------------------------------------------------------------------------------

def build_replicas(cfg, R, dev):
    """R input replicas over disjoint pages of one pool; returns (cache tensors, list of per-replica dicts)."""
    import numpy as np
    import torch
    import dsa_inputs

    import dataclasses
    big = dataclasses.replace(cfg, seq_lens=list(cfg.seq_lens) * R, batch=cfg.batch * R)
    t = dsa_inputs.make_inputs_torch(big, dev)
    reps = []
    B = cfg.batch
    for r in range(R):
        sl = slice(r * B, (r + 1) * B)
        reps.append(dict(seq_lens=t["seq_lens"][sl].contiguous(), page_table=t["page_table"][sl].contiguous(),
                         q_idx=t["q_idx"][sl].contiguous(), w=t["w"][sl].contiguous(),
                         q_mla=t["q_mla"][sl].contiguous(), k_cache=t["k_cache"], k_scale=t["k_scale"],
                         kv_cache=t["kv_cache"], kv_scale=t["kv_scale"]))
    return big, t, reps


def time_graph(fn_list, stream, reps=1):
    """Capture the launches of fn_list (called in order) into one graph; return ms of one replay
    measured with HIP events recorded on `stream` (the stream the kernels run on)."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for f in fn_list:
            f()
    with torch.cuda.stream(stream):          # replay() launches on the current stream
        g.replay()
    torch.cuda.synchronize()
    best = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        best.append(e0.elapsed_time(e1))
    return g, sorted(best)[len(best) // 2]


def cpu_baseline(cfg_name, seconds):
    """Time the fp64 oracle (as it stands) on a bounded sample of the workload on this host."""
    import numpy as np
    import dsa_inputs
    from oracle import dsa_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count()
    cfg = dsa_inputs.base_config(cfg_name)
    # bounded sample: whole sequences for decode shapes, a block of query rows for the prefill shape
    if cfg_name == "c4":
        sample = dsa_inputs.scaled_config("c4", cfg.seq_lens, seed=cfg.seed, q_per_seq=cfg.q_per_seq)
        sample_desc = "last 16 query rows of the 4096-token chunk (69617-69632 visible tokens each)"
        rows = 16
    else:
        rows = None
        nseq = 1 if cfg.batch > 1 else cfg.batch
        sample = dsa_inputs.scaled_config(cfg_name, cfg.seq_lens[:nseq], seed=cfg.seed)
        sample_desc = f"{nseq} of {cfg.batch} sequence(s), full step"
    inp = dsa_inputs.make_inputs(sample)
    if rows is not None:
        inp["q_idx"] = inp["q_idx"][:, -rows:]
        inp["w"] = inp["w"][:, -rows:]
        inp["q_mla"] = inp["q_mla"][:, -rows:]
        sample.q_per_seq = rows       # the last rows see the longest contexts
    reps, total = 0, 0.0
    while total < seconds or reps == 0:
        t0 = time.perf_counter()
        O.decode_step(inp, sample)
        total += time.perf_counter() - t0
        reps += 1
        if reps >= 1000:
            break
    per = total / reps
    by = step_bytes(sample, sample.seq_lens)["total"]
    return dict(value=round(by / per / 1e9, 4), unit="GB/s", cores=cores, kind="oracle",
                sample=f"{sample_desc}; {reps} run(s), {per * 1e3:.1f} ms each",
                ms_per_sample=round(per * 1e3, 2))


def kernel_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_attention_10_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(cfg_name, kernel):
    """HBM traffic per launch from committed rocprofv3 counter summaries, if they were taken on
    the current kernel sources (profiles/traffic_<config>.json); else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{cfg_name}.json")
    try:
        with open(path) as fh:
            d = json.load(fh)
    except OSError:
        return None
    if d.get("kernel_source_hash") != kernel_hash():
        return None
    ks = d.get("kernels", {})
    # a kernel with several template instances in the run is listed once per instance
    hits = [v for n, v in ks.items() if n == kernel or n.startswith(kernel + "<")]
    return hits[0].get("bytes_per_launch") if len(hits) == 1 else None


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def copy_calibration():
    """10 device-to-device copies of 1 GiB: under rocprofv3 --pmc FETCH_SIZE (WRITE_SIZE) each
    copy dispatch should read (write) 1 GiB = 1048576 KiB; the ratio scales the counters."""
    import torch
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_dispatch": src.numel() * 4, "dispatches": 10}))


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (got --gpus {args.gpus}): the path is single-GPU, "
              "see the sharding notes in DESIGN.md", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import dsa_inputs
    import sparse_attention_10_amd as dsa

    dev = "cuda:0"
    torch.cuda.set_device(0)
    dsa.lib()
    cfg = dsa_inputs.base_config(args.config)
    lens = cfg.seq_lens
    by = step_bytes(cfg, lens)
    R = args.rotate or max(1, min(64, math.ceil(2 * MALL_BYTES / max(1, by["total"]))))
    log(f"config {cfg.name}: generating inputs ({R} replicas)")
    big, pool, reps = build_replicas(cfg, R, dev)
    B, Q, H, k = cfg.batch, cfg.q_per_seq, cfg.mla_heads, cfg.top_k
    stream = torch.cuda.Stream()

    out = torch.empty((B, Q, H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Q, H), dtype=torch.float32, device=dev)
    step_args = []
    for r in reps:
        batch = dsa.make_batch(r["seq_lens"], r["page_table"], Q, cfg.page_size, cfg.max_seq_len, big.num_slots)
        step_args.append(dsa.decode_step_args(batch, r["q_idx"], r["w"], r["k_cache"], r["k_scale"], k,
                                               r["q_mla"], r["kv_cache"], r["kv_scale"], cfg.sm_scale, out, lse,
                                               n_split=args.n_split))
    ws_bytes = max(dsa.decode_step_workspace_bytes(a) for a in step_args)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    lib = dsa.lib()
    import ctypes
    sptr = stream.cuda_stream

    def step(j):
        st = lib.dsa_decode_step(ctypes.byref(step_args[j % R]), ws.data_ptr(), ws_bytes, sptr)
        if st != 0:
            raise RuntimeError(lib.dsa_last_error().decode())

    log("warmup")
    # --- warmup (eager) ---
    with torch.cuda.stream(stream):
        for j in range(args.warmup):
            step(j)
    torch.cuda.synchronize()

    # realised union of selected rows per sequence (speculative-verify rows share a cache)
    union = None
    if Q > 1 and cfg.q_per_seq <= 8:
        idx = torch.empty((B, Q, k), dtype=torch.int32, device=dev)
        a0 = step_args[0]
        dbg = dsa.decode_step_args(a0._keep[0], reps[0]["q_idx"], reps[0]["w"], reps[0]["k_cache"],
                                   reps[0]["k_scale"], k, reps[0]["q_mla"], reps[0]["kv_cache"],
                                   reps[0]["kv_scale"], cfg.sm_scale, out, lse, debug_idx=idx)
        dsa.dsa_decode_step(dbg, torch.zeros(dsa.decode_step_workspace_bytes(dbg), dtype=torch.uint8, device=dev),
                            stream=stream)
        torch.cuda.synchronize()
        ii = idx.cpu().numpy()
        union = int(sum(len(set(ii[b].ravel().tolist()) - {-1}) for b in range(B)))
        by = step_bytes(cfg, lens, union)

    log(f"timing {args.steps} steps")
    # --- timed: K steps ---
    K = args.steps
    if args.eager:
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            for j in range(K):
                step(j)
            e1.record(stream)
        torch.cuda.synchronize()
        ms_total = e0.elapsed_time(e1)
        eager_ms = ms_total / K
    else:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for j in range(K):
                step(j)
        with torch.cuda.stream(stream):  # replay() launches on the current stream
            g.replay()                   # untimed: first replay uploads the graph
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        ms_total = e0.elapsed_time(e1)
        del g
        # eager rate for reference (a shorter run)
        ke = min(K, 200)
        torch.cuda.synchronize()
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            f0.record(stream)
            for j in range(ke):
                step(j)
            f1.record(stream)
        torch.cuda.synchronize()
        eager_ms = f0.elapsed_time(f1) / ke
    ms_step = ms_total / K

    log("per-stage timing")
    # --- per-stage timing: each stage alone, K launches cycling the replicas, one graph ---
    stage = {}
    rows = B * Q
    ld = cfg.max_seq_len
    scores = torch.empty((B, Q, ld), dtype=torch.float32, device=dev)
    idx_t = torch.empty((B, Q, k), dtype=torch.int32, device=dev)
    slots_t = torch.empty((B, Q, k), dtype=torch.int32, device=dev)
    batches = [a._keep[0] for a in step_args]
    topk_ws = torch.zeros(max(1, max(dsa.topk_workspace_bytes(bt, k) for bt in batches)), dtype=torch.uint8,
                          device=dev)
    # fill scores / slots once so the isolated stages see realistic data
    with torch.cuda.stream(stream):
        dsa.dsa_indexer_scores(batches[0], reps[0]["q_idx"], reps[0]["w"], reps[0]["k_cache"], reps[0]["k_scale"],
                               scores, stream=stream)
        dsa.dsa_topk(batches[0], scores, k, idx_t, slots_t, workspace=topk_ws, stream=stream)
    torch.cuda.synchronize()
    kvd = dsa.dtype_code(reps[0]["kv_cache"])
    ns = args.n_split or dsa.lib().dsa_sparse_mla_default_split(B, Q, H, k, kvd)
    mla_ws_bytes = dsa.mla_workspace_bytes(B, Q, H, k, ns, dsa.dtype_code(reps[0]["q_mla"]), kvd)
    mla_ws = torch.empty(max(1, mla_ws_bytes), dtype=torch.uint8, device=dev)
    KS = max(20, min(K, 1000))
    # slots per replica (so the MLA stage alone gathers rows of the replica's own pages)
    rep_slots = []
    for r in range(R):
        sl = torch.empty_like(slots_t)
        with torch.cuda.stream(stream):
            dsa.dsa_indexer_scores(batches[r], reps[r]["q_idx"], reps[r]["w"], reps[r]["k_cache"],
                                   reps[r]["k_scale"], scores, stream=stream)
            dsa.dsa_topk(batches[r], scores, k, idx_t, sl, workspace=topk_ws, stream=stream)
        rep_slots.append(sl)
    torch.cuda.synchronize()
    fns = {
        "indexer": lambda j: dsa.dsa_indexer_scores(batches[j % R], reps[j % R]["q_idx"], reps[j % R]["w"],
                                                    reps[j % R]["k_cache"], reps[j % R]["k_scale"], scores,
                                                    stream=stream),
        "topk": lambda j: dsa.dsa_topk(batches[j % R], scores, k, idx_t, slots_t, workspace=topk_ws,
                                       stream=stream),
        "mla": lambda j: dsa.dsa_sparse_mla_decode(reps[j % R]["q_mla"], reps[j % R]["kv_cache"],
                                                   reps[j % R]["kv_scale"], rep_slots[j % R], cfg.sm_scale,
                                                   out, lse, n_split=ns, workspace=mla_ws, stream=stream),
    }
    for name, f in fns.items():
        _, ms = time_graph([(lambda j=j, f=f: f(j)) for j in range(KS)], stream)
        stage[name] = ms / KS
    if ns > 1:
        part_o = mla_ws[: rows * ns * H * 512 * 4].view(torch.float32).view(rows, ns, H, 512)
        off = (rows * ns * H * 512 * 4 + 255) // 256 * 256
        mlb = (rows * ns * H * 4 + 255) // 256 * 256
        part_m = mla_ws[off: off + rows * ns * H * 4].view(torch.float32).view(rows, ns, H)
        part_l = mla_ws[off + mlb: off + mlb + rows * ns * H * 4].view(torch.float32).view(rows, ns, H)
        _, ms = time_graph([(lambda: dsa.dsa_mla_combine(part_o, part_m, part_l, out, lse, stream=stream))
                            for _ in range(KS)], stream)
        stage["combine"] = ms / KS
        stage["mla"] -= stage["combine"]        # the MLA stage timing above includes its merge
    # the write before the path (not part of the timed step): the step's B*Q new tokens go
    # into both caches of each replica, bf16 rows into the workload's cache dtype
    kv_new = (torch.randn((B, Q, 576), device=dev) / 24).to(torch.bfloat16)
    k_new = (torch.randn((B, Q, cfg.idx_dim), device=dev) / math.sqrt(cfg.idx_dim)).to(torch.bfloat16)
    _, ms = time_graph([(lambda j=j: dsa.dsa_kv_cache_append(
        batches[j % R], kv_new, reps[j % R]["kv_cache"], reps[j % R]["kv_scale"], k_new, reps[j % R]["k_cache"],
        reps[j % R]["k_scale"], stream=stream)) for j in range(KS)], stream)
    esz = {"f32": 4, "bf16": 2, "fp8": 1}
    per_tok = (576 + cfg.idx_dim) * 2 + 576 * esz[cfg.kv_dtype] + cfg.idx_dim * esz[cfg.key_dtype] + \
        4 * (cfg.kv_dtype == "fp8") + 4 * (cfg.key_dtype == "fp8") + 4
    append_info = dict(us=round(ms / KS * 1e3, 3), bytes=rows * per_tok + B * 4,
                       kernel="cache_append_kernel", timing="hip-graph of launches, replicas cycled")
    append_info["GBps"] = round(append_info["bytes"] / (append_info["us"] * 1e-6) / 1e9, 1)
    fl = step_flops(cfg, lens)
    stage_info = {
        "indexer": dict(us=stage["indexer"] * 1e3, bytes=by["indexer"], flops=fl["indexer"]),
        # top-k reads each visible score once and writes k indices and k slots per row
        "topk": dict(us=stage["topk"] * 1e3,
                     bytes=sum(sum(L - Q + i + 1 for i in range(Q)) for L in lens) * 4 + rows * k * 8),
        "mla": dict(us=stage["mla"] * 1e3, bytes=by["mla"], flops=fl["mla"]),
    }
    if "combine" in stage:
        stage_info["combine"] = dict(us=stage["combine"] * 1e3, bytes=2 * rows * ns * H * 513 * 4)
    for v in stage_info.values():
        v["GBps"] = round(v["bytes"] / (v["us"] * 1e-6) / 1e9, 1)
        v["us"] = round(v["us"], 3)
    # the dominant kernel: the stage with the largest average launch time
    dom = max(stage_info, key=lambda s: stage_info[s]["us"])
    # split chunks of at most 1024 (fp8 rows) or 2048 (bf16 rows) selected rows run on the
    # direct-to-LDS ring kernels
    chunk = -(-(-(-k // ns)) // 32) * 32
    if cfg.kv_dtype == "fp8":
        mla_kern = "mla_fp8x_kernel" if chunk <= 1024 else "mla_fp8_kernel"
    else:
        mla_kern = "mla_bf16d_kernel" if chunk <= 2048 else "mla_mfma_kernel"
    # many rows per sequence with bf16 keys run on the prefill indexer (16 rows per workgroup)
    idx_kern = ("indexer_prefill_kernel" if Q >= 16 and cfg.key_dtype == "bf16" and cfg.page_size % 32 == 0
                else "indexer_mfma_kernel")
    kern = {"indexer": idx_kern, "mla": mla_kern, "topk": "topk_kernel",
            "combine": "mla_combine_few_kernel" if ns <= 4 and H % 2 == 0 else "mla_combine_kernel"}[dom]
    if cfg.name == "c4" and dom in ("indexer", "mla"):
        ach = stage_info[dom]["flops"] / (stage_info[dom]["us"] * 1e-6) / 1e12
        roof = dict(bound="mfma", achieved=round(ach, 2), peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(ach / BF16_PEAK_TFLOPS, 4))
    else:
        ach = stage_info[dom]["GBps"]
        roof = dict(bound="hbm", achieved=ach, peak=HBM_PEAK_GBS, unit="GB/s", frac=round(ach / HBM_PEAK_GBS, 4))
    roof["kernel"] = kern
    roof["traffic"] = load_traffic(cfg.name, kern)

    gbs = by["total"] / (ms_step * 1e-3) / 1e9
    res = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32" if cfg.q_mla_dtype == "f32" else "bf16",
        "storage_dtype": {"f32": "f32", "bf16": "bf16", "fp8": "fp8_e4m3fn"}[cfg.kv_dtype],
        "data": "synthetic (seeded, device-generated; pages rotated over %d replicas)" % R,
        "config": {"workload": {"c1": "tiny fp32 decode, 4K ctx", "c2": "single-stream decode layer, 32K ctx",
                                "c2_128k": "single-stream decode layer, 128K ctx",
                                "c3": "batch-32 ragged decode, 4K-128K ctx",
                                "c4": "4096-token chunked prefill over 64K ctx",
                                "c5": "fp8 decode, batch 64 x 2 verify rows, 64K ctx"}[cfg.name],
                   "name": cfg.name, "batch": B, "q_per_seq": Q, "context": (lens[0] if len(set(lens)) == 1
                                                                             else [min(lens), max(lens)]),
                   "idx_heads": cfg.idx_heads, "idx_dim": cfg.idx_dim, "top_k": k, "mla_heads": H,
                   "kv_dtype": cfg.kv_dtype, "n_split": ns},
        "us_per_layer": round(ms_step * 1e3, 3),
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "eager_us_per_layer": round(eager_ms * 1e3, 3),
        "algorithmic_bytes_per_step": by["total"],
        "timing": "hip-graph replay" if not args.eager else "eager",
        "stages": stage_info,
        "roofline": roof,
        "outside_step": {"kv_cache_append": append_info},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (fp64 oracle)")
        res["cpu_baseline"] = cpu_baseline(cfg.name, args.cpu_seconds)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
