#!/usr/bin/env python3
"""Benchmark of the routed-MoE layer over a bounded shared expert cache (one MI355X).

A step is one decode token through every MoE layer: router softmax/top-k, cache
lookup with LRU update, fills of misses from the pinned host pool, the SwiGLU
expert GEMVs and the rank-order combine.  Default workload: the DeepSeek-V4-Flash
shape (43 layers, 256 experts, top-6, hidden 4096, expert intermediate 2048, e2m1
weights with a bf16 scale per 32 elements, 14,155,776-byte records), batch 1, a
1695-slot (24 GB) cache, cold start, misses filled over PCIe (offload mode); the
155.8 GB pool is backed by 4500 page-locked records (key % 4500: the same record
size and access pattern, aliased contents).  Routing has temporal locality: a
per-layer Zipf(1.1) popularity bias plus a bonus for the previous token's experts
at the same layer.  The 35B-A3B shape (40 layers, top-8 of 256, hidden 2048,
intermediate 512, bf16, the 64.4 GB pool whole, 1280 slots) runs afterwards as a
secondary section with the batch-4 elastic hybrid leg.

Beside the timed decode: a prefill leg (2048 / 4096-token prompt through all layers
with full-layer double buffering), hybrid (q* split) and CPU-backend decode legs
with the per-step split balance, an all-resident decode leg, and plain HBM reads at
the kernels' transfer sizes (the practical ceiling).

Prints ONE JSON line.  `--gpus N` with N > 1 exits: the benchmark measures one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--config", default="dsv4", choices=["a3b", "dsv4", "dsv4mx"],
                    help="a3b: 35B-A3B shape, bf16; dsv4: DeepSeek-V4-Flash shape, e2m1 + bf16 scales; "
                         "dsv4mx: the same shape as MXFP4 (E8M0 scales)")
    ap.add_argument("--mode", default="offload", choices=["offload", "hybrid", "fused"])
    ap.add_argument("--host-fills", action="store_true",
                    help="issue decode fills from the host (read the step's fill list, DMA copies) "
                         "instead of the device copy kernel")
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-replayed decode leg")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-hybrid", action="store_true")
    ap.add_argument("--no-cpu-mode", action="store_true", help="skip the CPU-backend decode leg")
    ap.add_argument("--no-fused", action="store_true", help="skip the all-resident (FUSED) graph-replayed decode leg")
    ap.add_argument("--no-elastic", action="store_true",
                    help="skip the batch-4 hybrid leg with elastic cache resizes (A3B shape only)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="threads of the library's CPU branch (0: the library's default)")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=15.0)
    ap.add_argument("--repeats", type=int, default=3,
                    help="runs of the headline (graph-replayed) and hybrid decode legs; the median is reported")
    ap.add_argument("--secondary", default="a3b", choices=["a3b", "none"],
                    help="a second workload run after the first (its own context and pool), reported under "
                         "'secondary'")
    ap.add_argument("--no-hbm-probe", action="store_true", help="skip the plain HBM read legs")
    ap.add_argument("--alias-records", type=int, default=0,
                    help="back keys by key %% R records (smaller host pool; same transfer sizes)")
    ap.add_argument("--placement", action="store_true",
                    help="only replay the decode routing trace against the placement policies (miss rate vs "
                         "cache capacity) and print one JSON line of curves")
    ap.add_argument("--bank", action="store_true",
                    help="only time the expert bank file: write the first --bank-records records of the "
                         "workload's pool, then load them into a page-locked pool with parallel direct I/O")
    ap.add_argument("--bank-records", type=int, default=512)
    ap.add_argument("--bank-dir", default=None, help="directory for the bank file (default: the temp dir)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a 512 MiB device-to-device copy (calibrates the HBM byte counters)")
    return ap.parse_args()


PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, vendor figure
PEAK_BF16_TFLOPS = 2500.0   # dense bf16 / fp16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # dense fp8 MFMA (the MX prefill's fp8 x fp4 products)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


ROOT = os.path.dirname(os.path.abspath(__file__))
# sources the decode phase-1 kernel is built from; a traffic figure counts only if
# it was measured on exactly these
PHASE1_SOURCES = ("routed_expert_ffn_02_amd/csrc/decode.hip", "routed_expert_ffn_02_amd/csrc/common.hpp")


def phase1_source_sha1():
    """SHA-1 of the phase-1 sources with comments and whitespace removed (edits to
    comments leave a measurement valid; any code change invalidates it)."""
    import hashlib
    import re
    h = hashlib.sha1()
    for rel in PHASE1_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def measured_traffic(config):
    """HBM bytes per dec_phase1 launch from the committed counter summary for this config
    (FETCH_SIZE + WRITE_SIZE, calibrated on a plain copy), or None when that summary is
    missing or was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"dec_phase1_{config}_traffic.md")
    try:
        with open(path) as f:
            fields = dict(line.strip("- \n").split(": ", 1) for line in f if line.startswith("- ") and ": " in line)
        if fields.get("source_sha1") != phase1_source_sha1():
            return None
        return int(fields["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def copy_probe():
    """A plain 512 MiB device copy, three times: reads and writes of known size for the
    byte counters."""
    import torch
    n = 512 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "copies": 3}), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "this benchmark measures one GPU; runs on several GPUs are not supported",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return
    if args.placement:
        placement_curves(args)
        return
    if args.bank:
        bank_load(args)
        return
    out = run_workload(args, args.config, primary=True)
    if args.secondary != "none" and args.secondary != args.config:
        sec = run_workload(args, args.secondary, primary=False)
        keep = ("value", "unit", "ms_per_step", "headline_leg", "dtype", "config", "roofline", "repeats")
        out["secondary"] = {k_: sec[k_] for k_ in keep}
        out["secondary"].update({k_: v for k_, v in sec.items() if isinstance(v, dict) and k_ not in keep})
    print(json.dumps(out), flush=True)


def median(v):
    v = sorted(v)
    return v[len(v) // 2] if len(v) % 2 else 0.5 * (v[len(v) // 2 - 1] + v[len(v) // 2])


def run_workload(args, config, primary):
    """Every leg of one workload on its own context and pool; returns the JSON fields."""
    import torch
    import routed_expert_ffn_02_amd as R
    import workloads as W

    wl = {"a3b": W.A3B_DECODE, "dsv4": W.DSV4, "dsv4mx": W.DSV4_MX}[config]
    # The DSV4-shaped pool (155.8 GB) exceeds what the host lets us page-lock; by default
    # its keys are backed by key % 4500 records (63.7 GB): same record size and access
    # pattern, aliased contents (the oracle uses the same mapping).
    alias = args.alias_records or (4500 if config != "a3b" else 0)
    if alias:
        wl = wl.with_(alias_records=alias)
    mode = {"offload": R.MOE_MODE_OFFLOAD, "hybrid": R.MOE_MODE_HYBRID, "fused": R.MOE_MODE_FUSED}[args.mode]
    L, E, k, H = wl.n_layers, wl.n_experts, wl.top_k, wl.hidden
    T = wl.tokens
    total_steps = args.warmup + args.steps
    dev = torch.device("cuda:0")
    reps = max(1, args.repeats)

    # ---------------------------------------------------------------- set-up (untimed)
    t0 = time.time()
    prompt = W.A3B_PREFILL.prefill_tokens if config == "a3b" else wl.prefill_tokens
    max_tokens = 8 if args.no_prefill else max(8, prompt)
    flags = R.MOE_FLAG_PROFILE | (0 if args.host_fills else R.MOE_FLAG_DEVICE_FILLS)
    cfg = R.make_config(L, E, k, H, wl.inter, wl.wfmt, wl.afmt, max_tokens, mode, wl.renorm,
                        cpu_threads=args.cpu_threads, flags=flags)
    ctx = R.moe_create(cfg)
    S = R.moe_record_bytes(cfg)
    pool = R.moe_pool_alloc(ctx, wl.pool_records)
    wl.fill_pool(pool, 0, wl.pool_records, threads=min(16, len(os.sched_getaffinity(0))))
    log(f"[{config}] pool: {wl.pool_records} records x {S} B = {wl.pool_records * S / 1e9:.1f} GB in "
        f"{time.time() - t0:.1f}s")
    router = torch.from_numpy(np.stack([wl.router_weight(l) for l in range(L)])).to(dev)
    n_slots = L * E if mode == R.MOE_MODE_FUSED else wl.n_slots
    arena = torch.empty(n_slots * S, dtype=torch.uint8, device=dev)
    R.moe_bind(ctx, router, arena, arena.numel(), n_slots)
    if mode == R.MOE_MODE_FUSED:
        R.moe_fused_load(ctx)
    bw_p, bw_h = R.moe_bench_bw(ctx)
    R.moe_set_bandwidths(ctx, max(bw_p, 1), max(bw_h, 1))
    log(f"[{config}] B_P = {bw_p / 1e9:.1f} GB/s, B_H = {bw_h / 1e9:.1f} GB/s")

    # activations for every (step, layer), resident in HBM before timing
    X = np.empty((total_steps, L, T, H), np.uint16)
    for s in range(total_steps):
        for l in range(L):
            X[s, l] = wl.decode_activations(s, l, T)
    Xd = torch.from_numpy(X.view(np.int16)).to(dev)
    zipf = torch.from_numpy(np.stack([wl.zipf_bias(l) for l in range(L)])).to(dev)        # [L, E]
    bias = torch.empty((L, T, E), dtype=torch.float32, device=dev)
    bonus = torch.full((L, T, k), float(wl.prev_bonus), dtype=torch.float32, device=dev)
    idx = torch.zeros((L, T, k), dtype=torch.int32, device=dev)
    idx64 = torch.zeros((L, T, k), dtype=torch.int64, device=dev)
    wts = torch.zeros((L, T, k), dtype=torch.float32, device=dev)
    slot = torch.zeros((L, T, k), dtype=torch.int32, device=dev)
    y = torch.zeros((L, T, H), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    log(f"[{config}] set-up {time.time() - t0:.1f}s")

    def step(s, xsrc=None, strm=None, c=None):
        xsrc = Xd[s] if xsrc is None else xsrc
        strm = stream if strm is None else strm
        c = ctx if c is None else c
        # the synthetic routing bias of every layer (Zipf popularity plus the bonus for
        # the previous token's experts at that layer) depends only on the previous step,
        # so it is prepared for all layers at once before the step's layers run
        bias.copy_(zipf[:, None, :].expand(L, T, E))
        if s > 0 and wl.prev_bonus:
            idx64.copy_(idx)
            bias.scatter_add_(2, idx64, bonus)
        for l in range(L):
            b = bias[l]
            x = xsrc[l]
            R.moe_decode_layer(c, l, x, T, b, idx[l], wts[l], slot[l], y[l], strm)

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    R.moe_reset_stats(ctx)
    cold_steps = min(64, args.steps)
    t1 = time.perf_counter()
    for s in range(args.warmup, total_steps):
        step(s)
        if s == args.warmup + cold_steps - 1:
            torch.cuda.synchronize()
            cold_elapsed = time.perf_counter() - t1
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t1
    st = R.moe_get_stats(ctx)
    tok_s = args.steps * T / elapsed
    lookups = max(1, st["lookups"])
    distinct = st["hits"] + st["fills"] + st["cpu_experts"]
    miss_rate = (st["fills"] + st["cpu_experts"]) / max(1, distinct)
    p1_avg_ms = st["phase1_ms"] / max(1, st["phase1_launches"])
    p2_avg_ms = st["phase2_ms"] / max(1, st["phase2_launches"])
    p1_bytes = st["phase1_bytes"] / max(1, st["phase1_launches"])
    p2_bytes = st["phase2_bytes"] / max(1, st["phase2_launches"])
    p1_gbs = p1_bytes / (p1_avg_ms * 1e-3) / 1e9 if p1_avg_ms > 0 else 0.0
    p2_gbs = p2_bytes / (p2_avg_ms * 1e-3) / 1e9 if p2_avg_ms > 0 else 0.0
    log(f"[{config}] decode: {tok_s:.1f} tok/s, miss rate {miss_rate:.3f}, phase1 {p1_avg_ms * 1e3:.1f} us "
        f"{p1_gbs:.0f} GB/s, phase2 {p2_avg_ms * 1e3:.1f} us {p2_gbs:.0f} GB/s")
    decode_detail = {
        "fill_path": "host DMA" if args.host_fills else "device copy kernel",
        "eager_tokens_per_s": round(tok_s, 2), "eager_ms_per_step": round(elapsed * 1e3 / args.steps, 3),
        "cold_first_steps": cold_steps, "cold_tokens_per_s": round(cold_steps * T / cold_elapsed, 2),
        "steady_tokens_per_s": round((args.steps - cold_steps) * T / max(1e-9, elapsed - cold_elapsed), 2)
        if args.steps > cold_steps else None,
        "miss_rate": round(miss_rate, 4), "fills": st["fills"], "cpu_experts": st["cpu_experts"],
        "fill_GBps_wall": round(st["fill_bytes"] / elapsed / 1e9, 2),
        "copy_engine_ms": round(st["copy_ms"], 2),
        "phase1_avg_us": round(p1_avg_ms * 1e3, 2), "phase1_GBps": round(p1_gbs, 1),
        "phase2_avg_us": round(p2_avg_ms * 1e3, 2), "phase2_GBps": round(p2_gbs, 1),
        "phase2_bytes_per_launch": int(p2_bytes),
        "bw_pcie_GBps": round(bw_p / 1e9, 2), "bw_host_GBps": round(bw_h / 1e9, 2), "lookups": lookups,
    }

    # ---------------------------------------------------------------- graph leg (headline)
    # The same steps from a cold cache, each step (every layer's bias, route, lookup,
    # device fills and GEMVs) replayed from one captured HIP graph; the step's
    # activations are copied into the graph's static input first.  Repeated from a cold
    # cache; the median run is the headline.
    graph = None
    if mode == R.MOE_MODE_OFFLOAD and not args.host_fills and not args.no_graph:
        runs = []
        for _ in range(reps):
            R.moe_bind(ctx, router, arena, arena.numel(), n_slots)
            Xs = torch.empty_like(Xd[0])
            for s in range(args.warmup):
                step(s)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, capture_error_mode="thread_local"):
                step(1, Xs, torch.cuda.current_stream().cuda_stream)
            R.moe_reset_stats(ctx)
            tg = time.perf_counter()
            for s in range(args.warmup, total_steps):
                Xs.copy_(Xd[s])
                g.replay()
            torch.cuda.synchronize()
            gel = time.perf_counter() - tg
            R.moe_sync(ctx, stream)
            gs = R.moe_get_stats(ctx)
            runs.append({"tokens_per_s": round(args.steps * T / gel, 2), "ms_per_step": round(gel * 1e3 / args.steps, 3),
                         "fills": gs["fills"], "lookups": gs["lookups"],
                         "miss_rate": round(gs["fills"] / max(1, gs["hits"] + gs["fills"]), 4)})
            del g
        graph = dict(sorted(runs, key=lambda r: r["tokens_per_s"])[len(runs) // 2])
        graph["runs_tokens_per_s"] = [r["tokens_per_s"] for r in runs]
        log(f"[{config}] graph: {graph}")

    # ---------------------------------------------------------------- hybrid leg
    # Same steps from a cold cache with the misses split by q* between fills and the
    # host CPU branch (B_P and B_H measured above), repeated; the first run's per-step
    # log gives the split's balance (fill-kernel time against CPU-branch time).
    hybrid = None
    qstar = None
    if mode == R.MOE_MODE_OFFLOAD and not args.no_hybrid:
        runs, logs = [], []
        R.moe_set_mode(ctx, R.MOE_MODE_HYBRID)
        for _ in range(reps):
            R.moe_bind(ctx, router, arena, arena.numel(), n_slots)
            for s in range(args.warmup):
                step(s)
            torch.cuda.synchronize()
            R.moe_reset_stats(ctx)
            th = time.perf_counter()
            for s in range(args.warmup, total_steps):
                step(s)
            torch.cuda.synchronize()
            hel = time.perf_counter() - th
            hs = R.moe_get_stats(ctx)
            logs.append(R.moe_step_log(ctx))
            runs.append({"tokens_per_s": round(args.steps * T / hel, 2), "ms_per_step": round(hel * 1e3 / args.steps, 3),
                         "fills": hs["fills"], "cpu_experts": hs["cpu_experts"],
                         "cpu_branch_ms_per_step": round(hs["cpu_ms"] / args.steps, 3),
                         "fill_path": "host DMA" if args.host_fills else "device copy kernel",
                         "fill_GBps_wall": round(hs["fill_bytes"] / hel / 1e9, 2)})
        mid = sorted(range(len(runs)), key=lambda i: runs[i]["tokens_per_s"])[len(runs) // 2]
        hybrid = dict(runs[mid])
        hybrid["runs_tokens_per_s"] = [r["tokens_per_s"] for r in runs]
        qstar = qstar_balance(logs[mid], S, bw_p, bw_h, args.steps, L)
        if not args.host_fills and not args.no_graph:
            # the same hybrid steps from a cold cache, replayed from one captured graph: fills
            # by the device copy kernel, the CPU branch on the library's branch thread
            R.moe_bind(ctx, router, arena, arena.numel(), n_slots)
            Xs = torch.empty_like(Xd[0])
            for s in range(args.warmup):
                step(s)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, capture_error_mode="thread_local"):
                step(1, Xs, torch.cuda.current_stream().cuda_stream)
            R.moe_reset_stats(ctx)
            th = time.perf_counter()
            for s in range(args.warmup, total_steps):
                Xs.copy_(Xd[s])
                g.replay()
            torch.cuda.synchronize()
            hg = time.perf_counter() - th
            R.moe_sync(ctx, stream)
            gs = R.moe_get_stats(ctx)
            del g
            hybrid["graph_tokens_per_s"] = round(args.steps * T / hg, 2)
            hybrid["graph_ms_per_step"] = round(hg * 1e3 / args.steps, 3)
            hybrid["graph_fills"] = gs["fills"]
            hybrid["graph_cpu_experts"] = gs["cpu_experts"]
            hybrid["graph_cpu_branch_ms_per_step"] = round(gs["cpu_ms"] / args.steps, 3)
        log(f"[{config}] hybrid: {hybrid}")
        log(f"[{config}] q*: {qstar}")
        R.moe_set_mode(ctx, R.MOE_MODE_OFFLOAD)

    # ---------------------------------------------------------------- CPU leg
    # Every routed expert evaluated by the library's CPU branch (the pages' cpu backend:
    # q = 0), a bounded number of steps: host-DRAM-bound tokens/s beside the GPU legs.
    cpu_mode = None
    if mode == R.MOE_MODE_OFFLOAD and not args.no_cpu_mode:
        R.moe_bind(ctx, router, arena, arena.numel(), n_slots)  # cold cache: with q = 0 nothing becomes resident
        R.moe_set_mode(ctx, R.MOE_MODE_CPU)
        n_cpu = min(args.steps, 64)
        for s in range(min(args.warmup, 2)):
            step(s)
        torch.cuda.synchronize()
        R.moe_reset_stats(ctx)
        tc = time.perf_counter()
        for s in range(n_cpu):
            step(s)
        torch.cuda.synchronize()
        cel = time.perf_counter() - tc
        cs = R.moe_get_stats(ctx)
        clog = R.moe_step_log(ctx)
        cpu_bytes = cs["cpu_experts"] * S
        cpu_mode = {"tokens_per_s": round(n_cpu * T / cel, 2), "ms_per_step": round(cel * 1e3 / n_cpu, 3),
                    "steps": n_cpu, "cpu_experts": cs["cpu_experts"],
                    "cpu_branch_ms_per_step": round(cs["cpu_ms"] / n_cpu, 3),
                    "cpu_branch_ms_per_layer_step": round(float(np.mean(clog["cpu_ms"])), 4) if len(clog) else None,
                    "host_GBps": round(cpu_bytes / (cs["cpu_ms"] * 1e-3) / 1e9, 1) if cs["cpu_ms"] > 0 else None,
                    "bw_host_GBps": round(bw_h / 1e9, 2)}
        log(f"[{config}] cpu mode: {cpu_mode}")
        R.moe_set_mode(ctx, R.MOE_MODE_OFFLOAD)

    # ---------------------------------------------------------------- prefill leg
    # The prompt through every layer: route, whole layers double-buffered from the pool,
    # the grouped GEMMs.  MXFP4 experts also run it on a second context with the MX prefill
    # (MXFP8 activations on the scaled MFMA), over the same pool; its MFMA fraction is
    # against the fp8 peak.
    def prefill_leg(c):
        Tp = max_tokens
        R.moe_reset_stats(c)
        xs = [torch.from_numpy(wl.prefill_activations(l, Tp).view(np.int16)).to(dev) for l in range(L)]
        pb = torch.from_numpy(np.stack([wl.zipf_bias(l) for l in range(L)])).to(dev)
        pidx = torch.empty((Tp, k), dtype=torch.int32, device=dev)
        pw = torch.empty((Tp, k), dtype=torch.float32, device=dev)
        py = torch.empty((Tp, H), dtype=torch.float32, device=dev)
        pbias = torch.empty((Tp, E), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        R.moe_prefill_begin(c, stream)
        for l in range(L):
            pbias.copy_(pb[l].expand(Tp, E))
            R.moe_route(c, l, xs[l], Tp, pbias, None, pidx, pw, stream)
            R.moe_ffn_prefill(c, l, xs[l], Tp, pidx, pw, py, None, None, stream)
        R.moe_prefill_end(c, stream)
        torch.cuda.synchronize()
        pel = time.perf_counter() - t2
        ps = R.moe_get_stats(c)
        gemm_ms = ps["gemm1_ms"] + ps["gemm2_ms"]
        tflops = ps["gemm_flops"] / (gemm_ms * 1e-3) / 1e12 if gemm_ms > 0 else 0.0
        return {
            "tokens": Tp, "tokens_per_s": round(Tp / pel, 1), "wall_s": round(pel, 3),
            "copy_GBps": round(ps["copy_bytes"] / (ps["copy_ms"] * 1e-3) / 1e9, 2) if ps["copy_ms"] > 0 else None,
            "copy_bytes": ps["copy_bytes"], "copy_ms_per_layer": round(ps["copy_ms"] / L, 3),
            "gemm_ms_per_layer": round(gemm_ms / L, 3),
            "gemm1_ms_per_layer": round(ps["gemm1_ms"] / L, 3), "gemm2_ms_per_layer": round(ps["gemm2_ms"] / L, 3),
            "gemm_TFLOPs": round(tflops, 1),
            "gemm_weight_GBps": round(E * S / (gemm_ms / L * 1e-3) / 1e9, 1) if gemm_ms > 0 else None,
            # every record of the layer is read once per layer: below 2.5 PFLOP/s / 8 TB/s =
            # 312 flop per byte the GEMMs are bound by HBM, and this is their roofline fraction
            "gemm_flop_per_byte": round(ps["gemm_flops"] / L / (E * S), 1) if gemm_ms > 0 else None,
            "hbm_frac": round(E * S / (gemm_ms / L * 1e-3) / 1e9 / PEAK_HBM_GBS, 4) if gemm_ms > 0 else None,
            "overlap": round(max(0.0, (ps["copy_ms"] + gemm_ms - pel * 1e3) / max(1e-9, min(ps["copy_ms"], gemm_ms))), 3),
        }

    prefill = None
    prefill_mx = None
    if not args.no_prefill and mode != R.MOE_MODE_FUSED:
        prefill = prefill_leg(ctx)
        prefill["mfma_frac"] = round(prefill["gemm_TFLOPs"] / PEAK_BF16_TFLOPS, 4)
        log(f"[{config}] prefill: {prefill}")
        if wl.wfmt == W.WFMT_MXFP4:
            cfg_m = R.make_config(L, E, k, H, wl.inter, wl.wfmt, wl.afmt, max_tokens, mode, wl.renorm,
                                  cpu_threads=args.cpu_threads, flags=R.MOE_FLAG_PROFILE | R.MOE_FLAG_MX_PREFILL)
            ctx_m = R.moe_create(cfg_m)
            R.moe_pool_register(ctx_m, pool, wl.pool_records, 1)
            arena_m = torch.empty((2 * E + 1) * S, dtype=torch.uint8, device=dev)
            R.moe_bind(ctx_m, router, arena_m, arena_m.numel(), 2 * E + 1)
            prefill_mx = prefill_leg(ctx_m)
            prefill_mx["activations"] = "MXFP8 (E4M3, E8M0 per 32)"
            prefill_mx["mfma_frac_fp8_peak"] = round(prefill_mx["gemm_TFLOPs"] / PEAK_FP8_TFLOPS, 4)
            log(f"[{config}] prefill (MX): {prefill_mx}")
            R.moe_destroy(ctx_m)
            del arena_m
            torch.cuda.empty_cache()

    # ---------------------------------------------------------------- elastic leg
    # The batch-4 hybrid run of the elastic configuration on the same pool: four
    # sequences, each with its own previous-token bonus, misses split by q* (B_P, B_H
    # measured above), the cache resized 1280 -> 640 -> 960 slots at safe points a third
    # and two thirds into the run without reloading the host pool.
    elastic = None
    if mode == R.MOE_MODE_OFFLOAD and config == "a3b" and not args.no_elastic:
        elastic = elastic_leg(args, R, W, ctx, router, arena, n_slots, zipf, stream, dev)
        log(f"[{config}] elastic: {elastic}")

    # ---------------------------------------------------------------- HBM ceiling legs
    # Plain streaming reads of the sizes the kernels move per launch (phase 1, phase 2 of
    # a decode step, one prefill layer's records), from a region of the arena not read in
    # the previous passes (no cache reuse): the practical HBM read rate each kernel is
    # measured against beside the vendor peak.
    hbm = None
    if not args.no_hbm_probe and mode == R.MOE_MODE_OFFLOAD:
        hbm = {}
        sizes = {"phase1": int(p1_bytes), "phase2": int(p2_bytes), "prefill_layer": int(E * S)}
        for name, nb in sizes.items():
            nb = min(nb, arena.numel() // 2)
            if nb < (1 << 20):
                continue
            secs = R.moe_bench_hbm(arena, arena.numel(), nb, 40 if nb < (1 << 30) else 6, stream)[1:]
            hbm[name] = {"bytes": nb, "median_us": round(median(list(secs)) * 1e6, 2),
                         "median_GBps": round(nb / median(list(secs)) / 1e9, 1),
                         "best_GBps": round(nb / float(np.min(secs)) / 1e9, 1)}
        log(f"[{config}] hbm reads: {hbm}")

    # ---------------------------------------------------------------- fused leg
    # Every record resident (a second context over the same page-locked pool): the
    # all-hit decode step, captured once and replayed per token, against the whole
    # step's algorithmic HBM bytes (each routed expert's record, the router weights,
    # x and y of every layer).
    fused = None
    if mode == R.MOE_MODE_OFFLOAD and not args.no_fused and not args.no_graph:
        del arena
        torch.cuda.empty_cache()
        cfg_f = R.make_config(L, E, k, H, wl.inter, wl.wfmt, wl.afmt, 8, R.MOE_MODE_FUSED, wl.renorm,
                              flags=R.MOE_FLAG_PROFILE)
        ctx_f = R.moe_create(cfg_f)
        R.moe_pool_register(ctx_f, pool, wl.pool_records, 1)
        arena_f = torch.empty(L * E * S, dtype=torch.uint8, device=dev)
        R.moe_bind(ctx_f, router, arena_f, arena_f.numel(), L * E)
        R.moe_fused_load(ctx_f)
        Xs = torch.empty_like(Xd[0])
        for s in range(args.warmup):
            step(s, c=ctx_f)
        torch.cuda.synchronize()
        # eager all-resident steps with per-launch events: the routed phase 1 and the fused
        # down projection + combine as the graph below runs them
        R.moe_reset_stats(ctx_f)
        for s in range(args.warmup, min(total_steps, args.warmup + 8)):
            step(s, c=ctx_f)
        torch.cuda.synchronize()
        fs = R.moe_get_stats(ctx_f)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, capture_error_mode="thread_local"):
            step(1, Xs, torch.cuda.current_stream().cuda_stream, c=ctx_f)
        tf = time.perf_counter()
        for s in range(args.warmup, total_steps):
            Xs.copy_(Xd[s])
            g.replay()
        torch.cuda.synchronize()
        fel = time.perf_counter() - tf
        del g
        step_bytes = L * (k * S + E * H * 4 + T * H * (2 + 4))
        f1 = fs["phase1_ms"] / max(1, fs["phase1_launches"])
        f2 = fs["phase2_ms"] / max(1, fs["phase2_launches"])
        fused = {"tokens_per_s": round(args.steps * T / fel, 2), "ms_per_step": round(fel * 1e3 / args.steps, 3),
                 "step_bytes": step_bytes, "step_GBps": round(step_bytes * args.steps / fel / 1e9, 1),
                 "step_hbm_frac": round(step_bytes * args.steps / fel / 1e9 / PEAK_HBM_GBS, 4),
                 "routed_phase1_avg_us": round(f1 * 1e3, 2),
                 "routed_phase1_GBps": round(fs["phase1_bytes"] / max(1, fs["phase1_launches"]) / (f1 * 1e-3) / 1e9, 1)
                 if f1 > 0 else None,
                 "phase2_combine_avg_us": round(f2 * 1e3, 2),
                 "phase2_combine_GBps": round(fs["phase2_bytes"] / max(1, fs["phase2_launches"]) / (f2 * 1e-3) / 1e9, 1)
                 if f2 > 0 else None}
        log(f"[{config}] fused: {fused}")
        R.moe_destroy(ctx_f)
        del arena_f

    # ---------------------------------------------------------------- CPU baseline (oracle)
    cpu_baseline = None
    if primary and not args.no_cpu_baseline:
        cpu_baseline = oracle_baseline(wl, args.cpu_baseline_seconds)
        log(f"[{config}] cpu baseline: {cpu_baseline}")

    # headline: the graph-replayed step when it ran (the production path), else the eager one
    head_tok_s, head_ms = (graph["tokens_per_s"], graph["ms_per_step"]) if graph else \
        (round(tok_s, 2), round(elapsed * 1e3 / args.steps, 3))
    out = {
        "metric": "routed-MoE decode tokens/s + prefill tokens/s; achieved HBM GB/s vs peak",
        "value": head_tok_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": head_ms, "higher_is_better": True, "scaling": "weak",
        "headline_leg": "graph-replayed decode step" if graph else "eager decode step",
        "repeats": reps if graph else 1,
        "vs_baseline": None,
        "dtype": {W.WFMT_BF16: "bf16", W.WFMT_FP4: "fp4(e2m1)+bf16 scale", W.WFMT_MXFP4: "mxfp4(e2m1)+e8m0 scale",
                  W.WFMT_F32: "f32"}[wl.wfmt],
        "data": "synthetic (seeded; random-init weights of the stated shape)",
        "config": {"workload": f"{wl.name}: L={L} E={E} k={k} H={H} I={wl.inter}, batch {T}, "
                               f"{n_slots}-slot shared cache, {args.mode}, cold start"
                               + (f", pool aliased to {wl.alias_records} records" if wl.alias_records else ""),
                   "pool_records": wl.pool_records, "record_bytes": S,
                   "pool_aliased": bool(wl.alias_records)},
        "roofline": {"bound": "hbm", "kernel": "dec_phase1 (gate/up GEMV + SwiGLU)",
                     "achieved": round(p1_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(p1_gbs / PEAK_HBM_GBS, 4), "traffic": measured_traffic(config),
                     "bytes_per_launch": int(p1_bytes), "avg_launch_us": round(p1_avg_ms * 1e3, 3),
                     "practical_read_GBps": hbm["phase1"]["median_GBps"] if hbm and "phase1" in hbm else None},
        "cpu_baseline": cpu_baseline,
        "decode": decode_detail,
        "graph_decode": graph,
        "hybrid_decode": hybrid,
        "qstar": qstar,
        "cpu_mode_decode": cpu_mode,
        "fused_decode": fused,
        "elastic_hybrid_batch4": elastic,
        "prefill": prefill,
        "prefill_mx": prefill_mx,
        "hbm_ceiling": hbm,
    }
    R.moe_destroy(ctx)
    del ctx
    torch.cuda.empty_cache()
    return out


def qstar_balance(rec, S, bw_p, bw_h, steps, L):
    """The q* split per layer step (the library's step log of one hybrid run): how many
    misses went to fills and to the CPU, and the two branches' measured times against
    the closed form's T_fill = q S / B_P and T_cpu = (m - q) S / B_H."""
    if rec is None or len(rec) == 0:
        return None
    m = rec["misses"]
    q = rec["fills"]
    c = rec["cpu"]
    both = (q > 0) & (c > 0)
    hist = {int(v): int(n) for v, n in zip(*np.unique(q, return_counts=True))}
    mhist = {int(v): int(n) for v, n in zip(*np.unique(m, return_counts=True))}
    tf, tc = rec["fill_ms"], rec["cpu_ms"]
    out = {"layer_steps": int(len(rec)), "with_misses": int(np.sum(m > 0)),
           "q_hist": hist, "m_hist": mhist,
           "fills": int(q.sum()), "cpu_experts": int(c.sum()),
           "fill_ms_mean": round(float(tf[q > 0].mean()), 4) if np.any(q > 0) else None,
           "cpu_ms_mean": round(float(tc[c > 0].mean()), 4) if np.any(c > 0) else None,
           "model_fill_ms_per_record": round(S / bw_p * 1e3, 4) if bw_p else None,
           "model_cpu_ms_per_record": round(S / bw_h * 1e3, 4) if bw_h else None,
           "measured_fill_ms_per_record": round(float(tf[q > 0].sum() / max(1, q[q > 0].sum())), 4)
           if np.any(q > 0) else None,
           "measured_cpu_ms_per_record": round(float(tc[c > 0].sum() / max(1, c[c > 0].sum())), 4)
           if np.any(c > 0) else None}
    if np.any(both):
        r = tf[both] / np.maximum(tc[both], 1e-9)
        out["fill_over_cpu_median"] = round(float(np.median(r)), 3)
        out["steps_fill_longer"] = int(np.sum(tf[both] > tc[both]))
        out["steps_cpu_longer"] = int(np.sum(tf[both] <= tc[both]))
    out["exposed_ms_per_step"] = round(float(np.maximum(tf, tc).sum()) / steps, 3)
    out["serial_ms_per_step"] = round(float((tf + tc).sum()) / steps, 3)
    return out


def elastic_leg(args, R, W, ctx, router, arena, n_slots, zipf, stream, dev):
    """Batch 4, hybrid q* split, resizes at a third and two thirds of 2 x --steps steps."""
    import torch
    wl = W.A3B_DECODE.with_(tokens=4)
    L, E, k, H, T = wl.n_layers, wl.n_experts, wl.top_k, wl.hidden, 4
    steps = 2 * args.steps
    sched = {steps // 3: 640, (2 * steps) // 3: 960}
    X = np.empty((steps, L, T, H), np.uint16)
    for s in range(steps):
        for l in range(L):
            X[s, l] = wl.decode_activations(s, l, T)
    Xd = torch.from_numpy(X.view(np.int16)).to(dev)
    bias = torch.empty((L, T, E), dtype=torch.float32, device=dev)
    bonus = torch.full((L, T, k), float(wl.prev_bonus), dtype=torch.float32, device=dev)
    idx = torch.zeros((L, T, k), dtype=torch.int32, device=dev)
    idx64 = torch.zeros((L, T, k), dtype=torch.int64, device=dev)
    wts = torch.zeros((L, T, k), dtype=torch.float32, device=dev)
    slot = torch.zeros((L, T, k), dtype=torch.int32, device=dev)
    y = torch.zeros((T, H), dtype=torch.float32, device=dev)
    R.moe_bind(ctx, router, arena, arena.numel(), n_slots)
    R.moe_set_mode(ctx, R.MOE_MODE_HYBRID)
    R.moe_reset_stats(ctx)
    torch.cuda.synchronize()
    resize_s = 0.0
    t0 = time.perf_counter()
    for s in range(steps):
        bias.copy_(zipf[:, None, :].expand(L, T, E))
        if s > 0:
            idx64.copy_(idx)
            bias.scatter_add_(2, idx64, bonus)
        for l in range(L):
            R.moe_route_lookup(ctx, l, Xd[s, l], T, bias[l], None, idx[l], wts[l], slot[l], None, None, stream)
            R.moe_ffn_decode(ctx, l, Xd[s, l], T, idx[l], wts[l], slot[l], y, stream)
        if s + 1 in sched:
            tr = time.perf_counter()
            R.expert_cache_resize(ctx, sched[s + 1], None, 0, stream)
            resize_s += time.perf_counter() - tr
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    st = R.moe_get_stats(ctx)
    R.moe_set_mode(ctx, R.MOE_MODE_OFFLOAD)
    distinct = st["hits"] + st["fills"] + st["cpu_experts"]
    return {"tokens_per_s": round(steps * T / el, 2), "ms_per_step": round(el * 1e3 / steps, 3), "steps": steps,
            "batch": T, "resizes": [[k_, v] for k_, v in sorted(sched.items())], "resize_ms_total": round(resize_s * 1e3, 2),
            "miss_rate": round((st["fills"] + st["cpu_experts"]) / max(1, distinct), 4), "fills": st["fills"],
            "cpu_experts": st["cpu_experts"], "cpu_branch_ms_per_step": round(st["cpu_ms"] / steps, 3),
            "fill_GBps_wall": round(st["fill_bytes"] / el / 1e9, 2)}


def placement_curves(args):
    """Decode-time expert miss rate against cache capacity for the placement policies
    the pages compare (global LRU, prefill-time placement, routing-blind static split)
    plus the calibrated pinned set with per-layer LRU rings, all replayed by the
    library's host engine on one routing trace that the library's router produces on
    the GPU: `--steps` decode tokens with the benchmark's Zipf and previous-token
    locality bias from a cold start, and the prompt routing (Zipf bias only) as the
    calibration trace.  Capacities are fractions of the whole expert pool."""
    import torch
    import routed_expert_ffn_02_amd as R
    import workloads as W

    wl = {"a3b": W.A3B_DECODE, "dsv4": W.DSV4, "dsv4mx": W.DSV4_MX}[args.config]
    L, E, k, H = wl.n_layers, wl.n_experts, wl.top_k, wl.hidden
    prompt = W.A3B_PREFILL.prefill_tokens if args.config == "a3b" else wl.prefill_tokens
    dev = torch.device("cuda:0")
    cfg = R.make_config(L, E, k, H, wl.inter, wl.wfmt, wl.afmt, prompt, R.MOE_MODE_OFFLOAD)
    ctx = R.moe_create(cfg)
    router = torch.from_numpy(np.stack([wl.router_weight(l) for l in range(L)])).to(dev)
    R.moe_bind(ctx, router, None, 0, 0)
    zipf = torch.from_numpy(np.stack([wl.zipf_bias(l) for l in range(L)])).to(dev)
    T, steps = wl.tokens, args.steps
    idx = torch.zeros((steps, L, T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    bias = torch.empty((T, E), dtype=torch.float32, device=dev)
    bonus = torch.full((T, k), float(wl.prev_bonus), dtype=torch.float32, device=dev)
    t0 = time.time()
    for s in range(steps):
        xs = torch.from_numpy(np.stack([wl.decode_activations(s, l, T) for l in range(L)]).view(np.int16)).to(dev)
        for l in range(L):
            bias.copy_(zipf[l].expand(T, E))
            if s > 0 and wl.prev_bonus:
                bias.scatter_add_(1, idx[s - 1, l].long(), bonus)
            R.moe_route(ctx, l, xs[l], T, bias, None, idx[s, l], w)
    cal = torch.empty((prompt, L, k), dtype=torch.int32, device=dev)
    pidx = torch.empty((prompt, k), dtype=torch.int32, device=dev)
    pw = torch.empty((prompt, k), dtype=torch.float32, device=dev)
    pbias = torch.empty((prompt, E), dtype=torch.float32, device=dev)
    for l in range(L):
        x = torch.from_numpy(wl.prefill_activations(l, prompt).view(np.int16)).to(dev)
        pbias.copy_(zipf[l].expand(prompt, E))
        R.moe_route(ctx, l, x, prompt, pbias, None, pidx, pw)
        cal[:, l] = pidx
    torch.cuda.synchronize()
    decode = idx.reshape(steps, L, T * k).cpu().numpy()
    calib = cal.cpu().numpy()
    log(f"routing traces: {steps} decode steps, {prompt} prompt tokens in {time.time() - t0:.1f}s")
    R.moe_destroy(ctx)

    fracs = [0.02, 0.05, 0.08, 0.11, 0.125, 0.154, 0.2, 0.25, 0.3, 0.37, 0.5, 0.75, 1.0]
    policies = [("lru", R.MOE_PLACE_LRU), ("prefill_update", R.MOE_PLACE_PREFILL),
                ("static_split", R.MOE_PLACE_STATIC), ("pinned_ring", R.MOE_PLACE_PINNED_RING)]
    curves = {name: [] for name, _ in policies}
    t1 = time.perf_counter()
    replays = 0
    for f in fracs:
        cap = int(round(f * L * E))
        for name, pol in policies:
            ring = min(k, cap // L) if pol == R.MOE_PLACE_PINNED_RING else 0
            r = R.moe_placement_replay(L, E, pol, cap, decode, calib, ring_per_layer=ring)
            curves[name].append(round(r["misses"] / max(1, r["keys"]), 4))
            replays += 1
    rel = time.perf_counter() - t1
    out = {"placement_replay": f"{wl.name}: L={L} E={E} k={k}, batch {T}, {steps} decode steps from a cold cache, "
                               f"{prompt}-token prompt as the calibration trace",
           "capacity_frac_of_pool": fracs, "capacity_slots": [int(round(f * L * E)) for f in fracs],
           "miss_rate": curves, "pinned_ring_slots_per_layer": k,
           "replay_ms_per_policy": round(rel * 1e3 / replays, 2),
           "reads_per_replay": int(decode.size)}
    print(json.dumps(out), flush=True)


def bank_load(args):
    """Engine bootstrap from an expert bank file: the first `--bank-records` records of
    the workload's pool are generated, written as a bank file, and loaded into a fresh
    context's page-locked pool by `moe_pool_load` with 1, 4 and 16 reader threads
    (O_DIRECT where the file system allows it: the page cache holds the freshly written
    file, which buffered reads would hit)."""
    import ctypes
    import shutil
    import tempfile
    import routed_expert_ffn_02_amd as R
    import workloads as W

    base = {"a3b": W.A3B_DECODE, "dsv4": W.DSV4, "dsv4mx": W.DSV4_MX}[args.config]
    n = min(args.bank_records, base.n_keys)
    wl = base.with_(alias_records=n)
    L, E = wl.n_layers, wl.n_experts
    cfg = R.make_config(L, E, wl.top_k, wl.hidden, wl.inter, wl.wfmt, wl.afmt, 1, R.MOE_MODE_OFFLOAD)
    S = R.moe_record_bytes(cfg)
    d = tempfile.mkdtemp(prefix="rmoe_bank_", dir=args.bank_dir)
    path = os.path.join(d, "experts.bank")
    try:
        src = np.empty(n * S, np.uint8)
        t0 = time.perf_counter()
        wl.fill_pool(src.ctypes.data, 0, n, threads=min(16, len(os.sched_getaffinity(0))))
        gen_s = time.perf_counter() - t0
        t0 = time.perf_counter()
        R.moe_bank_write(path, cfg, src, n)
        write_s = time.perf_counter() - t0
        loads = []
        for threads in (1, 4, 16):
            ctx = R.moe_create(cfg)
            t0 = time.perf_counter()
            ptr, st = R.moe_pool_load(ctx, path, threads)
            total_s = time.perf_counter() - t0
            view = np.ctypeslib.as_array((ctypes.c_uint8 * (n * S)).from_address(ptr))
            ok = bool(np.array_equal(view, src))
            loads.append({"threads": threads, "mode": st["mode"], "direct_errno": st["direct_errno"],
                          "read_GBps": round(st["bytes"] / st["seconds"] / 1e9, 2),
                          "alloc_plus_read_s": round(total_s, 3), "bytes_match": ok})
            R.moe_destroy(ctx)
            log(f"bank load: {loads[-1]}")
        fs = os.popen(f"df -T {d} | tail -1").read().split()
        out = {"bank": f"{wl.name}: {n} records of {S} B ({n * S / 1e9:.2f} GB)",
               "file_system": fs[1] if len(fs) > 1 else "?",
               "generate_GBps": round(n * S / gen_s / 1e9, 2), "write_GBps": round(n * S / write_s / 1e9, 2),
               "loads": loads}
        print(json.dumps(out), flush=True)
    finally:
        shutil.rmtree(d, ignore_errors=True)


def oracle_baseline(wl, seconds):
    """The oracle (as it stands) timed on the host cores over the first decode steps of the same workload."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    orc = oracle.OracleMoE(wl, mode=oracle.MODE_OFFLOAD, weight_cache=False)
    T = wl.tokens
    prev = {}
    t0 = time.perf_counter()
    layers = 0
    while layers < 2 or time.perf_counter() - t0 < seconds:
        s, l = divmod(layers, wl.n_layers)
        x = wl.decode_activations(s, l, T)
        r = orc.decode_layer(l, x, orc.decode_bias(l, prev.get(l), T))
        prev[l] = r["idx"]
        layers += 1
    el = time.perf_counter() - t0
    return {"value": round(layers / wl.n_layers * T / el, 5), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {layers} decode layer steps ({layers / wl.n_layers:.2f} tokens) of {wl.name}, "
                      f"fp64 NumPy, routing + cache + expert FFN"}


if __name__ == "__main__":
    main()
