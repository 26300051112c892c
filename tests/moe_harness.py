"""Shared set-up for the GPU parity tests: a library context over a seeded workload,
plus small marshalling helpers.  Inputs come from `workloads`; expected values come
from `oracle`; nothing flows from the GPU into the oracle."""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
import workloads as W


def row_rel_err(y, ref):
    """max over rows of ||y - ref||_inf / ||ref||_inf."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(y - ref).max(axis=1)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    return float((num / den).max())


def oracle_outputs(wl, layer, x_np, idx, threads=None, ffn=None):
    """Per-pair expert outputs [T,k,H] (float64) of the oracle's all-resident definition,
    with the distinct experts evaluated in parallel threads (each runs the oracle's own
    dequantisation and SwiGLU for its rows; numpy releases the GIL in both).  ffn: the
    oracle's expert function (default the plain SwiGLU; oracle.expert_ffn_mx for the MX
    prefill)."""
    ffn = ffn or oracle.expert_ffn
    x64 = oracle.formats.activations_f64(x_np)
    idx = np.asarray(idx)
    T, k = idx.shape
    out = np.zeros((T, k, wl.hidden), np.float64)
    experts = sorted(set(idx.reshape(-1).tolist()))

    def one(e):
        rows = np.argwhere(idx == e)
        ys = ffn(x64[rows[:, 0]], *oracle.expert_weights_f64(wl, layer * wl.n_experts + e))
        return rows, ys

    threads = threads or min(16, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(max_workers=threads) as ex:
        for rows, ys in ex.map(one, experts):
            out[rows[:, 0], rows[:, 1]] = ys
    return out


def exact_f32(y64, grid=2.0 ** -16):
    """The exact value of an oracle result on the exact-arithmetic inputs, as fp32.

    Those inputs make every result of the method a multiple of 2^-6 (gate projections
    multiples of 32, up projections of 2^-4, down weights of 2^-5, gates at least 2^-2)
    and an fp32 number.  The oracle's fp64 value differs from it only by the fp64
    rounding of silu(g) = g / (1 + e^-g) at g >= 32 (a relative 2^-46 of each term,
    visible where terms cancel), so it is rounded to the grid; the premise is asserted:
    the fp64 value lies within fp64 noise of a grid point, and that point is an fp32
    number."""
    y64 = np.asarray(y64, np.float64)
    yg = np.round(y64 / grid) * grid
    assert np.all(np.abs(y64 - yg) <= 1e-3 * grid), "exact-input premise broken: the oracle result is off the grid"
    y32 = yg.astype(np.float32)
    assert np.array_equal(y32.astype(np.float64), yg), "exact-input premise broken: not an fp32 number"
    return y32


def tol_for(wl) -> float:
    return 1e-5 if wl.wfmt == W.WFMT_F32 else 2e-2


def dev_act(wl, x_np):
    """Workload activations (fp32 array or bf16 bit patterns) -> device tensor of the same bytes."""
    if x_np.dtype == np.uint16:
        return torch.from_numpy(x_np.view(np.int16).copy()).cuda()
    return torch.from_numpy(np.ascontiguousarray(x_np, np.float32)).cuda()


class Harness:
    """Context + pool + router + arena for one workload."""

    def __init__(self, wl, mode, n_slots=None, max_tokens=8, bw=(0, 0), flags=0, cpu_threads=0):
        import routed_expert_ffn_02_amd as R
        self.R = R
        self.wl = wl
        L, E = wl.n_layers, wl.n_experts
        self.cfg = R.make_config(L, E, wl.top_k, wl.hidden, wl.inter, wl.wfmt, wl.afmt, max_tokens, mode, wl.renorm,
                                 int(bw[0]), int(bw[1]), cpu_threads, flags)
        self.ctx = R.moe_create(self.cfg)
        self.S = R.moe_record_bytes(self.cfg)
        assert self.S == wl.record_bytes
        self.pool_ptr = R.moe_pool_alloc(self.ctx, wl.pool_records)
        wl.fill_pool(self.pool_ptr, 0, wl.pool_records)
        self.router = torch.from_numpy(np.stack([wl.router_weight(l) for l in range(L)])).cuda()
        if mode == R.MOE_MODE_FUSED:
            n_slots = L * E
        self.n_slots = wl.n_slots if n_slots is None else n_slots
        self.arena = torch.empty(max(self.n_slots, 1) * self.S, dtype=torch.uint8, device="cuda")
        R.moe_bind(self.ctx, self.router, self.arena, self.arena.numel(), self.n_slots)
        if mode == R.MOE_MODE_FUSED:
            R.moe_fused_load(self.ctx)
        torch.cuda.synchronize()

    # --- one decode layer step with caller-provided routing -------------------
    def lookup(self, layer, idx_np, trace=True):
        R = self.R
        T, k = idx_np.shape
        idx = torch.from_numpy(np.ascontiguousarray(idx_np, np.int32)).cuda()
        slot = torch.empty((T, k), dtype=torch.int32, device="cuda")
        tr = torch.full((max(1, min(T * k, self.wl.n_experts)), 4), -7, dtype=torch.int32, device="cuda")
        cnt = torch.zeros(4, dtype=torch.int32, device="cuda")
        R.expert_cache_lookup(self.ctx, layer, idx, T, slot, tr if trace else None, cnt)
        return idx, slot, tr, cnt

    def decode(self, layer, x_np, idx_np, w_np):
        R = self.R
        T = idx_np.shape[0]
        idx, slot, tr, cnt = self.lookup(layer, idx_np)
        w = torch.from_numpy(np.ascontiguousarray(w_np, np.float32)).cuda()
        x = dev_act(self.wl, x_np)
        y = torch.full((T, self.wl.hidden), float("nan"), dtype=torch.float32, device="cuda")
        R.moe_ffn_decode(self.ctx, layer, x, T, idx, w, slot, y)
        torch.cuda.synchronize()
        c = cnt.cpu().numpy()
        n_u = int(c[0] + c[1] + c[2])
        trace = [tuple(int(v) for v in r) for r in tr.cpu().numpy()[:n_u]]
        return y.cpu().numpy(), slot.cpu().numpy(), trace, c

    def route(self, layer, x_np, bias_np=None):
        R = self.R
        T = x_np.shape[0]
        x = dev_act(self.wl, x_np)
        bias = None if bias_np is None else torch.from_numpy(np.ascontiguousarray(bias_np, np.float32)).cuda()
        z = torch.empty((T, self.wl.n_experts), dtype=torch.float32, device="cuda")
        idx = torch.empty((T, self.wl.top_k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, self.wl.top_k), dtype=torch.float32, device="cuda")
        R.moe_route(self.ctx, layer, x, T, bias, z, idx, w)
        torch.cuda.synchronize()
        return z.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()

    def prefill_layer(self, layer, x_np, idx_np, w_np):
        R = self.R
        T, k = idx_np.shape
        idx = torch.from_numpy(np.ascontiguousarray(idx_np, np.int32)).cuda()
        w = torch.from_numpy(np.ascontiguousarray(w_np, np.float32)).cuda()
        x = dev_act(self.wl, x_np)
        y = torch.full((T, self.wl.hidden), float("nan"), dtype=torch.float32, device="cuda")
        tr = torch.full((max(1, min(T * k, self.wl.n_experts)), 4), -7, dtype=torch.int32, device="cuda")
        cnt = torch.zeros(4, dtype=torch.int32, device="cuda")
        R.moe_ffn_prefill(self.ctx, layer, x, T, idx, w, y, tr, cnt)
        torch.cuda.synchronize()
        c = cnt.cpu().numpy()
        return y.cpu().numpy(), tr.cpu().numpy(), c

    def snapshot(self):
        return self.R.moe_cache_snapshot(self.ctx)


def oracle_tables(cache):
    """Residency tables of an oracle ExpertCache in the snapshot's form."""
    return cache.slot_of.astype(np.int32), cache.key_of.astype(np.int32), cache.stamp.astype(np.uint64), cache.counter
