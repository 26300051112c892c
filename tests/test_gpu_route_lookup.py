"""GPU: moe_route_lookup (router GEMV, then the cache-control kernel taking the top k
from the logits itself) equals moe_route followed by expert_cache_lookup bit for bit:
indices, gates, logits, slot ids, traces, counts and the decode output that follows."""
import numpy as np
import pytest
import torch

import workloads as W
from moe_harness import Harness, dev_act

pytestmark = pytest.mark.gpu

BF16 = W.A3B_DECODE.with_(name="rl_bf16", n_layers=2, n_experts=32, top_k=4, hidden=256, inter=128)
MX = W.DSV4_MX.with_(name="rl_mx", n_layers=2, n_experts=16, top_k=3, hidden=512, inter=256)
# 8 tokens x top-10 = 80 pairs: beyond the one-wavefront lookup, so the top-k kernel runs
K10 = W.A3B_DECODE.with_(name="rl_k10", n_layers=2, n_experts=32, top_k=10, hidden=256, inter=128)


def _run(h, fused_call, layer, x_np, bias, T):
    R = h.R
    wl = h.wl
    k, E = wl.top_k, wl.n_experts
    x = dev_act(wl, x_np)
    idx = torch.full((T, k), -5, dtype=torch.int32, device="cuda")
    w = torch.full((T, k), -1.0, dtype=torch.float32, device="cuda")
    z = torch.full((T, E), -1.0, dtype=torch.float32, device="cuda")
    slot = torch.full((T, k), -9, dtype=torch.int32, device="cuda")
    tr = torch.full((min(T * k, E), 4), -7, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(4, dtype=torch.int32, device="cuda")
    if fused_call:
        R.moe_route_lookup(h.ctx, layer, x, T, bias, z, idx, w, slot, tr, cnt)
    else:
        R.moe_route(h.ctx, layer, x, T, bias, z, idx, w)
        R.expert_cache_lookup(h.ctx, layer, idx, T, slot, tr, cnt)
    y = torch.full((T, wl.hidden), float("nan"), dtype=torch.float32, device="cuda")
    R.moe_ffn_decode(h.ctx, layer, x, T, idx, w, slot, y)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (idx, w, z, slot, tr, cnt, y)]


@pytest.mark.parametrize("wl,T", [(BF16, 1), (BF16, 4), (MX, 1), (MX, 8), (K10, 8)],
                         ids=["bf16-1", "bf16-4", "mxfp4-1", "mxfp4-8", "k10-8-fallback"])
@pytest.mark.parametrize("mode", [0, 1, 3])
def test_route_lookup_equals_route_then_lookup(wl, mode, T):
    n_slots = max(2 * wl.top_k * T, wl.n_keys // 3)
    bw = (25_000_000_000, 100_000_000_000)
    a = Harness(wl, mode, n_slots=n_slots, max_tokens=T, bw=bw)
    b = Harness(wl, mode, n_slots=n_slots, max_tokens=T, bw=bw)
    for step in range(5):
        for layer in range(wl.n_layers):
            x_np = wl.decode_activations(step, layer, T)
            bias = torch.from_numpy(np.tile(wl.zipf_bias(layer), (T, 1)).astype(np.float32)).cuda()
            ra = _run(a, True, layer, x_np, bias, T)
            rb = _run(b, False, layer, x_np, bias, T)
            for name, u, v in zip(("idx", "w", "logits", "slot", "trace", "counts", "y"), ra, rb):
                assert np.array_equal(u.view(np.uint32) if u.dtype == np.float32 else u,
                                      v.view(np.uint32) if v.dtype == np.float32 else v), (name, step, layer)


FUSED_WL = {"bf16": W.A3B_DECODE.with_(name="dl_bf16", n_layers=2, n_experts=16, top_k=8, hidden=2048, inter=512),
            "fp4": W.DSV4.with_(name="dl_fp4", n_layers=2, n_experts=16, top_k=6, hidden=4096, inter=512),
            "mxfp4": W.DSV4_MX.with_(name="dl_mx", n_layers=2, n_experts=16, top_k=6, hidden=4096, inter=512),
            "fp32": W.TINY.with_(n_layers=2)}


@pytest.mark.parametrize("fmt", list(FUSED_WL))
@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("T", [1, 2])
def test_decode_layer_equals_the_two_calls(fmt, mode, T):
    """moe_decode_layer (all-resident batch 1: phase 1 routes itself) against
    moe_route_lookup + moe_ffn_decode: indices, gates, slot ids and y bit for bit."""
    import routed_expert_ffn_02_amd as R
    wl = FUSED_WL[fmt]
    n_slots = wl.n_keys if mode == 1 else None
    a = Harness(wl, mode, n_slots=n_slots, max_tokens=T)
    b = Harness(wl, mode, n_slots=n_slots, max_tokens=T)
    k, E, H = wl.top_k, wl.n_experts, wl.hidden
    for step in range(4):
        for layer in range(wl.n_layers):
            x = dev_act(wl, wl.decode_activations(step, layer, T))
            bias = torch.from_numpy(np.tile(wl.zipf_bias(layer), (T, 1)).astype(np.float32)).cuda()
            outs = []
            for h, one in ((a, True), (b, False)):
                idx = torch.full((T, k), -5, dtype=torch.int32, device="cuda")
                w = torch.full((T, k), -1.0, dtype=torch.float32, device="cuda")
                slot = torch.full((T, k), -9, dtype=torch.int32, device="cuda")
                y = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
                if one:
                    R.moe_decode_layer(h.ctx, layer, x, T, bias, idx, w, slot, y)
                else:
                    R.moe_route_lookup(h.ctx, layer, x, T, bias, None, idx, w, slot)
                    R.moe_ffn_decode(h.ctx, layer, x, T, idx, w, slot, y)
                torch.cuda.synchronize()
                outs.append([t.cpu().numpy() for t in (idx, w.view(torch.int32), slot, y.view(torch.int32))])
            for name, u, v in zip(("idx", "w", "slot", "y"), *outs):
                assert np.array_equal(u, v), (name, step, layer)


@pytest.mark.parametrize("fmt", ["bf16", "fp4", "mxfp4"])
def test_fused_phase2_combine_equals_separate_kernels(fmt):
    """Batch 1 with no CPU branch possible (offload) takes phase 2 and the combine in one
    kernel; hybrid mode with B_H <= B_P fills every miss too but keeps the separate
    kernels.  Same routing, same fills: y must agree bit for bit."""
    import routed_expert_ffn_02_amd as R
    wl = FUSED_WL[fmt]
    n_slots = wl.n_keys // 2
    a = Harness(wl, R.MOE_MODE_OFFLOAD, n_slots=n_slots, max_tokens=1)
    b = Harness(wl, R.MOE_MODE_HYBRID, n_slots=n_slots, max_tokens=1, bw=(100, 50))
    k, H = wl.top_k, wl.hidden
    for step in range(5):
        for layer in range(wl.n_layers):
            x = dev_act(wl, wl.decode_activations(step, layer, 1))
            bias = torch.from_numpy(wl.zipf_bias(layer)[None, :].astype(np.float32)).cuda()
            ys = []
            for h in (a, b):
                idx = torch.empty((1, k), dtype=torch.int32, device="cuda")
                w = torch.empty((1, k), dtype=torch.float32, device="cuda")
                slot = torch.empty((1, k), dtype=torch.int32, device="cuda")
                cnt = torch.zeros(4, dtype=torch.int32, device="cuda")
                y = torch.full((1, H), float("nan"), dtype=torch.float32, device="cuda")
                R.moe_route_lookup(h.ctx, layer, x, 1, bias, None, idx, w, slot, None, cnt)
                R.moe_ffn_decode(h.ctx, layer, x, 1, idx, w, slot, y)
                torch.cuda.synchronize()
                assert int(cnt[2]) == 0          # nothing ran on the CPU
                ys.append(y.view(torch.int32).cpu().numpy())
            assert np.array_equal(ys[0], ys[1]), (step, layer)
