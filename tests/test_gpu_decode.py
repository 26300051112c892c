"""GPU parity: the decode path (lookup -> fills / CPU branch -> GEMV phases -> combine)
against the oracle's all-resident output and cache traces, per mode and format."""
import numpy as np
import pytest

import oracle
import workloads as W
from moe_harness import Harness, row_rel_err, tol_for

pytestmark = pytest.mark.gpu

BF16 = W.A3B_DECODE.with_(name="dec_bf16", n_layers=2, n_experts=16, top_k=4, hidden=256, inter=128)
FP4 = W.DSV4.with_(name="dec_fp4", n_layers=2, n_experts=16, top_k=3, hidden=256, inter=128)
MX = W.DSV4_MX.with_(name="dec_mxfp4", n_layers=2, n_experts=16, top_k=3, hidden=256, inter=256)
FMT = {"fp32": W.TINY, "bf16": BF16, "fp4": FP4, "mxfp4": MX}


def _gates(wl, step, layer, T):
    u = wl.uniforms(1000 + step * 64 + layer, T * wl.top_k).reshape(T, wl.top_k) + 0.05
    return (u / u.sum(axis=1, keepdims=True)).astype(np.float32)


def _expected(wl, layer, x, idx, w):
    x64 = oracle.formats.activations_f64(x)
    outs = oracle.moe_layer_dense(x64, idx, lambda e: oracle.expert_weights_f64(wl, layer * wl.n_experts + e))
    return oracle.moe_combine(outs, w)


@pytest.mark.parametrize("fmt", ["fp32", "bf16", "fp4", "mxfp4"])
@pytest.mark.parametrize("mode", [0, 1, 2, 3])
@pytest.mark.parametrize("T", [1, 4])
def test_decode_matches_oracle(fmt, mode, T):
    import routed_expert_ffn_02_amd as R
    wl = FMT[fmt]
    if wl.top_k * T > wl.n_experts * 2:
        pytest.skip("shape")
    n_slots = max(2, wl.n_keys // 3)
    bw = (25_000_000_000, 100_000_000_000)
    h = Harness(wl, mode, n_slots=n_slots, bw=bw)
    ref = oracle.ExpertCache(wl.n_layers, wl.n_experts, n_slots)
    routes = {l: wl.synthetic_routing(10, l, T) for l in range(wl.n_layers)}
    for step in range(10):
        for layer in range(wl.n_layers):
            idx = routes[layer][step]
            x = wl.decode_activations(step, layer, T)
            w = _gates(wl, step, layer, T)
            y, slot, trace, cnt = h.decode(layer, x, idx, w)
            assert row_rel_err(y, _expected(wl, layer, x, idx, w)) <= tol_for(wl), (step, layer)
            if mode != R.MOE_MODE_FUSED:
                r = ref.lookup(layer, idx, mode, *bw)
                assert trace == r.trace and np.array_equal(slot, r.slot_idx), (step, layer)
    st = R.moe_get_stats(h.ctx)
    if mode in (R.MOE_MODE_CPU, R.MOE_MODE_HYBRID):
        assert st["cpu_experts"] > 0


@pytest.mark.parametrize("fmt", ["fp32", "bf16", "fp4", "mxfp4"])
def test_full_residency_bit_identical_to_fused(fmt):
    """Once every expert is resident, the cached path equals the all-resident path bit for bit."""
    import routed_expert_ffn_02_amd as R
    wl = FMT[fmt]
    fused = Harness(wl, R.MOE_MODE_FUSED)
    cached = Harness(wl, R.MOE_MODE_OFFLOAD, n_slots=wl.n_keys)
    for layer in range(wl.n_layers):   # warm: touch every expert
        for e0 in range(0, wl.n_experts, wl.top_k):
            idx = np.array([[(e0 + j) % wl.n_experts for j in range(wl.top_k)]])
            x = wl.decode_activations(99, layer, 1)
            cached.decode(layer, x, idx, _gates(wl, 99, layer, 1))
    for step in range(6):
        for layer in range(wl.n_layers):
            idx = wl.synthetic_routing(6, layer, 2)[step]
            x = wl.decode_activations(step, layer, 2)
            w = _gates(wl, step, layer, 2)
            ya, _, _, _ = fused.decode(layer, x, idx, w)
            yb, _, trace, cnt = cached.decode(layer, x, idx, w)
            assert cnt[1] == 0 and cnt[2] == 0          # all hits
            assert np.array_equal(ya.view(np.uint32), yb.view(np.uint32)), (step, layer)


def test_decode_requires_lookup_first():
    import routed_expert_ffn_02_amd as R
    import torch
    h = Harness(BF16, R.MOE_MODE_OFFLOAD, n_slots=8)
    x = torch.zeros((1, BF16.hidden), dtype=torch.int16, device="cuda")
    idx = torch.zeros((1, BF16.top_k), dtype=torch.int32, device="cuda")
    w = torch.zeros((1, BF16.top_k), dtype=torch.float32, device="cuda")
    y = torch.zeros((1, BF16.hidden), dtype=torch.float32, device="cuda")
    with pytest.raises(R.MoeError) as e:
        R.moe_ffn_decode(h.ctx, 0, x, 1, idx, w, idx, y)
    assert e.value.status == R.MOE_ESTATE
    bad = torch.full((1, BF16.top_k), BF16.n_experts + 3, dtype=torch.int32, device="cuda")
    slot = torch.empty_like(bad)
    R.expert_cache_lookup(h.ctx, 0, bad, 1, slot)
    with pytest.raises(R.MoeError) as e:
        R.moe_ffn_decode(h.ctx, 0, x, 1, bad, w, slot, y)
    assert e.value.status == R.MOE_EINVAL


REAL_ROWS = {
    "a3b_bf16": W.A3B_DECODE.with_(name="a3b_rows", n_layers=2, n_experts=16, n_slots=12),
    "dsv4_fp4": W.DSV4.with_(name="dsv4_rows", n_layers=2, n_experts=8, n_slots=6),
    "dsv4_mxfp4": W.DSV4_MX.with_(name="dsv4mx_rows", n_layers=2, n_experts=8, n_slots=6),
    "wide_bf16": W.A3B_DECODE.with_(name="wide_rows", n_layers=1, n_experts=8, top_k=4, hidden=4096, inter=512,
                                    n_slots=6),
}


@pytest.mark.parametrize("name", list(REAL_ROWS))
@pytest.mark.parametrize("T", [1, 4])
@pytest.mark.parametrize("mode", [1, 3])
def test_decode_real_row_widths(name, T, mode):
    """The register-resident GEMV variants used at the A3B and DSV4 row widths."""
    wl = REAL_ROWS[name]
    bw = (25_000_000_000, 100_000_000_000)
    h = Harness(wl, mode, bw=bw)
    ref = oracle.ExpertCache(wl.n_layers, wl.n_experts, wl.n_slots)
    routes = {l: wl.synthetic_routing(4, l, T) for l in range(wl.n_layers)}
    for step in range(4):
        for layer in range(wl.n_layers):
            idx = routes[layer][step]
            x = wl.decode_activations(step, layer, T)
            w = _gates(wl, step, layer, T)
            y, slot, trace, cnt = h.decode(layer, x, idx, w)
            r = ref.lookup(layer, idx, mode, *bw)
            assert trace == r.trace
            assert row_rel_err(y, _expected(wl, layer, x, idx, w)) <= tol_for(wl), (step, layer)
