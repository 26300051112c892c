"""GPU parity: elastic cache resize at safe points (shrink, grow, new arena), with traces,
residency tables and outputs against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from moe_harness import Harness, row_rel_err, tol_for

pytestmark = pytest.mark.gpu

RS = W.A3B_DECODE.with_(name="resize_small", n_layers=3, n_experts=32, top_k=4, hidden=256, inter=128)


def _gates(wl, step, layer, T):
    u = wl.uniforms(5000 + step * 64 + layer, T * wl.top_k).reshape(T, wl.top_k) + 0.05
    return (u / u.sum(axis=1, keepdims=True)).astype(np.float32)


@pytest.mark.parametrize("mode", [1, 3])
def test_resize_schedule(mode):
    import routed_expert_ffn_02_amd as R
    wl = RS
    bw = (30_000_000_000, 90_000_000_000)
    schedule = {8: 12, 16: 30, 24: 5}
    cap = max([40] + list(schedule.values()))
    h = Harness(wl, mode, n_slots=40, bw=bw, max_tokens=4)
    ref = oracle.ExpertCache(wl.n_layers, wl.n_experts, 40)
    T = 2
    routes = {l: wl.synthetic_routing(32, l, T) for l in range(wl.n_layers)}
    for step in range(32):
        if step in schedule:
            n_new = schedule[step]
            if step == 16:   # grow into a new arena
                new = torch.empty(n_new * h.S, dtype=torch.uint8, device="cuda")
                R.expert_cache_resize(h.ctx, n_new, new, new.numel())
                h.arena = new
            else:
                R.expert_cache_resize(h.ctx, n_new)
            ref.resize(n_new)
            slot_of, key_of, stamp, counter = h.snapshot()
            assert np.array_equal(key_of, ref.key_of.astype(np.int32))
            assert np.array_equal(stamp, ref.stamp.astype(np.uint64))
        for layer in range(wl.n_layers):
            idx = routes[layer][step]
            x = wl.decode_activations(step, layer, T)
            w = _gates(wl, step, layer, T)
            y, slot, trace, cnt = h.decode(layer, x, idx, w)
            r = ref.lookup(layer, idx, mode, *bw)
            assert trace == r.trace, (step, layer)
            x64 = oracle.formats.activations_f64(x)
            outs = oracle.moe_layer_dense(x64, idx, lambda e: oracle.expert_weights_f64(wl, layer * wl.n_experts + e))
            assert row_rel_err(y, oracle.moe_combine(outs, w)) <= tol_for(wl), (step, layer)


def test_resize_rejected_in_prefill_and_fused():
    import routed_expert_ffn_02_amd as R
    h = Harness(RS, R.MOE_MODE_OFFLOAD, n_slots=70)
    R.moe_prefill_begin(h.ctx)
    with pytest.raises(R.MoeError) as e:
        R.expert_cache_resize(h.ctx, 10)
    assert e.value.status == R.MOE_ESTATE
    R.moe_prefill_end(h.ctx)
    f = Harness(RS, R.MOE_MODE_FUSED)
    with pytest.raises(R.MoeError) as e:
        R.expert_cache_resize(f.ctx, 10)
    assert e.value.status == R.MOE_ENOTSUP
