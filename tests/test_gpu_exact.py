"""GPU parity, bit for bit, on exact-arithmetic inputs (workloads `exact=True`).

Every product and partial sum of these inputs is an fp32 number and the SwiGLU
intermediate is exact in the 16-bit operand types (tests/test_exact_inputs.py checks
the premise on the CPU), so the library's outputs must equal the oracle's exactly,
whatever the summation order, for every format, mode and path: one wrong weight row,
code nibble, block scale, activation, slot or group index changes some element.
Gates are chosen from {1, 1/2, 1/4} so the combine is exact too.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from moe_harness import Harness, dev_act, exact_f32, oracle_outputs, row_rel_err

pytestmark = pytest.mark.gpu

BW = (25_000_000_000, 100_000_000_000)   # B_P : B_H = 1 : 4 (hybrid steps split their misses)
SMALL = dict(n_layers=2, n_experts=16)
DEC = {
    "fp32": W.TINY.with_(name="ex_f32", exact=True, top_k=4, hidden=256, inter=128, **SMALL),
    "bf16": W.A3B_DECODE.with_(name="ex_bf16", exact=True, top_k=4, hidden=512, inter=256, **SMALL),
    "fp4": W.DSV4.with_(name="ex_fp4", exact=True, top_k=3, hidden=512, inter=256, **SMALL),
    "mxfp4": W.DSV4_MX.with_(name="ex_mxfp4", exact=True, top_k=3, hidden=512, inter=256, **SMALL),
}
# the real row widths of the benchmarked shapes (the GEMV variants the benchmark runs)
ROWS = {
    "a3b_bf16": W.A3B_DECODE.with_(name="ex_rows_a3b", exact=True, **SMALL),
    "dsv4_fp4": W.DSV4.with_(name="ex_rows_dsv4", exact=True, **SMALL),
    "dsv4_mxfp4": W.DSV4_MX.with_(name="ex_rows_dsv4mx", exact=True, **SMALL),
}


def _gates(rng, shape):
    return rng.choice(np.array([1.0, 0.5, 0.25], np.float32), size=shape)


def _routes(rng, wl, T):
    return np.stack([rng.permutation(wl.n_experts)[: wl.top_k] for _ in range(T)]).astype(np.int32)


PATHS = {  # mode, slots (None: a third of the keys), flags
    "offload_host_fills": (1, None, 0),
    "offload_device_fills": (1, "tight", 2),
    "hybrid": (3, None, 0),
    "hybrid_device_fills": (3, None, 2),
    "cpu": (2, None, 0),
    "fused": (0, None, 0),
}


def _decode_run(wl, path, T, steps, seed):
    import routed_expert_ffn_02_amd as R
    mode, slots, flags = PATHS[path]
    n_slots = max(2, wl.n_keys // 3) if slots is None else 2 * T * wl.top_k + 2
    h = Harness(wl, mode, n_slots=n_slots, bw=BW, flags=flags, max_tokens=max(8, T))
    ref = oracle.ExpertCache(wl.n_layers, wl.n_experts, n_slots)
    rng = np.random.default_rng(seed)
    try:
        for step in range(steps):
            for layer in range(wl.n_layers):
                idx, w = _routes(rng, wl, T), _gates(rng, (T, wl.top_k))
                x = wl.decode_activations(step, layer, T)
                y, slot, trace, cnt = h.decode(layer, x, idx, w)
                want = exact_f32(oracle.moe_combine(oracle_outputs(wl, layer, x, idx), w))
                assert np.array_equal(y, want), (path, step, layer, int(np.sum(y != want)))
                if mode != R.MOE_MODE_FUSED:
                    r = ref.lookup(layer, idx, mode, *BW)
                    assert trace == r.trace and np.array_equal(slot, r.slot_idx), (step, layer)
        R.moe_sync(h.ctx)
        return R.moe_get_stats(h.ctx)
    finally:
        R.moe_destroy(h.ctx)


@pytest.mark.parametrize("fmt", sorted(DEC))
@pytest.mark.parametrize("path", sorted(PATHS))
@pytest.mark.parametrize("T", [1, 4])
def test_exact_decode(fmt, path, T):
    st = _decode_run(DEC[fmt], path, T, steps=5, seed=T)
    if path.startswith("hybrid") or path == "cpu":
        assert st["cpu_experts"] > 0


@pytest.mark.parametrize("shape", sorted(ROWS))
@pytest.mark.parametrize("path", ["offload_device_fills", "hybrid_device_fills", "fused", "offload_host_fills"])
def test_exact_decode_real_rows(shape, path):
    T = 1 if path != "offload_host_fills" else 4
    _decode_run(ROWS[shape], path, T, steps=3, seed=11)


@pytest.mark.parametrize("shape", sorted(ROWS))
def test_exact_router_and_fused_layer_call(shape):
    """Router logits bit-exact; the all-resident per-layer call (top k inside phase 1)
    picks exactly the oracle's experts from exact, often tied, logits (ties to the lower
    index); its output equals the oracle's combine of the GPU's own gates to fp32
    rounding of the combine (the expert outputs are exact)."""
    import routed_expert_ffn_02_amd as R
    wl = ROWS[shape]
    h = Harness(wl, R.MOE_MODE_FUSED, max_tokens=64)
    E, k, H = wl.n_experts, wl.top_k, wl.hidden
    try:
        for layer in range(wl.n_layers):
            x = wl.prefill_activations(layer, 64)
            z, idx, w = h.route(layer, x)
            z_ref = oracle.router_logits(oracle.formats.activations_f64(x), wl.router_weight(layer))
            assert np.array_equal(z, z_ref), layer
            i_ref, w_ref = oracle.route(z_ref, k, wl.renorm)
            assert np.array_equal(idx, i_ref), layer
            assert np.abs(w - w_ref).max() <= 1e-5
            assert any(len(np.unique(z_ref[t])) < E for t in range(64)), "no tied logits: tie-break not exercised"
            gi = torch.empty((1, k), dtype=torch.int32, device="cuda")
            gw = torch.empty((1, k), dtype=torch.float32, device="cuda")
            gs = torch.empty((1, k), dtype=torch.int32, device="cuda")
            y = torch.empty((1, H), dtype=torch.float32, device="cuda")
            for t in range(0, 64, 9):
                R.moe_decode_layer(h.ctx, layer, dev_act(wl, x[t:t + 1]), 1, None, gi, gw, gs, y)
                torch.cuda.synchronize()
                assert np.array_equal(gi.cpu().numpy()[0], i_ref[t]), (layer, t)
                assert np.array_equal(gs.cpu().numpy()[0], layer * E + i_ref[t])
                ref = oracle.moe_combine(oracle_outputs(wl, layer, x[t:t + 1], i_ref[t:t + 1]), gw.cpu().numpy())
                assert row_rel_err(y.cpu().numpy(), ref) <= 1e-6, (layer, t)
    finally:
        R.moe_destroy(h.ctx)


PF = {
    "bf16": W.A3B_PREFILL.with_(name="exp_bf16", exact=True, n_layers=3, n_experts=16, top_k=4, hidden=256,
                                inter=128),
    "fp4": W.DSV4.with_(name="exp_fp4", exact=True, n_layers=3, n_experts=16, top_k=3, hidden=256, inter=128),
    "fp4_staged": W.DSV4.with_(name="exp_fp4s", exact=True, n_layers=3, n_experts=16, top_k=3, hidden=512,
                               inter=256),
    "mxfp4": W.DSV4_MX.with_(name="exp_mx", exact=True, n_layers=3, n_experts=16, top_k=3, hidden=512, inter=256),
    "fp4_staged_h768": W.DSV4.with_(name="exp_fp4_768", exact=True, n_layers=2, n_experts=16, top_k=3, hidden=768,
                                    inter=256),
    "fp32": W.TINY.with_(name="exp_f32", exact=True, n_layers=2, n_experts=8, top_k=2, hidden=128, inter=128),
}


def _prefill_run(wl, T, routes_of, buffered=True):
    import routed_expert_ffn_02_amd as R
    n_slots = 2 * wl.n_experts + 5 if buffered else max(2, wl.n_experts // 2)
    h = Harness(wl, R.MOE_MODE_OFFLOAD, n_slots=n_slots, max_tokens=T)
    rng = np.random.default_rng(T)
    try:
        R.moe_prefill_begin(h.ctx)
        for layer in range(wl.n_layers):
            x = wl.prefill_activations(layer, T)
            idx = routes_of(rng, layer)
            w = _gates(rng, idx.shape)
            y, _, _ = h.prefill_layer(layer, x, idx, w)
            want = exact_f32(oracle.moe_combine(oracle_outputs(wl, layer, x, idx), w))
            bad = np.nonzero(np.any(y != want, axis=1))[0]
            assert bad.size == 0, (layer, bad[:8].tolist(), int(bad.size))
        R.moe_prefill_end(h.ctx)
    finally:
        R.moe_destroy(h.ctx)


@pytest.mark.parametrize("fmt", sorted(PF))
@pytest.mark.parametrize("T", [1, 100, 257])
def test_exact_prefill(fmt, T):
    wl = PF[fmt]
    _prefill_run(wl, T, lambda rng, layer: _routes(rng, wl, T), buffered=(fmt != "fp32"))


def test_exact_prefill_ondemand():
    wl = PF["bf16"]
    _prefill_run(wl, 64, lambda rng, layer: _routes(rng, wl, 64), buffered=False)


def _skewed_routes(rng, wl, T, n_hot):
    """Every token picks k distinct experts; layer routing concentrated on n_hot experts
    (groups of many 64-row tiles) or spread over all with a skew (ragged groups)."""
    E, k = wl.n_experts, wl.top_k
    if n_hot:
        pool = rng.permutation(E)[:n_hot]
        return np.stack([rng.choice(pool, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    p = 1.0 / np.arange(1, E + 1) ** 0.7
    p = p[rng.permutation(E)]
    p /= p.sum()
    return np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)


FULL = {
    "dsv4_fp4": W.DSV4.with_(name="exf_dsv4", exact=True, n_layers=2),
    "dsv4_mxfp4": W.DSV4_MX.with_(name="exf_dsv4mx", exact=True, n_layers=2),
    "a3b_bf16": W.A3B_PREFILL.with_(name="exf_a3b", exact=True, n_layers=2),
}


@pytest.mark.parametrize("shape", sorted(FULL))
def test_exact_prefill_full_layer(shape):
    """Every row of two full-size layers, the prompt lengths the benchmark runs (DSV4
    2048 tokens, A3B 4096): layer 0 routes to 24 experts (groups of many row tiles, the
    middle tiles included), layer 1 to all experts with a skew (ragged group tails)."""
    wl = FULL[shape]
    T = wl.prefill_tokens
    _prefill_run(wl, T, lambda rng, layer: _skewed_routes(rng, wl, T, 24 if layer == 0 else 0))
