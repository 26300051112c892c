"""GPU: the MX prefill of MXFP4 experts (MOE_FLAG_MX_PREFILL: MXFP8 activations, the
scaled MFMA over e2m1 codes and E8M0 scales) against the oracle's MX expert FFN
(oracle/mx.py), through the C ABI.  Exact-arithmetic inputs (which MXFP8 holds exactly,
activations and SwiGLU intermediates alike) must match bit for bit on every row, at small
shapes over several tiles and ragged tails and on whole layers of the DSV4 shape; general
inputs within the format's tolerance."""
import numpy as np
import pytest

import oracle
import workloads as W
from moe_harness import Harness, exact_f32, oracle_outputs, row_rel_err, tol_for

pytestmark = pytest.mark.gpu

SMALL = W.DSV4_MX.with_(name="mx_small", n_layers=2, n_experts=16, top_k=3, hidden=512, inter=256)
SMALL_X = SMALL.with_(name="mx_small_exact", exact=True)
SMALL_H768 = W.DSV4_MX.with_(name="mx_h768", exact=True, n_layers=2, n_experts=16, top_k=3, hidden=768, inter=512)
FULL_X = W.DSV4_MX.with_(name="mx_full_exact", exact=True, n_layers=2)
FULL = W.DSV4_MX.with_(name="mx_full", n_layers=1)


def _gates(rng, shape):
    return rng.choice(np.array([1.0, 0.5, 0.25], np.float32), size=shape)


def _routes(rng, wl, T):
    return np.stack([rng.permutation(wl.n_experts)[: wl.top_k] for _ in range(T)]).astype(np.int32)


def _skewed(rng, wl, T, n_hot):
    E, k = wl.n_experts, wl.top_k
    if n_hot:
        pool = rng.permutation(E)[:n_hot]
        return np.stack([rng.choice(pool, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    p = 1.0 / np.arange(1, E + 1) ** 0.7
    p = p[rng.permutation(E)]
    p /= p.sum()
    return np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)


def _run(wl, T, routes_of, check, buffered=True, seed=None):
    import routed_expert_ffn_02_amd as R
    n_slots = 2 * wl.n_experts + 5 if buffered else max(2, wl.n_experts // 2)
    h = Harness(wl, R.MOE_MODE_OFFLOAD, n_slots=n_slots, max_tokens=T, flags=R.MOE_FLAG_MX_PREFILL)
    rng = np.random.default_rng(T if seed is None else seed)
    try:
        R.moe_prefill_begin(h.ctx)
        for layer in range(wl.n_layers):
            x = wl.prefill_activations(layer, T)
            idx = routes_of(rng, layer)
            w = _gates(rng, idx.shape)
            y, _, _ = h.prefill_layer(layer, x, idx, w)
            check(layer, x, idx, w, y)
        R.moe_prefill_end(h.ctx)
    finally:
        R.moe_destroy(h.ctx)


def _exact_check(wl):
    def check(layer, x, idx, w, y):
        want = exact_f32(oracle.moe_combine(oracle_outputs(wl, layer, x, idx, ffn=oracle.expert_ffn_mx), w))
        bad = np.nonzero(np.any(y != want, axis=1))[0]
        assert bad.size == 0, (layer, bad[:8].tolist(), int(bad.size))
    return check


@pytest.mark.parametrize("T", [1, 100, 257])
def test_mx_prefill_exact(T):
    _run(SMALL_X, T, lambda rng, layer: _routes(rng, SMALL_X, T), _exact_check(SMALL_X))


def test_mx_prefill_exact_h768_ondemand():
    """Three 256-k chunks in GEMM1, two in GEMM2, experts loaded on demand."""
    _run(SMALL_H768, 64, lambda rng, layer: _routes(rng, SMALL_H768, 64), _exact_check(SMALL_H768), buffered=False)


def test_mx_prefill_full_layers_exact():
    """Every row of two DSV4-shaped layers (2048 tokens): one routed to 24 experts (groups of
    many 64-row tiles), one to all 256 with a skew (ragged group tails, 32-row tiles)."""
    T = FULL_X.prefill_tokens
    _run(FULL_X, T, lambda rng, layer: _skewed(rng, FULL_X, T, 24 if layer == 0 else 0), _exact_check(FULL_X))


@pytest.mark.parametrize("T", [1, 100, 257])
def test_mx_prefill_general_inputs(T):
    """Seeded Gaussian-like activations and the workload's MXFP4 weights: MXFP8 rounding of
    the SwiGLU intermediate may differ where the GPU's fp32 value and the oracle's sit on
    opposite sides of a rounding boundary, so the bar is the format's tolerance."""
    def check(layer, x, idx, w, y):
        ref = oracle.moe_combine(oracle_outputs(SMALL, layer, x, idx, ffn=oracle.expert_ffn_mx), w)
        assert row_rel_err(y, ref) <= tol_for(SMALL), layer
    _run(SMALL, T, lambda rng, layer: _routes(rng, SMALL, T), check)


def test_mx_prefill_full_layer_sampled_rows():
    """A DSV4-shaped layer with the workload's inputs: 64 sampled token rows against the
    oracle's MX expert FFN."""
    T = FULL.prefill_tokens

    def check(layer, x, idx, w, y):
        rows = np.random.default_rng(1).choice(T, 64, replace=False)
        ref = oracle.moe_combine(oracle_outputs(FULL, layer, x[rows], idx[rows], ffn=oracle.expert_ffn_mx), w[rows])
        assert row_rel_err(y[rows], ref) <= tol_for(FULL)
    _run(FULL, T, lambda rng, layer: _skewed(rng, FULL, T, 0), check)


def test_mx_flag_needs_mxfp4():
    import routed_expert_ffn_02_amd as R
    wl = W.DSV4.with_(name="mx_fp4_refused", n_layers=1, n_experts=8, top_k=2, hidden=256, inter=256)
    cfg = R.make_config(wl.n_layers, wl.n_experts, wl.top_k, wl.hidden, wl.inter, wl.wfmt, wl.afmt, 8,
                        R.MOE_MODE_OFFLOAD, wl.renorm, flags=R.MOE_FLAG_MX_PREFILL)
    with pytest.raises(R.MoeError) as e:
        R.moe_create(cfg)
    assert e.value.status == R.MOE_ENOTSUP
