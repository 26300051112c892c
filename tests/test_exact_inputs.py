"""The exact-arithmetic inputs (workloads `exact=True`): their premise, checked on the CPU.

With these inputs every product and every partial sum of the expert FFN, the combine
and the router is an fp32 number, the gate projection is 0 or at least 32 (so
silu(g) = g / (1 + e^-g) rounds to g in fp32: e^-32 < 2^-24), and the SwiGLU
intermediate h = silu(g) * u has at most 4 significant bits (exact in bf16 and f16,
the operand types the GPU kernels round h to).  The GPU parity tests built on them
then demand bit-identical results, which catches a single wrong index that a
relative tolerance would let through.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from moe_harness import exact_f32

SHAPE = dict(n_layers=2, n_experts=8, hidden=512, inter=256)
FMT = {"fp32": W.TINY, "bf16": W.A3B_DECODE, "fp4": W.DSV4, "mxfp4": W.DSV4_MX}


def _bits(v):
    """Significant bits of each nonzero value (mantissa width of an exact binary fraction)."""
    v = np.abs(np.asarray(v, np.float64))
    v = v[v != 0]
    m, _ = np.frexp(v)
    bits = np.zeros(v.shape, np.int64)
    while np.any(m != 0):
        nz = m != 0
        bits[nz] += 1
        m = np.where(nz, m * 2 - np.floor(m * 2), 0)
    return bits


@pytest.mark.parametrize("fmt", sorted(FMT))
def test_exact_inputs_keep_every_result_representable(fmt):
    wl = FMT[fmt].with_(exact=True, top_k=4, **SHAPE)
    rng = np.random.default_rng(7)
    T = 16
    x = wl.prefill_activations(1, T)
    x64 = oracle.formats.activations_f64(x)
    assert set(np.unique(x64).tolist()) <= {0.0, 1.0, 2.0}
    for e in range(wl.n_experts):
        wg, wu, wd = oracle.expert_weights_f64(wl, wl.n_experts + e)
        assert np.all(wg >= 0) and np.all((wg != 0).sum(axis=1) <= 1) and np.all((wu != 0).sum(axis=1) == 1)
        assert np.all((wd != 0).sum(axis=1) <= 4) and np.all((wd != 0).sum(axis=1) >= 1)
        g = x64 @ wg.T
        assert np.all((g == 0) | (g >= 32))
        h = oracle.silu(g) * (x64 @ wu.T)
        hr = np.where(g == 0, 0.0, g * (x64 @ wu.T))          # silu(g) = g where g >= 32
        assert np.allclose(h, hr, rtol=1e-12, atol=0)
        assert _bits(hr).max(initial=0) <= 4 and np.abs(hr).max() < 65504
        assert np.all((hr == 0) | (np.abs(hr) >= 2 ** -14))    # f16 normal range
    idx = np.stack([rng.permutation(wl.n_experts)[: wl.top_k] for _ in range(T)]).astype(np.int32)
    gates = rng.choice([1.0, 0.5, 0.25], size=idx.shape).astype(np.float32)
    outs = oracle.moe_layer_dense(x64, idx, lambda e: oracle.expert_weights_f64(wl, wl.n_experts + e))
    exact_f32(outs)
    y = exact_f32(oracle.moe_combine(outs, gates))
    assert np.count_nonzero(y) > y.size // 4
    z = oracle.router_logits(x64, wl.router_weight(1))
    assert np.array_equal(z.astype(np.float64), x64 @ wl.router_weight(1).astype(np.float64).T)


def test_exact_premise_detects_a_planted_error():
    """exact_f32 refuses a result off the 2^-16 grid (a planted 1e-6 error) or one that is
    not an fp32 number, and absorbs only fp64 noise (a cancelled sum left at 1e-14)."""
    with pytest.raises(AssertionError):
        exact_f32(np.array([[1.0 + 1e-6]]))
    with pytest.raises(AssertionError):
        exact_f32(np.array([[2.0 ** 30 + 2.0 ** -10]]))
    got = exact_f32(np.array([[1.5, -2.0 ** -10, 1.4e-14]]))
    assert got.dtype == np.float32 and got.tolist() == [[1.5, -2.0 ** -10, 0.0]]
