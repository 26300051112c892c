"""GPU parity: prefill (full-layer double buffers, on-demand fallback, FUSED, CPU mode),
the token permutation and the grouped GEMMs, against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from moe_harness import Harness, row_rel_err, tol_for

pytestmark = pytest.mark.gpu

PF_BF16 = W.A3B_PREFILL.with_(name="pf_bf16", n_layers=3, n_experts=16, top_k=4, hidden=256, inter=128)
PF_FP4 = W.DSV4.with_(name="pf_fp4", n_layers=3, n_experts=16, top_k=3, hidden=256, inter=128)
# inter a multiple of 256 takes the LDS-staged FP4 kernels; 128 takes the register-streamed ones
PF_FP4_256 = W.DSV4.with_(name="pf_fp4_256", n_layers=3, n_experts=16, top_k=3, hidden=512, inter=256)
PF_MX = W.DSV4_MX.with_(name="pf_mxfp4", n_layers=3, n_experts=16, top_k=3, hidden=512, inter=256)
# hidden a multiple of 512 takes the down-projection blocks of 512 columns; 768 the 256-column ones
PF_FP4_768 = W.DSV4.with_(name="pf_fp4_768", n_layers=2, n_experts=16, top_k=3, hidden=768, inter=256)
PF_MX_768 = W.DSV4_MX.with_(name="pf_mxfp4_768", n_layers=2, n_experts=16, top_k=3, hidden=768, inter=256)


def _route_np(wl, layer, x):
    orc = oracle.OracleMoE(wl)
    _, idx, w = orc.route(layer, x, np.tile(wl.zipf_bias(layer), (x.shape[0], 1)))
    return idx, w


def _expected(wl, layer, x, idx, w):
    x64 = oracle.formats.activations_f64(x)
    outs = oracle.moe_layer_dense(x64, idx, lambda e: oracle.expert_weights_f64(wl, layer * wl.n_experts + e))
    return oracle.moe_combine(outs, w)


@pytest.mark.parametrize("wl", [PF_BF16, PF_FP4, PF_FP4_256, PF_MX, PF_FP4_768, PF_MX_768],
                         ids=["bf16", "fp4", "fp4_staged", "mxfp4", "fp4_staged_h768", "mxfp4_h768"])
@pytest.mark.parametrize("T", [1, 100, 257])
def test_buffered_prefill_matches_oracle(wl, T):
    import routed_expert_ffn_02_amd as R
    n_slots = 2 * wl.n_experts + 5
    h = Harness(wl, R.MOE_MODE_OFFLOAD, n_slots=n_slots, max_tokens=T)
    ref = oracle.ExpertCache(wl.n_layers, wl.n_experts, n_slots)
    # some decode residency first; prefill must not corrupt it
    for layer in range(wl.n_layers):
        idx0 = np.array([[(layer + j) % wl.n_experts for j in range(wl.top_k)]])
        h.lookup(layer, idx0)
        ref.lookup(layer, idx0, R.MOE_MODE_OFFLOAD)
    R.moe_prefill_begin(h.ctx)
    assert ref.prefill_begin()
    for layer in range(wl.n_layers):
        x = wl.prefill_activations(layer, T)
        idx, w = _route_np(wl, layer, x)
        y, tr, cnt = h.prefill_layer(layer, x, idx, w)
        r = ref.prefill_buffer_lookup(layer, idx)
        assert [tuple(int(v) for v in t) for t in tr[: len(r.trace)]] == r.trace
        assert row_rel_err(y, _expected(wl, layer, x, idx, w)) <= tol_for(wl)
    R.moe_prefill_end(h.ctx)
    ref.prefill_end()
    slot_of, key_of, stamp, counter = h.snapshot()
    assert np.array_equal(slot_of, ref.slot_of.astype(np.int32))
    assert np.array_equal(key_of, ref.key_of.astype(np.int32))
    assert np.array_equal(stamp, ref.stamp.astype(np.uint64)) and counter == ref.counter


def test_ondemand_prefill_tiny_fp32():
    import routed_expert_ffn_02_amd as R
    wl = W.TINY
    T = wl.prefill_tokens
    h = Harness(wl, R.MOE_MODE_OFFLOAD, n_slots=wl.n_slots, max_tokens=T)
    ref = oracle.ExpertCache(wl.n_layers, wl.n_experts, wl.n_slots)
    R.moe_prefill_begin(h.ctx)
    assert not ref.prefill_begin()
    x = wl.prefill_activations(0, T)
    idx, w = _route_np(wl, 0, x)
    y, tr, cnt = h.prefill_layer(0, x, idx, w)
    rounds = ref.prefill_ondemand(0, idx)
    R.moe_prefill_end(h.ctx)
    ref.prefill_end()
    final = {}
    for r in rounds:
        for t in r.trace:
            if t[1] in (oracle.KIND_HIT, oracle.KIND_FILL):
                final[t[0]] = t
    order = oracle.cache.unique_first_appearance(0 * wl.n_experts + idx)
    assert [tuple(int(v) for v in t) for t in tr[: len(order)]] == [final[u] for u in order]
    assert row_rel_err(y, _expected(wl, 0, x, idx, w)) <= tol_for(wl)
    slot_of, key_of, stamp, counter = h.snapshot()
    assert np.array_equal(key_of, ref.key_of.astype(np.int32)) and counter == ref.counter


@pytest.mark.parametrize("mode", [0, 2])
def test_fused_and_cpu_mode_prefill(mode):
    import routed_expert_ffn_02_amd as R
    wl = PF_BF16
    T = 70
    h = Harness(wl, mode, n_slots=6, max_tokens=T)
    R.moe_prefill_begin(h.ctx)
    for layer in range(wl.n_layers):
        x = wl.prefill_activations(layer, T)
        idx, w = _route_np(wl, layer, x)
        y, tr, cnt = h.prefill_layer(layer, x, idx, w)
        assert row_rel_err(y, _expected(wl, layer, x, idx, w)) <= tol_for(wl), layer
    R.moe_prefill_end(h.ctx)


def test_permute_is_stable_sort_by_slot():
    import routed_expert_ffn_02_amd as R
    wl = PF_BF16
    h = Harness(wl, R.MOE_MODE_OFFLOAD, n_slots=40, max_tokens=600)
    rng = np.random.default_rng(4)
    for T in (1, 5, 600):
        slot = rng.integers(-3, 40, size=(T, wl.top_k)).astype(np.int32)
        st = torch.from_numpy(slot).cuda()
        P = T * wl.top_k
        perm = torch.full((P,), -9, dtype=torch.int32, device="cuda")
        offs = torch.full((P + 1,), -9, dtype=torch.int32, device="cuda")
        gs = torch.full((P,), -9, dtype=torch.int32, device="cuda")
        ng = torch.zeros(1, dtype=torch.int32, device="cuda")
        R.moe_permute(h.ctx, st, T, perm, offs, gs, ng)
        torch.cuda.synchronize()
        flat = slot.reshape(-1)
        gpu_pairs = np.nonzero(flat >= 0)[0]
        ref_perm = gpu_pairs[np.argsort(flat[gpu_pairs], kind="stable")]
        groups = np.unique(flat[gpu_pairs])
        n = int(ng.item())
        assert n == len(groups)
        assert np.array_equal(gs.cpu().numpy()[:n], groups)
        assert np.array_equal(perm.cpu().numpy()[: len(ref_perm)], ref_perm)
        counts = np.array([np.sum(flat == g) for g in groups])
        assert np.array_equal(offs.cpu().numpy()[: n + 1], np.concatenate([[0], np.cumsum(counts)]))


@pytest.mark.parametrize("wl", [PF_BF16, PF_FP4_256], ids=["bf16", "fp4_staged"])
@pytest.mark.parametrize("T", [33, 600])
def test_prefill_skewed_groups(wl, T):
    """Uneven groups, as a prompt's routing makes them: every token's first pick is expert
    0 (one group of T rows: several 64-row tiles, the last possibly a short one), the second
    alternates between experts 1 and 2, the third spreads over the rest; the GEMMs' tile
    tables and their split of the tiles over the XCDs must cover every row exactly once."""
    import routed_expert_ffn_02_amd as R
    E, k = wl.n_experts, wl.top_k
    assert k == 3 or k == 4
    h = Harness(wl, R.MOE_MODE_OFFLOAD, n_slots=2 * E + 1, max_tokens=T)
    rng = np.random.default_rng(T)
    R.moe_prefill_begin(h.ctx)
    for layer in range(wl.n_layers):
        x = wl.prefill_activations(layer, T)
        t = np.arange(T)
        cols = [np.zeros(T, dtype=np.int64), 1 + t % 2, 3 + (7 * t) % (E - 3)]
        if k == 4:
            cols.append(3 + (7 * t + 1) % (E - 3))
        idx = np.stack(cols, axis=1).astype(np.int32)
        w = rng.uniform(0.1, 1.0, size=(T, k))
        w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
        y, tr, cnt = h.prefill_layer(layer, x, idx, w)
        assert row_rel_err(y, _expected(wl, layer, x, idx, w)) <= tol_for(wl), layer
    R.moe_prefill_end(h.ctx)
