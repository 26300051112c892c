"""GPU parity: the cache-control kernel (expert_cache_lookup) against the oracle's
ExpertCache -- traces, slot ids, counts and residency tables bit-exact."""
import numpy as np
import pytest

import oracle
import workloads as W
from moe_harness import Harness

pytestmark = pytest.mark.gpu

LK = W.A3B_DECODE.with_(name="lookup_small", n_layers=3, n_experts=64, top_k=4, hidden=64, inter=64)


def _traces_equal(gpu, ref):
    return [tuple(r) for r in gpu] == [tuple(r) for r in ref]


# T*k <= 64 takes the one-wavefront path of the kernel, larger steps the block-wide one
@pytest.mark.parametrize("mode,n_slots,T", [
    (1, 40, 1), (1, 7, 1), (1, 0, 1), (1, 200, 4), (1, 5, 4), (1, 3000, 4), (1, 70, 16),
    (3, 40, 1), (3, 13, 4), (2, 40, 1), (2, 9, 4),
    (1, 150, 20), (1, 30, 20), (3, 90, 20), (2, 40, 20)])
def test_lookup_sequence_matches_oracle(mode, n_slots, T):
    import routed_expert_ffn_02_amd as R
    bw = (25_000_000_000, 100_000_000_000) if mode == R.MOE_MODE_HYBRID else (0, 0)
    h = Harness(LK, mode, n_slots=n_slots, bw=bw, max_tokens=max(8, T))
    ref = oracle.ExpertCache(LK.n_layers, LK.n_experts, n_slots)
    routes = {l: LK.synthetic_routing(50, l, T) for l in range(LK.n_layers)}
    for step in range(50):
        for layer in range(LK.n_layers):
            idx = routes[layer][step]
            _, slot, tr, cnt = h.lookup(layer, idx)
            r = ref.lookup(layer, idx, mode, *bw)
            c = cnt.cpu().numpy()
            assert tuple(int(v) for v in c) == r.counts, (step, layer)
            nU = len(r.trace)
            assert _traces_equal(tr.cpu().numpy()[:nU], r.trace), (step, layer)
            assert np.array_equal(slot.cpu().numpy(), r.slot_idx), (step, layer)
    slot_of, key_of, stamp, counter = h.snapshot()
    assert np.array_equal(slot_of, ref.slot_of.astype(np.int32))
    assert np.array_equal(key_of, ref.key_of.astype(np.int32))
    assert np.array_equal(stamp, ref.stamp.astype(np.uint64))
    assert counter == ref.counter


def test_lookup_fused_mode_is_identity():
    import routed_expert_ffn_02_amd as R
    h = Harness(LK, R.MOE_MODE_FUSED)
    idx = LK.synthetic_routing(3, 2, 4)[2]
    _, slot, tr, cnt = h.lookup(2, idx)
    assert np.array_equal(slot.cpu().numpy(), 2 * LK.n_experts + idx)
    assert all(t[1] == R.MOE_KIND_HIT for t in tr.cpu().numpy()[: int(cnt[0])])
