"""GPU: moe_permute_noalloc (no context, scratch in the library's static device array)
against moe_permute through the C ABI: bit-identical permutation, offsets, group slots
and group count on two calls in a row, the second with a smaller input, and the error
report (n_groups = -1) for an out-of-range slot id and for too many distinct slots."""
import numpy as np
import pytest
import torch

import workloads as W
from moe_harness import Harness

pytestmark = pytest.mark.gpu

WL = W.A3B_PREFILL.with_(name="na_bf16", n_layers=3, n_experts=16, top_k=4, hidden=256, inter=128)


def _outputs(P):
    return [torch.full((n,), -9, dtype=torch.int32, device="cuda") for n in (P, P + 1, P, 1)]


def _both(R, h, slot):
    T, k = slot.shape
    P = T * k
    st = torch.from_numpy(np.ascontiguousarray(slot, np.int32)).cuda()
    a = _outputs(P)
    R.moe_permute(h.ctx, st, T, *a)
    b = _outputs(P)
    R.moe_permute_noalloc(st, P, 4096, *b)   # the context's slot range: max(L*E, 4096)
    torch.cuda.synchronize()
    a = [t.cpu().numpy() for t in a]
    b = [t.cpu().numpy() for t in b]
    n = int(a[3][0])
    npairs = int(np.sum(slot >= 0))
    assert int(b[3][0]) == n
    assert np.array_equal(b[0][:npairs], a[0][:npairs])     # perm
    assert np.array_equal(b[1][: n + 1], a[1][: n + 1])     # offsets
    assert np.array_equal(b[2][:n], a[2][:n])               # group slots
    return n


def test_noalloc_permute_matches_moe_permute():
    import routed_expert_ffn_02_amd as R
    h = Harness(WL, R.MOE_MODE_OFFLOAD, n_slots=40, max_tokens=2048)
    rng = np.random.default_rng(5)
    # two calls in a row, the second smaller; then a large one with many distinct slots
    for T, hi in ((1500, 40), (7, 40), (2048, 1000)):
        slot = rng.integers(-3, hi, size=(T, WL.top_k)).astype(np.int32)
        n = _both(R, h, slot)
        assert n == len(np.unique(slot[slot >= 0]))


def test_noalloc_permute_reports_errors():
    import routed_expert_ffn_02_amd as R
    rng = np.random.default_rng(6)
    slot = rng.integers(0, 40, size=(300, 4)).astype(np.int32)
    slot[17, 2] = 5000                                       # >= n_slot_range
    P = slot.size
    b = _outputs(P)
    R.moe_permute_noalloc(torch.from_numpy(slot).cuda(), P, 4096, *b)
    torch.cuda.synchronize()
    assert int(b[3].item()) == -1
    many = np.arange(2048 * 4, dtype=np.int32).reshape(2048, 4) % 3000   # 3000 distinct > 1024
    b = _outputs(many.size)
    R.moe_permute_noalloc(torch.from_numpy(many).cuda(), many.size, 4096, *b)
    torch.cuda.synchronize()
    assert int(b[3].item()) == -1
    with pytest.raises(R.MoeError):
        R.moe_permute_noalloc(torch.from_numpy(many).cuda(), 1 << 17, 4096, *b)
    # a valid call afterwards still matches (the shared scratch holds the failed calls' state)
    h = Harness(WL, R.MOE_MODE_OFFLOAD, n_slots=40, max_tokens=600)
    _both(R, h, rng.integers(-3, 40, size=(600, 4)).astype(np.int32))
