"""GPU: a pool loaded from a bank file serves decode from a cold cache exactly like the
oracle (the first request fills through the ordinary miss path)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from moe_harness import dev_act, row_rel_err, tol_for

pytestmark = pytest.mark.gpu

WL = W.DSV4_MX.with_(name="bank_gpu_mx", n_layers=2, n_experts=16, top_k=3, hidden=512, inter=256)


def test_pool_from_bank_file_serves_cold_cache(tmp_path):
    import routed_expert_ffn_02_amd as R
    wl = WL
    L, E, k, H = wl.n_layers, wl.n_experts, wl.top_k, wl.hidden
    cfg = R.make_config(L, E, k, H, wl.inter, wl.wfmt, wl.afmt, 4, R.MOE_MODE_OFFLOAD)
    src = np.empty(wl.pool_records * wl.record_bytes, np.uint8)
    wl.fill_pool(src.ctypes.data, 0, wl.pool_records)
    path = str(tmp_path / "experts.bank")
    R.moe_bank_write(path, cfg, src, wl.pool_records)
    ctx = R.moe_create(cfg)
    ptr, st = R.moe_pool_load(ctx, path, 4)
    assert st["bytes"] == src.size
    # a second pool on the same context is refused
    with pytest.raises(R.MoeError):
        R.moe_pool_load(ctx, path, 4)
    S = R.moe_record_bytes(cfg)
    n_slots = E  # half the keys: misses continue after the cold start
    router = torch.from_numpy(np.stack([wl.router_weight(l) for l in range(L)])).cuda()
    arena = torch.empty(n_slots * S, dtype=torch.uint8, device="cuda")
    R.moe_bind(ctx, router, arena, arena.numel(), n_slots)
    ref = oracle.ExpertCache(L, E, n_slots)
    T = 2
    for step in range(6):
        for layer in range(L):
            idx_np = wl.synthetic_routing(6, layer, T)[step]
            x_np = wl.decode_activations(step, layer, T)
            w_np = np.full((T, k), 1.0 / k, np.float32)
            idx = torch.from_numpy(np.ascontiguousarray(idx_np, np.int32)).cuda()
            w = torch.from_numpy(w_np).cuda()
            slot = torch.empty((T, k), dtype=torch.int32, device="cuda")
            tr = torch.full((T * k, 4), -7, dtype=torch.int32, device="cuda")
            cnt = torch.zeros(4, dtype=torch.int32, device="cuda")
            R.expert_cache_lookup(ctx, layer, idx, T, slot, tr, cnt)
            y = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
            R.moe_ffn_decode(ctx, layer, dev_act(wl, x_np), T, idx, w, slot, y)
            torch.cuda.synchronize()
            r = ref.lookup(layer, idx_np, oracle.MODE_OFFLOAD)
            c = cnt.cpu().numpy()
            got = [tuple(int(v) for v in row) for row in tr.cpu().numpy()[:int(c[0] + c[1] + c[2])]]
            assert got == r.trace, (step, layer)
            x64 = oracle.formats.activations_f64(x_np)
            outs = oracle.moe_layer_dense(x64, idx_np, lambda e: oracle.expert_weights_f64(wl, layer * E + e))
            assert row_rel_err(y.cpu().numpy(), oracle.moe_combine(outs, w_np)) <= tol_for(wl), (step, layer)
            if step == 0 and layer == 0:
                assert c[0] == 0   # cold start: nothing resident
