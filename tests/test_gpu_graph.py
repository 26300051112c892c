"""GPU: a whole decode step (route + lookup + decode of every layer) captured into one
HIP graph and replayed must reproduce eager execution bit for bit, replay after replay,
with the cache state advancing on the device, and every replayed step must match the
oracle (top-k indices and gates, cache trace and slot ids, outputs).  Paths that
qualify: OFFLOAD and HYBRID with device fills (the CPU branch served by the library's
branch thread, joined on the device by a bounded wait), FUSED."""
import numpy as np
import pytest

import oracle
import workloads as W
from moe_harness import Harness, oracle_outputs, row_rel_err, tol_for

pytestmark = pytest.mark.gpu

BF16 = W.A3B_DECODE.with_(name="graph_bf16", n_layers=3, n_experts=16, top_k=4, hidden=256, inter=128)
FP4 = W.DSV4.with_(name="graph_fp4", n_layers=3, n_experts=16, top_k=3, hidden=256, inter=128)
# real row widths: the register-resident GEMV variants inside the graph
ROWS = W.A3B_DECODE.with_(name="graph_rows", n_layers=2, n_experts=16)


class StepBuffers:
    """Static device buffers of one decode step over all layers."""

    def __init__(self, wl, T):
        import torch
        L, k, H = wl.n_layers, wl.top_k, wl.hidden
        xdt = torch.int16 if wl.afmt == W.AFMT_BF16 else torch.float32
        K = max(1, min(T * k, wl.n_experts))
        self.T = T
        self.x = torch.zeros((L, T, H), dtype=xdt, device="cuda")
        self.idx = torch.zeros((L, T, k), dtype=torch.int32, device="cuda")
        self.w = torch.zeros((L, T, k), dtype=torch.float32, device="cuda")
        self.slot = torch.zeros((L, T, k), dtype=torch.int32, device="cuda")
        self.y = torch.zeros((L, T, H), dtype=torch.float32, device="cuda")
        self.trace = torch.zeros((L, K, 4), dtype=torch.int32, device="cuda")
        self.cnt = torch.zeros((L, 4), dtype=torch.int32, device="cuda")

    def load(self, wl, step):
        import torch
        for l in range(wl.n_layers):
            xs = wl.decode_activations(step, l, self.T)
            xs = xs.view(np.int16) if xs.dtype == np.uint16 else np.ascontiguousarray(xs, np.float32)
            self.x[l].copy_(torch.from_numpy(xs.copy()))

    def outputs(self):
        return [t.cpu().numpy().copy() for t in (self.y, self.idx, self.slot, self.trace, self.cnt, self.w)]


def check_against_oracle(wl, b, step, cache, mode, bw, fused):
    """One executed step (buffers b) against the oracle: routing on its own logits, the
    LRU trace and slot ids of its cache simulation, outputs from its FFN and combine."""
    y, idx, slot, trace, cnt, w = b.outputs()
    for l in range(wl.n_layers):
        x = wl.decode_activations(step, l, b.T)
        z_ref = oracle.router_logits(oracle.formats.activations_f64(x), wl.router_weight(l))
        i_ref, w_ref = oracle.route(z_ref, wl.top_k, wl.renorm)
        assert np.array_equal(idx[l], i_ref), (step, l)
        assert np.abs(w[l] - w_ref).max() <= 1e-5, (step, l)
        ref = oracle.moe_combine(oracle_outputs(wl, l, x, idx[l]), w[l])
        assert row_rel_err(y[l], ref) <= tol_for(wl), (step, l)
        if fused:
            assert np.array_equal(slot[l], l * wl.n_experts + idx[l])
            continue
        r = cache.lookup(l, idx[l], mode, *bw)
        n_u = int(cnt[l][0] + cnt[l][1] + cnt[l][2])
        assert [tuple(int(v) for v in t) for t in trace[l][:n_u]] == r.trace, (step, l)
        assert np.array_equal(slot[l], r.slot_idx), (step, l)


def run_step(R, h, b, stream, layer_call=False):
    for l in range(h.wl.n_layers):
        if layer_call:  # one call per layer (all resident at batch 1: router + top k in one launch)
            R.moe_decode_layer(h.ctx, l, b.x[l], b.T, None, b.idx[l], b.w[l], b.slot[l], b.y[l], stream)
            continue
        R.moe_route(h.ctx, l, b.x[l], b.T, None, None, b.idx[l], b.w[l], stream)
        R.expert_cache_lookup(h.ctx, l, b.idx[l], b.T, b.slot[l], b.trace[l], b.cnt[l], stream)
        R.moe_ffn_decode(h.ctx, l, b.x[l], b.T, b.idx[l], b.w[l], b.slot[l], b.y[l], stream)


@pytest.mark.parametrize("wl", [BF16, FP4, ROWS], ids=["bf16", "fp4", "rows"])
@pytest.mark.parametrize("mode", ["offload_device_fills", "hybrid_device_fills", "fused", "fused_layer_call"])
def test_captured_step_replays_like_eager(wl, mode):
    import routed_expert_ffn_02_amd as R
    import torch
    T = 1
    bw = (0, 0)
    lc = mode == "fused_layer_call"
    if mode.startswith("fused"):
        kw = dict(mode=R.MOE_MODE_FUSED)
        flags = 0
    elif mode == "hybrid_device_fills":  # few slots: the CPU branch runs on the branch thread
        kw = dict(mode=R.MOE_MODE_HYBRID, n_slots=wl.top_k + 1)
        flags = R.MOE_FLAG_DEVICE_FILLS
        bw = (25_000_000_000, 100_000_000_000)
    else:
        kw = dict(mode=R.MOE_MODE_OFFLOAD, n_slots=2 * T * wl.top_k + 2)
        flags = R.MOE_FLAG_DEVICE_FILLS
    eager = Harness(wl, kw["mode"], n_slots=kw.get("n_slots"), flags=flags, bw=bw)
    # profiling is requested on the captured context: captured launches must skip it
    graph = Harness(wl, kw["mode"], n_slots=kw.get("n_slots"), flags=flags | R.MOE_FLAG_PROFILE, bw=bw)
    be, bg = StepBuffers(wl, T), StepBuffers(wl, T)
    fused = mode.startswith("fused")
    cache = None if fused else oracle.ExpertCache(wl.n_layers, wl.n_experts, graph.n_slots)
    # step 0 eagerly on both
    be.load(wl, 0)
    bg.load(wl, 0)
    run_step(R, eager, be, None, lc)
    run_step(R, graph, bg, None, lc)
    torch.cuda.synchronize()
    check_against_oracle(wl, bg, 0, cache, kw["mode"], bw, fused)
    g = torch.cuda.CUDAGraph()
    # thread-local capture: only this thread's calls are checked against the capture
    # (the branch thread and the CPU worker pool run on threads of their own)
    with torch.cuda.graph(g, capture_error_mode="thread_local"):
        run_step(R, graph, bg, torch.cuda.current_stream().cuda_stream, lc)
    scratch = torch.randn(1 << 16, device="cuda")
    for step in range(1, 9):
        bg.load(wl, step)
        g.replay()
        scratch.mul_(0.5).add_(1.0)  # unrelated eager work between replays
        torch.cuda.synchronize()
        be.load(wl, step)
        run_step(R, eager, be, None, lc)
        torch.cuda.synchronize()
        for a, b_, name in zip(bg.outputs(), be.outputs(), ("y", "idx", "slot", "trace", "cnt", "w")):
            assert np.array_equal(a.view(np.uint8), b_.view(np.uint8)), (step, name)
        check_against_oracle(wl, bg, step, cache, kw["mode"], bw, fused)
    R.moe_sync(graph.ctx)
    R.moe_sync(eager.ctx)
    sg, se = R.moe_get_stats(graph.ctx), R.moe_get_stats(eager.ctx)
    if not mode.startswith("fused"):
        assert sg["fills"] == se["fills"] > 0 and sg["hits"] == se["hits"] and sg["lookups"] == se["lookups"]
        assert sg["cpu_experts"] == se["cpu_experts"]
        if mode == "hybrid_device_fills":
            assert se["cpu_experts"] > 0
    sa, ka, stamp_a, ca = graph.snapshot()
    sb, kb, stamp_b, cb = eager.snapshot()
    assert np.array_equal(sa, sb) and np.array_equal(ka, kb) and np.array_equal(stamp_a, stamp_b) and ca == cb


def test_capture_refuses_host_issued_fills():
    import routed_expert_ffn_02_amd as R
    import torch
    wl = BF16
    h = Harness(wl, R.MOE_MODE_OFFLOAD, n_slots=2 * wl.top_k + 2)  # no device fills
    b = StepBuffers(wl, 1)
    b.load(wl, 0)
    g = torch.cuda.CUDAGraph()
    with pytest.raises(R.MoeError) as e:
        with torch.cuda.graph(g):
            run_step(R, h, b, torch.cuda.current_stream().cuda_stream)
    assert e.value.status == R.MOE_ESTATE


@pytest.mark.parametrize("new_arena", [False, True], ids=["in_place", "new_arena"])
def test_replay_follows_resize(new_arena):
    """A step captured before expert_cache_resize replays on the resized cache: shrink
    (in place, or into a new arena) and grow between replays, every replayed step and the
    final tables checked against the oracle's cache with the same resizes."""
    import routed_expert_ffn_02_amd as R
    import torch
    wl, T = BF16, 1
    n0 = 4 * T * wl.top_k + 4
    h = Harness(wl, R.MOE_MODE_OFFLOAD, n_slots=n0, flags=R.MOE_FLAG_DEVICE_FILLS)
    b = StepBuffers(wl, T)
    cache = oracle.ExpertCache(wl.n_layers, wl.n_experts, n0)
    b.load(wl, 0)
    run_step(R, h, b, None)
    torch.cuda.synchronize()
    check_against_oracle(wl, b, 0, cache, R.MOE_MODE_OFFLOAD, (0, 0), False)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="thread_local"):
        run_step(R, h, b, torch.cuda.current_stream().cuda_stream)
    sizes = {4: 2 * T * wl.top_k + 1, 8: 3 * T * wl.top_k}
    arena2 = torch.empty(max(sizes.values()) * h.S, dtype=torch.uint8, device="cuda") if new_arena else None
    for step in range(1, 12):
        if step in sizes:
            if arena2 is not None:
                R.expert_cache_resize(h.ctx, sizes[step], arena2, arena2.numel())
            else:
                R.expert_cache_resize(h.ctx, sizes[step])
            cache.resize(sizes[step])
            slot_of, key_of, stamp, _ = h.snapshot()
            assert np.array_equal(slot_of, cache.slot_of.astype(np.int32)) and np.array_equal(
                key_of, cache.key_of.astype(np.int32)) and np.array_equal(stamp, cache.stamp.astype(np.uint64))
        b.load(wl, step)
        g.replay()
        torch.cuda.synchronize()
        check_against_oracle(wl, b, step, cache, R.MOE_MODE_OFFLOAD, (0, 0), False)
    R.moe_sync(h.ctx)
    slot_of, key_of, stamp, counter = h.snapshot()
    assert np.array_equal(slot_of, cache.slot_of.astype(np.int32)) and counter == cache.counter
    assert np.array_equal(key_of, cache.key_of.astype(np.int32)) and np.array_equal(stamp, cache.stamp.astype(np.uint64))
    del g


def test_replay_after_shrink_below_capture_is_reported():
    """A step captured without a CPU branch (OFFLOAD, n_slots >= 2*T*k) replayed after a
    shrink that leaves too few slots: the lookup sends misses to the CPU, which the graph
    cannot run, and moe_sync reports it instead of returning silently short outputs."""
    import routed_expert_ffn_02_amd as R
    import torch
    wl, T = BF16, 1
    h = Harness(wl, R.MOE_MODE_OFFLOAD, n_slots=2 * T * wl.top_k + 2, flags=R.MOE_FLAG_DEVICE_FILLS)
    b = StepBuffers(wl, T)
    b.load(wl, 0)
    run_step(R, h, b, None)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="thread_local"):
        run_step(R, h, b, torch.cuda.current_stream().cuda_stream)
    R.moe_sync(h.ctx)
    R.expert_cache_resize(h.ctx, 1)
    for step in range(1, 4):
        b.load(wl, step)
        g.replay()
    torch.cuda.synchronize()
    with pytest.raises(R.MoeError) as e:
        R.moe_sync(h.ctx)
    assert e.value.status == R.MOE_ESTATE
    R.moe_sync(h.ctx)  # reported once
    del g


def test_expired_cpu_branch_wait_is_reported(monkeypatch):
    """A captured HYBRID step whose CPU branch answers after the wait bound (the branch
    thread is told to answer 100 ms late, the bound is 50 us): the wait kernel gives up and
    ends, the step's CPU experts are left out, and moe_sync reports MOE_ETIMEDOUT once.  With
    the bound raised, the following replays match the oracle again."""
    import routed_expert_ffn_02_amd as R
    import torch
    wl, T = BF16, 1
    bw = (25_000_000_000, 100_000_000_000)
    monkeypatch.setenv("RMOE_CPU_BRANCH_DELAY_US", "100000")  # read when the branch thread starts
    h = Harness(wl, R.MOE_MODE_HYBRID, n_slots=wl.top_k + 1, flags=R.MOE_FLAG_DEVICE_FILLS, bw=bw)
    b = StepBuffers(wl, T)
    cache = oracle.ExpertCache(wl.n_layers, wl.n_experts, h.n_slots)
    b.load(wl, 0)
    run_step(R, h, b, None)
    torch.cuda.synchronize()
    check_against_oracle(wl, b, 0, cache, R.MOE_MODE_HYBRID, bw, False)
    R.moe_set_cpu_wait(h.ctx, 0.05)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="thread_local"):
        run_step(R, h, b, torch.cuda.current_stream().cuda_stream)
    step, expired = 0, False
    while step < 6 and not expired:
        step += 1
        b.load(wl, step)
        g.replay()
        torch.cuda.synchronize()
        _, idx, _, _, cnt, _ = b.outputs()
        for l in range(wl.n_layers):  # the tables advance on the device all the same
            cache.lookup(l, idx[l], R.MOE_MODE_HYBRID, *bw)
        if int(cnt[:, 2].sum()) > 0:  # a step with CPU work
            with pytest.raises(R.MoeError) as e:
                R.moe_sync(h.ctx)
            assert e.value.status == R.MOE_ETIMEDOUT
            expired = True
        else:
            R.moe_sync(h.ctx)
    assert expired, "no replayed step sent experts to the CPU"
    R.moe_sync(h.ctx)  # reported once
    R.moe_set_cpu_wait(h.ctx, 5000.0)
    for step in range(step + 1, step + 3):
        b.load(wl, step)
        g.replay()
        torch.cuda.synchronize()
        check_against_oracle(wl, b, step, cache, R.MOE_MODE_HYBRID, bw, False)
    R.moe_sync(h.ctx)
    del g
