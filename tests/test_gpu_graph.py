"""GPU: a whole decode step (route + lookup + decode of every layer) captured into one
HIP graph and replayed must reproduce eager execution bit for bit, replay after replay,
with the cache state advancing on the device.  Two paths qualify: OFFLOAD with device
fills, and FUSED."""
import numpy as np
import pytest

import workloads as W
from moe_harness import Harness

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
        return [t.cpu().numpy().copy() for t in (self.y, self.idx, self.slot, self.trace, self.cnt)]


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
    elif mode == "hybrid_device_fills":  # few slots: the CPU branch runs as host nodes
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
    # step 0 eagerly on both
    be.load(wl, 0)
    bg.load(wl, 0)
    run_step(R, eager, be, None, lc)
    run_step(R, graph, bg, None, lc)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    # thread-local capture: only this thread's calls are checked against the capture
    # (host nodes and the CPU worker pool run on threads of their own)
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
        for a, b_, name in zip(bg.outputs(), be.outputs(), ("y", "idx", "slot", "trace", "cnt")):
            assert np.array_equal(a.view(np.uint8), b_.view(np.uint8)), (step, name)
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
