"""Layer- and run-level oracle: route -> cache lookup -> expert FFN -> combine.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Outputs: the method reaches exactly the plain top-k SwiGLU MoE result (the
merge is exact and GPU memory never changes correctness: [FT-KR]
"측정된 대역폭이 분할을 결정합니다" and "탄력적 메모리 관리"), so the output
oracle is the all-resident definition; the cache oracle runs beside it to
produce the traces, slot ids and fill / CPU lists the GPU must reproduce.
"""
import numpy as np

from .formats import expert_weights_f64, activations_f64
from .router import router_logits, route
from .cache import ExpertCache
from .ffn import moe_layer_dense, moe_combine
from .qstar import MODE_FUSED, MODE_CPU


class OracleMoE:
    """Oracle for one workload (workloads.Workload)."""

    def __init__(self, workload, n_slots=None, mode=MODE_FUSED, bw_pcie=0, bw_host=0, weight_cache=True):
        self.w = workload
        self.mode = mode
        self.bw_pcie, self.bw_host = int(bw_pcie), int(bw_host)
        self.cache = ExpertCache(workload.n_layers, workload.n_experts,
                                 workload.n_slots if n_slots is None else n_slots)
        self._wcache = {} if weight_cache else None
        self._router = {}

    # -- inputs ------------------------------------------------------------
    def weights(self, key):
        if self._wcache is None:
            return expert_weights_f64(self.w, key)
        if key not in self._wcache:
            self._wcache[key] = expert_weights_f64(self.w, key)
        return self._wcache[key]

    def router(self, layer):
        if layer not in self._router:
            self._router[layer] = self.w.router_weight(layer)
        return self._router[layer]

    # -- one layer -----------------------------------------------------------
    def route(self, layer, x, bias=None):
        """x: workload activations [T,H] -> (logits fp32, idx, w)."""
        z = router_logits(activations_f64(x), self.router(layer), bias)
        idx, w = route(z, self.w.top_k, self.w.renorm)
        return z, idx, w

    def expert_outputs(self, layer, x, idx):
        E = self.w.n_experts
        return moe_layer_dense(activations_f64(x), idx,
                               lambda e: self.weights(layer * E + e))

    def decode_layer(self, layer, x, bias=None, idx=None, w=None):
        """One decode layer step.  Returns dict(logits, idx, w, lookup, y, y_gpu, y_cpu)."""
        z = None
        if idx is None:
            z, idx, w = self.route(layer, x, bias)
        lk = self.cache.lookup(layer, idx, self.mode, self.bw_pcie, self.bw_host)
        outs = self.expert_outputs(layer, x, idx)
        y = moe_combine(outs, w)
        on_cpu = lk.slot_idx < 0
        y_gpu = moe_combine(outs, w, ~on_cpu)
        y_cpu = moe_combine(outs, w, on_cpu)
        return dict(logits=z, idx=idx, w=w, lookup=lk, y=y.astype(np.float32),
                    y_exact=y, y_split=(y_gpu + y_cpu))

    def prefill_layer(self, layer, x, bias=None):
        """One prefill layer.  Returns dict(logits, idx, w, lookups, y)."""
        z, idx, w = self.route(layer, x, bias)
        if self.mode == MODE_FUSED:
            lks = [self.cache.lookup(layer, idx, MODE_FUSED)]
        elif self.mode == MODE_CPU:
            lks = [self.cache.lookup(layer, idx, MODE_CPU)]
        elif self.cache.buffers_active():
            lks = [self.cache.prefill_buffer_lookup(layer, idx)]
        else:
            lks = self.cache.prefill_ondemand(layer, idx)
        outs = self.expert_outputs(layer, x, idx)
        y = moe_combine(outs, w)
        return dict(logits=z, idx=idx, w=w, lookups=lks, y=y.astype(np.float32), y_exact=y)

    # -- decode chain with the previous-token locality bonus ---------------
    def decode_bias(self, layer, prev_idx, tokens):
        """Per-token logit bias: Zipf popularity plus prev_bonus on the previous step's experts."""
        b = np.tile(self.w.zipf_bias(layer), (tokens, 1)).astype(np.float32)
        if prev_idx is not None and self.w.prev_bonus != 0.0:
            for t in range(tokens):
                b[t, prev_idx[t]] = b[t, prev_idx[t]] + np.float32(self.w.prev_bonus)
        return b
