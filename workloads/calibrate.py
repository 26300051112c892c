"""Calibrate the synthetic routing locality against the pages' miss-rate band.

Writes workloads/calibration.json.  Calls only the oracle (routing and the LRU
cache) on inputs from this package; nothing comes from the GPU path.

Targets (FreeToken summary, "무엇이 성능을 만들었나", expert-locality paragraph):
the global LRU misses 39% of decode-time expert reads at 11% of the
DeepSeek-V4-Flash pool and 16% at 37% of the Qwen3.6 pool, on replayed agent
traces.  The A3B-shaped decode workload keeps 12.5% of the pool resident, so
the rule is: among settings whose 4096-token prompt routes to at least 95% of a
layer's experts (prefill "activates nearly the whole expert set"), take the
one whose steady-state miss rate (after the cold fill) is closest to 39%.

    python -m workloads.calibrate
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))

import oracle  # noqa: E402
import workloads as W  # noqa: E402

ALPHAS = (0.25, 0.5, 0.75)
BONUSES = (0.0, 0.25, 0.5, 0.75, 1.0)
TARGET = 0.39
MIN_COVERAGE = 0.95
STEPS, WARM = 160, 32


def coverage(wl, T=4096, layer=0):
    orc = oracle.OracleMoE(wl)
    x = oracle.formats.activations_f64(wl.prefill_activations(layer, T))
    z = oracle.router_logits(x, orc.router(layer), np.tile(wl.zipf_bias(layer), (T, 1)))
    idx, _ = oracle.route(z, wl.top_k)
    return len(np.unique(idx)) / wl.n_experts


def steady_miss_rate(wl, steps=STEPS, warm=WARM):
    """Miss rate of the oracle's shared LRU cache over decode steps [warm, steps).

    Routing only: the expert outputs do not feed back into the routing."""
    orc = oracle.OracleMoE(wl, mode=oracle.MODE_OFFLOAD)
    prev = {}
    miss = tot = 0
    for s in range(steps):
        for layer in range(wl.n_layers):
            _, idx, _ = orc.route(layer, wl.decode_activations(s, layer, 1), orc.decode_bias(layer, prev.get(layer), 1))
            prev[layer] = idx
            c = orc.cache.lookup(layer, idx, oracle.MODE_OFFLOAD).counts
            if s >= warm:
                miss += c[1] + c[2]
                tot += c[0] + c[1] + c[2]
    return miss / tot


def main():
    rows = []
    for a in ALPHAS:
        cov = coverage(W.A3B_DECODE.with_(zipf_alpha=a, prev_bonus=0.0))
        for b in BONUSES:
            mr = steady_miss_rate(W.A3B_DECODE.with_(zipf_alpha=a, prev_bonus=b))
            rows.append({"zipf_alpha": a, "prev_bonus": b, "prefill_coverage": cov, "miss_rate": round(mr, 4)})
            print(rows[-1], flush=True)
    ok = [r for r in rows if r["prefill_coverage"] >= MIN_COVERAGE]
    best = min(ok, key=lambda r: (abs(r["miss_rate"] - TARGET), r["prev_bonus"]))
    out = {"rule": f"coverage >= {MIN_COVERAGE}, steady-state miss rate closest to {TARGET} at 1280 slots",
           "chosen": best, "grid": rows, "steps": STEPS, "warm": WARM}
    with open(os.path.join(HERE, "calibration.json"), "w") as f:
        json.dump(out, f, indent=1)
    print("chosen", best)


if __name__ == "__main__":
    main()
