"""Decode-time expert miss rate of GPU placement policies replayed on one routing trace.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix (FreeToken summary, "무엇이 성능을 만들었나", the expert-locality
paragraph, and the reading notes, Figure 4b): the same routing trace is replayed
against several placement policies at the same cache capacity, and the figure of
merit is the fraction of decode-time expert reads that miss the GPU.  The policies
compared there are FreeToken's global LRU over all layers, KTransformers' placement
updated at prefill time, and llama.cpp's routing-blind static split; the Luce Spark
post adds a placement pinned from measured routing frequencies plus a bounded ring of
spare slots evicted LRU-first.

Readings of what the pages leave open (each listed in the design notes):
 * A decode read is one routed (token, rank) pair at one layer; a step's pairs are
   deduplicated into U (first-appearance order), and a key of U misses when it is not
   resident when the layer step begins.  Miss rate = missed keys / keys of U, summed
   over every (step, layer); at batch 1 the k experts of a token are distinct, so this
   is the fraction of reads.
 * LRU: exactly the shared cache of the hot path in offload mode (every miss filled,
   victims the least recently used slots holding no hit of the step), from a cold,
   empty cache.
 * Prefill update: the C keys most often routed by the prompt (ties to the lower key)
   are resident for the whole decode; decode misses are not admitted.
 * Static split: llama.cpp keeps the experts of the first layers on the CPU, so the
   GPU holds whole layers from the top: layers L - C // E .. L - 1, and the remaining
   C % E slots hold experts 0 .. C % E - 1 of the layer below them.
 * Pinned ring: R slots per layer form an LRU ring (R = ring_per_layer); the other
   C - L R slots pin the keys most often routed by the prompt (the calibration trace),
   ties to the lower key.  A miss of an unpinned key is filled into its layer's ring,
   evicting the least recently used entry that is not a hit of the same step (empty
   slots first, lowest slot first); with no such entry the miss is not admitted.
Parity: LRU is the oracle cache (itself pinned against an explicit MRU list); the
other policies are pinned against brute-force set computations and closed forms in
the tests.
"""
from __future__ import annotations

from typing import Dict, List, Sequence

import numpy as np

from .cache import ExpertCache, unique_first_appearance
from .qstar import MODE_OFFLOAD

POLICY_LRU, POLICY_PREFILL, POLICY_STATIC, POLICY_PINNED_RING = 0, 1, 2, 3


def routing_counts(calib: np.ndarray, n_layers: int, n_experts: int) -> np.ndarray:
    """How often each key l*E + e is routed by a calibration trace [tokens, L, k]."""
    calib = np.asarray(calib, dtype=np.int64)
    counts = np.zeros(n_layers * n_experts, np.int64)
    for l in range(n_layers):
        for e in calib[:, l, :].reshape(-1).tolist():
            counts[l * n_experts + e] += 1
    return counts


def top_keys(counts: np.ndarray, c: int) -> List[int]:
    """The c keys with the largest counts, ties to the lower key."""
    order = sorted(range(len(counts)), key=lambda key: (-int(counts[key]), key))
    return order[:max(0, c)]


def static_resident(n_layers: int, n_experts: int, capacity: int) -> set:
    """Whole layers from the top, then the first experts of the layer below."""
    capacity = max(0, min(capacity, n_layers * n_experts))
    full, rest = divmod(capacity, n_experts)
    keys = set()
    for l in range(n_layers - full, n_layers):
        keys.update(range(l * n_experts, (l + 1) * n_experts))
    if rest:
        l = n_layers - full - 1
        keys.update(range(l * n_experts, l * n_experts + rest))
    return keys


class _Ring:
    """One layer's LRU ring as an explicit most-recent-first list of slot contents."""

    def __init__(self, n: int):
        self.n = n
        self.keys: List[int] = []   # resident keys, most recent first

    def step(self, U_unpinned: Sequence[int]) -> List[bool]:
        """Classify then update: hits refresh, misses fill the LRU-most non-hit entries."""
        hit = [u in self.keys for u in U_unpinned]
        hitset = {u for u, h in zip(U_unpinned, hit) if h}
        misses = [u for u, h in zip(U_unpinned, hit) if not h]
        # victims: empty slots first, then resident keys from the least recent end,
        # skipping this step's hits
        free = self.n - len(self.keys)
        evictable = [kk for kk in reversed(self.keys) if kk not in hitset]
        admitted = misses[:free + len(evictable)]
        n_evict = max(0, len(admitted) - free)
        for kk in evictable[:n_evict]:
            self.keys.remove(kk)
        # every key of U that is a hit or was admitted moves to the front in U order
        admitted_set = set(admitted)
        for u in U_unpinned:
            if u in hitset or u in admitted_set:
                if u in self.keys:
                    self.keys.remove(u)
                self.keys.insert(0, u)
        return hit


def replay(policy: int, n_layers: int, n_experts: int, capacity: int, decode: np.ndarray,
           calib: np.ndarray = None, ring_per_layer: int = 0) -> Dict[str, object]:
    """Replay a decode trace [steps, L, T*k] (expert ids, token-major then rank).

    Returns keys (distinct keys over all layer steps), misses, and miss[s][l] = the
    miss flag of each key of that step's U, in U order.
    """
    decode = np.asarray(decode, dtype=np.int64)
    steps, L, _ = decode.shape
    assert L == n_layers
    E = n_experts
    flags = []
    n_keys = n_miss = 0
    if policy == POLICY_LRU:
        cache = ExpertCache(L, E, capacity) if capacity > 0 else None
    elif policy == POLICY_PREFILL:
        resident = set(top_keys(routing_counts(calib, L, E), capacity))
    elif policy == POLICY_STATIC:
        resident = static_resident(L, E, capacity)
    elif policy == POLICY_PINNED_RING:
        R = ring_per_layer
        assert R >= 0 and capacity >= L * R
        pinned = set(top_keys(routing_counts(calib, L, E), capacity - L * R))
        rings = [_Ring(R) for _ in range(L)]
    else:
        raise ValueError(policy)
    for s in range(steps):
        per_layer = []
        for l in range(L):
            keys = l * E + decode[s, l]
            U = unique_first_appearance(keys)
            if policy == POLICY_LRU:
                if cache is None:
                    miss = [True] * len(U)
                else:
                    res = cache.lookup(l, decode[s, l].reshape(1, -1), MODE_OFFLOAD)
                    kinds = {key: kind for key, kind, _, _ in res.trace}
                    miss = [kinds[u] != 0 for u in U]
            elif policy in (POLICY_PREFILL, POLICY_STATIC):
                miss = [u not in resident for u in U]
            else:
                unpinned = [u for u in U if u not in pinned]
                ring_hit = dict(zip(unpinned, rings[l].step(unpinned))) if rings[l].n else {u: False for u in unpinned}
                miss = [False if u in pinned else not ring_hit[u] for u in U]
            per_layer.append(miss)
            n_keys += len(U)
            n_miss += sum(miss)
        flags.append(per_layer)
    return {"keys": n_keys, "misses": n_miss, "miss": flags}
