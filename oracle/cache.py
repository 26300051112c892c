"""The bounded GPU expert cache shared by all MoE layers, with LRU replacement.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix:
 * One cache of complete expert slots serves every MoE layer; residency,
   lookup and execution use the logical (layer, expert) id, flattened to
   key = layer*E + expert ([FT-KR] "FreeToken의 설계", "전문가 뱅크와 FTW 포맷").
 * A hit refreshes recency, a fill admits the newly selected expert, and
   eviction removes the expert least recently demanded ([FT-KR] "라우터를
   따라 움직이는 LRU 캐시").  CPU-executed misses leave residency unchanged
   ([FT-KR] "측정된 대역폭이 분할을 결정합니다").
 * Per layer, one device-side step dedupes the routed experts, classifies
   them against the residency table, derives q, selects victims, and
   rewrites logical ids to slot ids or CPU flags; victim search finds K
   candidates in one pass and the miss path takes the first q <= K
   ([FT-KR] "CUDA Graph와 공존하는 LRU 캐시"; [FT-CN] 05 Implementation).
 * Prefill reserves two full-layer buffers from the same slot pool; layer
   l+1 is loaded whole while layer l computes; entries surviving prefill seed
   decode; if the pool cannot spare two full layers, prefill loads on demand
   ([FT-KR] "전층 이중 버퍼링"; [FT-CN] 04 Design, mechanism 1).
 * The cache can be rebuilt for a new budget at a safe point without
   reloading the host pool ([FT-KR] "탄력적 메모리 관리").

Readings of what the pages leave open (each listed in the design notes):
 * U, the distinct routed keys, is taken in first-appearance order over
   (token, rank) pairs; F = the first q misses of U.
 * Recency is a per-access stamp from one global counter; after victims are
   chosen, every key of U in H or F gets the next stamp in U order.
 * Victims: the q slots with the smallest (stamp, slot) among slots that hold
   no hit of this step and are not reserved; empty slots have stamp 0.
 * Prefill buffers are slots [0, E) and [E, 2E); layer l uses buffer l % 2
   at slot base + expert.  At prefill end the last layer held in each buffer
   is admitted (lower layer first, experts ascending), replacing any older
   copy of the same key.
 * On-demand prefill: rounds of the offload lookup; a round's leftover misses
   wait for the next round, in which every slot is evictable again.
 * Resize: shrinking keeps the N' most recent entries packed into slots
   0..N'-1 in ascending old-slot order with stamps kept; growing adds empty
   slots at the end.
Parity: the stamp form is pinned against NaiveListCache (an explicit
MRU->LRU list) on random traces, and against first-touch and repeat-step
closed cases.
"""
from dataclasses import dataclass, field
from typing import List, Tuple

import numpy as np

from .qstar import MODE_FUSED, MODE_OFFLOAD, MODE_CPU, MODE_HYBRID, qstar_split

KIND_HIT, KIND_FILL, KIND_CPU, KIND_BUF = 0, 1, 2, 3


@dataclass
class LookupResult:
    slot_idx: np.ndarray                 # [T,k] int32: slot >= 0, or -1-c for CPU list entry c
    trace: List[Tuple[int, int, int, int]]   # per key of U: (key, kind, slot or -1, evicted key or -1)
    fills: List[Tuple[int, int]]         # (key, slot) in U order
    cpu: List[int]                       # keys in U order
    counts: Tuple[int, int, int, int]    # (n_hit, n_fill, n_cpu, n_evict)


def unique_first_appearance(keys_tk: np.ndarray) -> List[int]:
    """Distinct keys of a [T,k] array walked token-major then rank, in first-appearance order."""
    seen, out = set(), []
    for kk in np.asarray(keys_tk).reshape(-1).tolist():
        if kk not in seen:
            seen.add(kk)
            out.append(kk)
    return out


class ExpertCache:
    """Timestamp form of the shared LRU expert cache (the form the GPU implements)."""

    def __init__(self, n_layers: int, n_experts: int, n_slots: int):
        self.L, self.E = n_layers, n_experts
        self.n_slots = n_slots
        self.slot_of = np.full(n_layers * n_experts, -1, np.int64)
        self.key_of = np.full(n_slots, -1, np.int64)
        self.stamp = np.zeros(n_slots, np.int64)
        self.reserved = np.zeros(n_slots, bool)
        self.counter = 0
        self.in_prefill = False
        self.buffer_layer = [-1, -1]

    # -- helpers ---------------------------------------------------------
    def _next(self) -> int:
        self.counter += 1
        return self.counter

    def _evict_slot(self, s: int) -> int:
        old = int(self.key_of[s])
        if old >= 0:
            self.slot_of[old] = -1
        self.key_of[s] = -1
        self.stamp[s] = 0
        return old

    def resident_keys(self):
        return {int(k): int(s) for s, k in enumerate(self.key_of) if k >= 0}

    # -- decode-step lookup ------------------------------------------------
    def lookup(self, layer: int, idx: np.ndarray, mode: int, bw_pcie: int = 0, bw_host: int = 0,
               candidates: List[int] = None) -> LookupResult:
        """One layer step of the cache-control kernel.

        idx: [T,k] expert ids of this layer in rank order.  `candidates`, when
        given, replaces U (used by the on-demand prefill rounds).
        """
        idx = np.asarray(idx, dtype=np.int64)
        keys = layer * self.E + idx
        U = unique_first_appearance(keys) if candidates is None else list(candidates)
        if mode == MODE_FUSED:
            trace = [(u, KIND_HIT, u, -1) for u in U]
            return LookupResult(keys.astype(np.int32), trace, [], [], (len(U), 0, 0, 0))
        hits = [u for u in U if self.slot_of[u] >= 0]
        hitset = set(hits)
        misses = [u for u in U if u not in hitset]
        m = len(misses)
        protected = {int(self.slot_of[u]) for u in hits}
        eligible = [s for s in range(self.n_slots) if s not in protected and not self.reserved[s]]
        q = qstar_split(m, bw_pcie, bw_host, mode, len(eligible))
        eligible.sort(key=lambda s: (int(self.stamp[s]), s))
        victims = eligible[:q]
        F, C = misses[:q], misses[q:]
        evicted = {}
        n_evict = 0
        for u, s in zip(F, victims):
            old = self._evict_slot(s)
            evicted[u] = old
            n_evict += old >= 0
            self.slot_of[u] = s
            self.key_of[s] = u
        Fset = set(F)
        for u in U:
            if u in hitset or u in Fset:
                self.stamp[self.slot_of[u]] = self._next()
        cpu_index = {u: c for c, u in enumerate(C)}
        trace = []
        for u in U:
            if u in hitset:
                trace.append((u, KIND_HIT, int(self.slot_of[u]), -1))
            elif u in Fset:
                trace.append((u, KIND_FILL, int(self.slot_of[u]), int(evicted[u])))
            else:
                trace.append((u, KIND_CPU, -1, -1))
        slot_idx = np.empty(keys.shape, np.int32)
        for pos, kk in np.ndenumerate(keys):
            kk = int(kk)
            if kk in cpu_index:
                slot_idx[pos] = -1 - cpu_index[kk]
            elif candidates is not None and kk not in hitset and kk not in Fset:
                slot_idx[pos] = -1 - len(C) - 1     # not part of this round (on-demand prefill)
            else:
                slot_idx[pos] = int(self.slot_of[kk])
        fills = [(u, int(self.slot_of[u])) for u in F]
        return LookupResult(slot_idx, trace, fills, list(C), (len(hits), q, len(C), n_evict))

    # -- prefill -----------------------------------------------------------
    def prefill_begin(self) -> bool:
        """Reserve slots [0, 2E) as the two full-layer buffers; False = on-demand fallback."""
        if self.n_slots < 2 * self.E:
            self.in_prefill = True
            self.buffer_layer = [-1, -1]
            return False
        for s in range(2 * self.E):
            self._evict_slot(s)
            self.reserved[s] = True
        self.in_prefill = True
        self.buffer_layer = [-1, -1]
        return True

    def buffers_active(self) -> bool:
        return bool(self.reserved[: 2 * self.E].all()) if self.n_slots >= 2 * self.E else False

    def prefill_buffer_lookup(self, layer: int, idx: np.ndarray) -> LookupResult:
        """Layer `layer` is held whole in buffer layer % 2: expert e sits at slot base + e."""
        b = layer % 2
        self.buffer_layer[b] = layer
        base = b * self.E
        idx = np.asarray(idx, dtype=np.int64)
        keys = layer * self.E + idx
        U = unique_first_appearance(keys)
        trace = [(u, KIND_BUF, base + (u - layer * self.E), -1) for u in U]
        return LookupResult((base + idx).astype(np.int32), trace, [], [], (len(U), 0, 0, 0))

    def prefill_ondemand(self, layer: int, idx: np.ndarray):
        """On-demand prefill rounds: list of LookupResult, one per round (offload semantics)."""
        keys = layer * self.E + np.asarray(idx, dtype=np.int64)
        pending = unique_first_appearance(keys)
        rounds = []
        while pending:
            if self.n_slots == 0:
                raise ValueError("on-demand prefill needs at least one slot")
            r = self.lookup(layer, idx, MODE_OFFLOAD, candidates=pending)
            done = {t[0] for t in r.trace if t[1] in (KIND_HIT, KIND_FILL)}
            # leftover misses are deferred, not CPU-executed: relabel them
            r.trace = [t if t[1] != KIND_CPU else (t[0], KIND_CPU, -1, -1) for t in r.trace]
            rounds.append(r)
            pending = [u for u in pending if u not in done]
        return rounds

    def prefill_end(self) -> None:
        """Buffers return to the pool; their entries survive to seed decode."""
        if self.buffers_active():
            held = sorted([(self.buffer_layer[b], b) for b in (0, 1) if self.buffer_layer[b] >= 0])
            for layer, b in held:
                base = b * self.E
                for e in range(self.E):
                    key = layer * self.E + e
                    old = int(self.slot_of[key])
                    if old >= 0:
                        self._evict_slot(old)
                    s = base + e
                    self.key_of[s] = key
                    self.slot_of[key] = s
                    self.stamp[s] = self._next()
            self.reserved[: 2 * self.E] = False
        self.in_prefill = False
        self.buffer_layer = [-1, -1]

    # -- elastic resize ----------------------------------------------------
    def resize(self, new_n_slots: int):
        """Rebuild for a new slot budget.  Returns [(old_slot, new_slot)] moves of surviving records."""
        if self.in_prefill:
            raise RuntimeError("resize inside prefill")
        occupied = [s for s in range(self.n_slots) if self.key_of[s] >= 0]
        if new_n_slots < self.n_slots:
            by_recency = sorted(occupied, key=lambda s: (-int(self.stamp[s]), s))
            keep = sorted(by_recency[:new_n_slots])
        else:
            keep = occupied
        moves = []
        key_of = np.full(new_n_slots, -1, np.int64)
        stamp = np.zeros(new_n_slots, np.int64)
        self.slot_of[:] = -1
        if new_n_slots < self.n_slots:
            for ns, s in enumerate(keep):
                key_of[ns] = self.key_of[s]
                stamp[ns] = self.stamp[s]
                moves.append((s, ns))
        else:
            for s in keep:
                key_of[s] = self.key_of[s]
                stamp[s] = self.stamp[s]
                moves.append((s, s))
        for s in range(new_n_slots):
            if key_of[s] >= 0:
                self.slot_of[key_of[s]] = s
        self.key_of, self.stamp = key_of, stamp
        self.reserved = np.zeros(new_n_slots, bool)
        self.n_slots = new_n_slots
        return moves


class NaiveListCache:
    """An explicit MRU->LRU list of resident keys plus a set of free slots.

    Independent restatement of the same policy used to pin ExpertCache: per
    step, victims are free slots (lowest first) then the least recently used
    entries not hit in this step; then each key of U in H or F moves to the
    MRU end in U order.
    """

    def __init__(self, n_slots: int):
        self.n_slots = n_slots
        self.order = []          # LRU first, MRU last: list of keys
        self.where = {}          # key -> slot
        self.free = list(range(n_slots))

    def step(self, keys_tk, mode, bw_pcie=0, bw_host=0):
        U = []
        for kk in np.asarray(keys_tk).reshape(-1).tolist():
            if kk not in U:
                U.append(kk)
        hits = [u for u in U if u in self.where]
        misses = [u for u in U if u not in self.where]
        hitset = set(hits)
        evictable_lru = [kk for kk in self.order if kk not in hitset]
        ev = len(self.free) + len(evictable_lru)
        q = qstar_split(len(misses), bw_pcie, bw_host, mode, ev)
        free_sorted = sorted(self.free)
        victims = []            # (slot, old key or -1)
        for s in free_sorted[:q]:
            victims.append((s, -1))
        for kk in evictable_lru[: q - len(victims)]:
            victims.append((self.where[kk], kk))
        F = misses[:q]
        out = []
        fills = {}
        for u, (s, old) in zip(F, victims):
            if old >= 0:
                self.order.remove(old)
                del self.where[old]
            else:
                self.free.remove(s)
            self.where[u] = s
            self.order.append(u)   # position fixed below
            fills[u] = (s, old)
        for u in U:
            if u in hitset or u in fills:
                self.order.remove(u)
                self.order.append(u)
        for u in U:
            if u in hitset:
                out.append((u, KIND_HIT, self.where[u], -1))
            elif u in fills:
                out.append((u, KIND_FILL, fills[u][0], fills[u][1]))
            else:
                out.append((u, KIND_CPU, -1, -1))
        return out

    def resize(self, new_n_slots):
        if new_n_slots < self.n_slots:
            keep_keys = self.order[-new_n_slots:] if new_n_slots > 0 else []
            keep = sorted((self.where[kk], kk) for kk in keep_keys)
            order_pos = {kk: i for i, kk in enumerate(self.order)}
            self.where = {kk: ns for ns, (s, kk) in enumerate(keep)}
            self.order = sorted(self.where, key=lambda kk: order_pos[kk])
            self.free = [s for s in range(new_n_slots) if s not in set(self.where.values())]
        else:
            self.free = self.free + list(range(self.n_slots, new_n_slots))
        self.n_slots = new_n_slots
