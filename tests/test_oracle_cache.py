"""Pins for the expert cache (oracle/cache.py): the stamp form equals an explicit LRU list."""
import numpy as np
import pytest

import workloads as W
from oracle import (ExpertCache, NaiveListCache, MODE_OFFLOAD, MODE_HYBRID, MODE_CPU,
                    KIND_HIT, KIND_FILL, KIND_CPU, KIND_BUF)


def _random_steps(rng, L, E, k, T, steps):
    out = []
    for s in range(steps):
        layer = int(rng.integers(0, L))
        idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
        out.append((layer, idx))
    return out


@pytest.mark.parametrize("seed", range(12))
def test_stamp_lru_equals_naive_list(seed):
    rng = np.random.default_rng(seed)
    L, E = int(rng.integers(1, 4)), int(rng.integers(4, 24))
    k = int(rng.integers(1, min(E, 6) + 1))
    T = int(rng.integers(1, 4))
    n_slots = int(rng.integers(0, L * E + 3))
    mode = [MODE_OFFLOAD, MODE_HYBRID, MODE_CPU][seed % 3]
    bp, bh = [(1, 4), (3, 5), (7, 2)][seed % 3]
    a, b = ExpertCache(L, E, n_slots), NaiveListCache(n_slots)
    for step, (layer, idx) in enumerate(_random_steps(rng, L, E, k, T, 60)):
        ra = a.lookup(layer, idx, mode, bp, bh)
        tb = b.step(layer * E + idx, mode, bp, bh)
        assert ra.trace == tb, f"step {step}"
        if step in (20, 40) and n_slots > 2:
            new = max(1, n_slots // 2) if step == 20 else n_slots + 3
            a.resize(new)
            b.resize(new)
            assert a.resident_keys() == dict(b.where)


def test_first_touch_when_everything_fits():
    rng = np.random.default_rng(3)
    L, E, k = 3, 16, 4
    c = ExpertCache(L, E, L * E)
    seen, misses = set(), 0
    for layer, idx in _random_steps(rng, L, E, k, 2, 80):
        r = c.lookup(layer, idx, MODE_OFFLOAD)
        keys = set((layer * E + idx).reshape(-1).tolist())
        assert r.counts[1] == len(keys - seen)
        assert r.counts[3] == 0
        seen |= keys


def test_repeated_step_hits_after_first():
    c = ExpertCache(2, 32, 8)
    idx = np.array([[3, 9, 1, 30]])
    r0 = c.lookup(1, idx, MODE_OFFLOAD)
    assert [t[1] for t in r0.trace] == [KIND_FILL] * 4
    for _ in range(5):
        r = c.lookup(1, idx, MODE_OFFLOAD)
        assert [t[1] for t in r.trace] == [KIND_HIT] * 4


def test_fig2_scenario_end_to_end():
    """8 of 12 routed experts resident, 4 misses, B_P:B_H = 1:4 -> 1 fill + 3 CPU."""
    E = 64
    c = ExpertCache(1, E, 12)
    c.lookup(0, np.arange(8).reshape(1, 8), MODE_OFFLOAD)       # make experts 0..7 resident
    idx = np.array([[0, 1, 2, 3, 4, 5, 6, 7, 40, 41, 42, 43]])
    r = c.lookup(0, idx, MODE_HYBRID, 1, 4)
    kinds = [t[1] for t in r.trace]
    assert kinds.count(KIND_HIT) == 8 and kinds.count(KIND_FILL) == 1 and kinds.count(KIND_CPU) == 3
    assert r.fills[0][0] == 40 and r.cpu == [41, 42, 43]
    assert r.slot_idx[0, 9:].tolist() == [-1, -2, -3]


def test_hits_never_evicted_and_victims_lru():
    c = ExpertCache(1, 10, 3)
    c.lookup(0, np.array([[0]]), MODE_OFFLOAD)
    c.lookup(0, np.array([[1]]), MODE_OFFLOAD)
    c.lookup(0, np.array([[2]]), MODE_OFFLOAD)
    r = c.lookup(0, np.array([[0, 5]]), MODE_OFFLOAD)   # 0 hits; victim must be 1 (LRU, not 0)
    assert r.trace[1][3] == 1
    r = c.lookup(0, np.array([[6, 7, 8, 9]]), MODE_OFFLOAD)   # only 3 slots: 3 fills, 1 CPU
    assert r.counts == (0, 3, 1, 3)


def test_prefill_buffers_and_seed_decode():
    L, E = 4, 8
    c = ExpertCache(L, E, 2 * E + 3)
    c.lookup(0, np.array([[1, 2]]), MODE_OFFLOAD)
    assert c.prefill_begin()
    for layer in range(L):
        r = c.prefill_buffer_lookup(layer, np.array([[5, 1], [1, 7]]))
        assert all(t[1] == KIND_BUF for t in r.trace)
        assert r.slot_idx.tolist() == [[(layer % 2) * E + 5, (layer % 2) * E + 1], [(layer % 2) * E + 1, (layer % 2) * E + 7]]
    c.prefill_end()
    res = c.resident_keys()
    for layer in (L - 2, L - 1):
        for e in range(E):
            assert res[layer * E + e] == (layer % 2) * E + e
    # the stamps order layer L-2 before L-1: layer L-2's expert 0 is the LRU entry
    occ = [(c.stamp[s], s) for s in range(c.n_slots) if c.key_of[s] >= 0]
    assert min(occ)[1] == ((L - 2) % 2) * E


def test_prefill_ondemand_rounds_cover_every_expert_once():
    L, E = 1, 8
    c = ExpertCache(L, E, 3)
    assert not c.prefill_begin()
    idx = np.array([[0, 1], [2, 3], [4, 5], [6, 7], [1, 2]])
    rounds = c.prefill_ondemand(0, idx)
    done = [t[0] for r in rounds for t in r.trace if t[1] in (KIND_HIT, KIND_FILL)]
    assert sorted(done) == list(range(8)) and len(rounds) == 3
    c.prefill_end()


def test_resize_keeps_most_recent_packed():
    c = ExpertCache(1, 20, 6)
    for e in [3, 4, 5, 6, 7, 8]:
        c.lookup(0, np.array([[e]]), MODE_OFFLOAD)
    c.lookup(0, np.array([[4]]), MODE_OFFLOAD)          # 4 becomes the most recent
    moves = c.resize(3)
    assert set(c.resident_keys()) == {4, 7, 8}
    assert moves == [(1, 0), (4, 1), (5, 2)]
    c.resize(5)
    assert set(c.resident_keys()) == {4, 7, 8} and c.n_slots == 5


def test_synthetic_routing_has_locality_and_distinct_experts():
    w = W.A3B_DECODE
    tr = w.synthetic_routing(40, layer=3, tokens=2)
    assert tr.shape == (40, 2, 8)
    for s in range(40):
        for t in range(2):
            assert len(set(tr[s, t].tolist())) == 8
    overlap = np.mean([len(set(tr[s, 0]) & set(tr[s - 1, 0])) for s in range(1, 40)])
    assert overlap > 3
