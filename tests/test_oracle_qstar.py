"""Pins for the q* split (oracle/qstar.py) against what the pages fix."""
import json
import os
import random
from fractions import Fraction

import pytest

from oracle import qstar_split, qstar_real, MODE_HYBRID, MODE_OFFLOAD, MODE_CPU, MODE_FUSED

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_fig2_worked_example():
    g = _load("fig2_worked_example.json")
    bp, bh = g["bw_ratio_pcie_to_host"]
    q = qstar_split(g["misses"], bp, bh, MODE_HYBRID, evictable=1000)
    assert q == g["fills"]
    assert g["misses"] - q == g["cpu"]
    # the same ratio at realistic byte rates
    assert qstar_split(4, 25_000_000_000, 100_000_000_000, MODE_HYBRID, 1000) == 1


def test_balance_identity_real_valued():
    """q* = m B_P / B_H makes T_fill(q) = q S / B_P equal T_cpu(m-q) = (m-q) S / (B_H - B_P)."""
    rnd = random.Random(7)
    for _ in range(200):
        bp = rnd.randint(1, 10**11)
        bh = bp + rnd.randint(1, 10**11)
        m = rnd.randint(1, 64)
        S = rnd.randint(1, 10**8)
        q = Fraction(m * bp, bh)                       # exact q*
        t_fill = q * S / bp
        t_cpu = (m - q) * S / (bh - bp)
        assert t_fill == t_cpu
        assert abs(qstar_real(m, bp, bh) - float(q)) <= 1e-9 * m


def test_limit_bh_to_bp_is_pure_fill():
    """As B_H approaches B_P, q* approaches m; at or below it every miss is filled."""
    for m in range(1, 40):
        assert qstar_split(m, 50, 50, MODE_HYBRID, 10**6) == m
        assert qstar_split(m, 60, 50, MODE_HYBRID, 10**6) == m
        near = qstar_split(m, 10**9 - 1, 10**9, MODE_HYBRID, 10**6)
        assert near == m


def test_rounding_and_at_least_one_fill():
    for m in range(1, 33):
        for bp, bh in [(1, 4), (1, 3), (2, 7), (11, 47), (1, 100)]:
            q = qstar_split(m, bp, bh, MODE_HYBRID, 10**6)
            exact = Fraction(m * bp, bh)
            assert q >= 1
            if exact >= Fraction(1, 2):
                assert abs(Fraction(q) - exact) <= Fraction(1, 2)
            else:
                assert q == 1


def test_table1_profiles_split_properties():
    tab = _load("table1_bandwidths.json")
    for sysd in tab["systems"]:
        bp = int(round(sysd["bw_pcie"] * 1e9))
        bh = int(round(sysd["bw_host"] * 1e9))
        prev = 0
        for m in range(1, 17):
            q = qstar_split(m, bp, bh, MODE_HYBRID, 10**6)
            assert 1 <= q <= m
            assert q >= prev            # monotone in m
            prev = q
            assert abs(q - m * bp / bh) <= 0.5 or q == 1
        # the 4060 laptop (1:4.0) and PRO 6000 (1:3.5) send most misses to the CPU
    lap = next(s for s in tab["systems"] if s["name"] == "4060 laptop")
    assert qstar_split(4, int(lap["bw_pcie"] * 1e9), int(lap["bw_host"] * 1e9), MODE_HYBRID, 99) == 1


def test_modes_and_edges():
    assert qstar_split(0, 1, 4, MODE_HYBRID, 10) == 0
    assert qstar_split(5, 1, 4, MODE_HYBRID, 0) == 0           # nothing evictable
    assert qstar_split(9, 1, 1, MODE_HYBRID, 3) == 3            # capped by evictable
    assert qstar_split(7, 1, 4, MODE_OFFLOAD, 5) == 5
    assert qstar_split(7, 1, 4, MODE_CPU, 5) == 0
    assert qstar_split(7, 1, 4, MODE_FUSED, 5) == 0
    with pytest.raises(ValueError):
        qstar_split(-1, 1, 4, MODE_HYBRID, 5)
