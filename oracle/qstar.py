"""The q* split of the miss set between cache fills and CPU execution.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[FT-KR] "측정된 대역폭이 분할을 결정합니다" and [FT-CN] 04 Design, mechanism 2:
the m distinct missed experts split into fills F (q = |F|, PCIe at B_P) and
CPU execution C.  A saturated PCIe transfer leaves B_R = max(B_H - B_P, 0) of
host bandwidth; T_fill(q) = qS/B_P and T_cpu(m-q) = (m-q)S/(B_H - B_P);
balancing them gives q/(m-q) = B_P/(B_H - B_P), i.e. q* = m B_P / B_H.  As
B_H approaches B_P, q* approaches m (pure on-demand fill).  q* is rounded to
an integer and at least one fill is kept so the cache keeps warming.

Readings (not fixed by the pages): rounding is half-up in exact integer
arithmetic; "at least one fill" applies only when there is a miss and an
evictable slot; fills beyond the evictable slots go to the CPU; with
B_H <= B_P there is no residual host bandwidth, so every miss is filled.
Parity: pinned by the Figure 2 worked example (m=4, B_P:B_H = 1:4 -> 1 fill,
3 CPU), the B_H -> B_P limit, the real-valued balance identity and Table 1.
"""
from fractions import Fraction

MODE_FUSED, MODE_OFFLOAD, MODE_CPU, MODE_HYBRID = 0, 1, 2, 3


def qstar_real(m: int, bw_pcie: float, bw_host: float) -> float:
    """The real-valued balance point q* = m * B_P / B_H (equations of the q* section)."""
    return m * bw_pcie / bw_host


def qstar_split(m: int, bw_pcie: int, bw_host: int, mode: int, evictable: int) -> int:
    """Number of misses to fill (the rest run on the CPU); bandwidths are integer bytes/s."""
    if m < 0 or evictable < 0:
        raise ValueError("negative count")
    if mode == MODE_FUSED:
        return 0
    if mode == MODE_CPU:
        return 0
    cap = min(m, evictable)
    if mode == MODE_OFFLOAD:
        return cap
    if mode != MODE_HYBRID:
        raise ValueError("unknown mode")
    if m == 0 or evictable == 0:
        return 0
    if bw_host <= bw_pcie:
        return cap
    # round-half-up of m * B_P / B_H, exactly
    q = int(Fraction(m * bw_pcie, bw_host) + Fraction(1, 2))
    return min(cap, max(1, q))
