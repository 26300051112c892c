"""The pool check for the f16 prefill (no GPU needed): every bf16 and E8M0 scale value
against the definition it implements (every nonzero weight e2m1(code) x scale of the
block within f16's normal range), the seeded generators' pools, and argument errors."""
import numpy as np
import pytest

import workloads as W

E2M1 = np.array([0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])  # nonzero magnitudes
F16_MIN_NORMAL, F16_MAX = 2.0 ** -14, 65504.0


def _cfg(R, wfmt, hidden=64, inter=32):
    return R.make_config(1, 1, 1, hidden, inter, wfmt, R.MOE_AFMT_BF16, 1, R.MOE_MODE_OFFLOAD)


def _in_range(s):
    if s == 0.0:
        return True
    if not np.isfinite(s):
        return False
    w = E2M1 * abs(s)
    return bool(np.all((w >= F16_MIN_NORMAL) & (w <= F16_MAX)))


def test_every_bf16_scale_against_the_definition():
    import routed_expert_ffn_02_amd as R
    cfg = _cfg(R, R.MOE_WFMT_FP4)
    S = R.moe_record_bytes(cfg)
    n = 64 * 32
    rec = np.zeros(S, np.uint8)
    scales = rec[3 * (n // 2):].view(np.uint16)
    bits = np.arange(1 << 16, dtype=np.uint32)
    with np.errstate(invalid="ignore"):  # NaN patterns
        values = (bits << 16).view(np.float32).astype(np.float64)
    got = np.empty(1 << 16, bool)
    for b in range(1 << 16):
        scales[5] = b  # one scale of the gate tensor; the others are zero (in range)
        got[b] = R.moe_pool_check_f16(cfg, rec.ctypes.data, 1) == -1
    want = np.array([_in_range(v) for v in values])
    assert np.array_equal(got, want), np.nonzero(got != want)[0][:10]
    # the bounds the header states
    for v, ok in [(10880.0, True), (10944.0, False), (2.0 ** -13, True), (-10880.0, True), (0.0, True)]:
        assert _in_range(v) == ok


def test_every_e8m0_scale_against_the_definition():
    import routed_expert_ffn_02_amd as R
    cfg = _cfg(R, R.MOE_WFMT_MXFP4)
    S = R.moe_record_bytes(cfg)
    n = 64 * 32
    rec = np.full(S, 127, np.uint8)  # codes don't matter; every scale 2^0
    for e in range(256):
        rec[3 * (n // 2) + 70] = e  # a scale of the down tensor
        want = e != 255 and _in_range(2.0 ** (e - 127))
        assert (R.moe_pool_check_f16(cfg, rec.ctypes.data, 1) == -1) == want, e
    assert [e for e in range(256) if e != 255 and _in_range(2.0 ** (e - 127))] == list(range(114, 141))


def test_first_failing_record_and_other_formats():
    import routed_expert_ffn_02_amd as R
    cfg = _cfg(R, R.MOE_WFMT_FP4)
    S = R.moe_record_bytes(cfg)
    n = 64 * 32
    pool = np.zeros(9 * S, np.uint8)
    for r in (7, 4):
        pool[r * S + 3 * (n // 2):(r + 1) * S].view(np.uint16)[-1] = 0x7F80  # +inf, the last scale
    assert R.moe_pool_check_f16(cfg, pool.ctypes.data, 9) == 4
    assert R.moe_pool_check_f16(cfg, pool.ctypes.data, 4) == -1
    assert R.moe_pool_check_f16(cfg, pool.ctypes.data, 0) == -1
    for wfmt in (R.MOE_WFMT_F32, R.MOE_WFMT_BF16):  # no block scales: nothing to check
        c = _cfg(R, wfmt)
        assert R.moe_pool_check_f16(c, np.zeros(R.moe_record_bytes(c), np.uint8).ctypes.data, 1) == -1
    with pytest.raises(R.MoeError):
        R.moe_pool_check_f16(cfg, pool.ctypes.data, -1)


@pytest.mark.parametrize("wl", [W.DSV4, W.DSV4_MX], ids=["fp4", "mxfp4"])
def test_generated_pools_pass(wl):
    """The seeded generators keep every nonzero weight in f16's normal range (the reading
    the f16 prefill relies on), so their pools pass."""
    import routed_expert_ffn_02_amd as R
    small = wl.with_(name=wl.name + "_chk", n_layers=2, n_experts=4, hidden=512, inter=256, alias_records=0)
    cfg = R.make_config(small.n_layers, small.n_experts, small.top_k, small.hidden, small.inter, small.wfmt,
                        small.afmt, 1, R.MOE_MODE_OFFLOAD)
    buf = np.empty(small.pool_records * small.record_bytes, np.uint8)
    small.fill_pool(buf.ctypes.data, 0, small.pool_records)
    assert R.moe_pool_check_f16(cfg, buf.ctypes.data, small.pool_records) == -1
