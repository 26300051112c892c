"""Pins of the MX-activation oracle (oracle/mx.py): the E4M3 table, the MXFP8 quantiser
and the MX expert FFN, each against something other than its own code."""
import json
import os

import numpy as np
import pytest

import oracle.mx as mx
from oracle.ffn import expert_ffn

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_ocp.json")


def test_e4m3_named_values():
    """The values the OCP 8-bit floating point specification names for E4M3 (golden file):
    smallest subnormal 2^-9, largest subnormal 0.875 * 2^-6, smallest normal 2^-6, one,
    largest normal 448, signed zero, NaN at S.1111.111 and nowhere else."""
    g = json.load(open(GOLDEN))
    for code, value in g["named"].items():
        got = mx.e4m3_decode(np.array([int(code, 16)]))[0]
        assert got == value and np.signbit(got) == np.signbit(value), code
    allv = mx.e4m3_decode(np.arange(256))
    nan = {int(c, 16) for c in g["nan_codes"]}
    assert {i for i in range(256) if np.isnan(allv[i])} == nan
    pos = allv[:0x7F]
    assert np.all(np.diff(pos) > 0)                       # monotone over the finite codes
    assert np.array_equal(allv[0x80:0xFF], -pos)          # sign symmetry


def _brute_codes(q):
    """Nearest finite E4M3 code by scanning all 254 of them; ties to the even code; clamp."""
    vals = mx.e4m3_decode(np.arange(256))
    finite = [c for c in range(256) if not np.isnan(vals[c])]
    out = np.empty(q.shape, np.int64)
    for idx, v in np.ndenumerate(q):
        v = float(np.clip(v, -448.0, 448.0))
        best = None
        for c in finite:
            if (vals[c] < 0) != (v < 0) and vals[c] != 0:
                continue
            d = abs(vals[c] - v)
            key = (d, c & 1)
            if best is None or key < best[0]:
                best = (key, c)
        out[idx] = best[1]
    return out


def test_quantiser_matches_brute_force():
    rng = np.random.default_rng(11)
    v = rng.normal(size=(6, 64)) * np.exp2(rng.integers(-12, 12, size=(6, 1)))
    v[0, :32] = 0.0                       # a block of zeros
    v[1, 5] = -0.0
    codes, scales = mx.mxfp8_quantize(v)
    amax = np.abs(v.reshape(6, 2, 32)).max(axis=2)
    for r in range(6):
        for b in range(2):
            s = -127 if amax[r, b] == 0 else int(np.floor(np.log2(amax[r, b]))) - 8
            assert scales[r, b] == s + 127
            q = v[r, 32 * b:32 * b + 32] / 2.0 ** s
            brute = _brute_codes(q)
            got = codes[r, 32 * b:32 * b + 32].astype(np.int64)
            # codes may differ only in the sign of a zero
            vals = mx.e4m3_decode(np.arange(256))
            assert np.array_equal(vals[got], vals[brute]), (r, b)


def test_scale_rule_closed_forms():
    base = np.zeros((1, 32))
    for k in (-20, -3, 0, 7):
        v = base.copy()
        v[0, 0] = 2.0 ** k                 # amax exactly 2^k -> s = k - 8, element 256
        v[0, 1] = 1.75 * 2.0 ** k * 0.999  # below the max: representable neighbourhood
        codes, scales = mx.mxfp8_quantize(v)
        assert scales[0, 0] == k - 8 + 127
        assert mx.e4m3_decode(codes[0, 0]) == 256.0
    v = base.copy()
    v[0, 0] = 1.9                           # 1.9 * 2^8 = 486.4 > 448: saturates
    codes, scales = mx.mxfp8_quantize(v)
    assert scales[0, 0] == 127 - 8 and mx.e4m3_decode(codes[0, 0]) == 448.0
    v[0, 0] = -1.9
    codes, _ = mx.mxfp8_quantize(v)
    assert mx.e4m3_decode(codes[0, 0]) == -448.0


def test_representable_blocks_round_trip():
    rng = np.random.default_rng(3)
    vals = mx.e4m3_decode(np.arange(0x7F))
    for s in (-30, -7, 0, 5):
        q = rng.choice(vals, size=(3, 32)) * rng.choice([-1.0, 1.0], size=(3, 32))
        q[:, 0] = 256.0 + 32.0 * rng.integers(0, 6, size=3)   # the block max in [256, 448]
        v = q * 2.0 ** s
        assert np.array_equal(mx.mxfp8_round(v), v)


def test_mx_ffn_equals_plain_ffn_on_representable_inputs():
    """Activations with few significant bits over a narrow range (MXFP8 holds them, and the
    SwiGLU intermediate, exactly): the MX expert equals the plain fp64 SwiGLU expert; a
    planted off-grid activation makes them differ."""
    rng = np.random.default_rng(5)
    H, I = 64, 64
    x = rng.choice([0.0, 1.0, 2.0], size=(3, H))
    wg = np.zeros((I, H)); wu = np.zeros((I, H)); wd = np.zeros((H, I))
    for i in range(I):
        wg[i, rng.integers(H)] = rng.choice([1, 2, 3, 4]) * 64.0
        wu[i, rng.integers(H)] = rng.choice([-1, 1]) * rng.choice([0.5, 1.0, 1.5]) / 8
    for h in range(H):
        for j in rng.choice(I, 4, replace=False):
            wd[h, j] = rng.choice([-1, 1]) * rng.choice([0.5, 1.0]) / 16
    plain = expert_ffn(x, wg, wu, wd)
    mxo = mx.expert_ffn_mx(x, wg, wu, wd)
    assert np.abs(mxo - plain).max() <= 1e-9 * max(1.0, np.abs(plain).max())
    x2 = x.copy()
    x2[0, :] = 0.0
    x2[0, 0] = 2.0
    x2[0, 1] = 1.0 + 2.0 ** -6     # needs 7 significant bits: MXFP8 rounds it
    wg2 = wg.copy()
    wg2[:, 1] = 64.0
    assert not np.allclose(mx.expert_ffn_mx(x2, wg2, wu, wd), expert_ffn(x2, wg2, wu, wd), rtol=0, atol=1e-12)


def test_ties_to_even():
    """Values halfway between neighbouring E4M3 values take the even code (the block max is
    fixed at 256 so the scale is 2^0)."""
    cases = [(1.0625, 1.0), (1.1875, 1.25), (-1.0625, -1.0), (2.0 ** -10, 0.0), (3 * 2.0 ** -10, 2.0 ** -8),
             (440.0, 448.0), (424.0, 416.0)]
    for v, want in cases:
        x = np.zeros((1, 32))
        x[0, 0] = 256.0
        x[0, 1] = v
        assert mx.mxfp8_round(x)[0, 1] == want, v
