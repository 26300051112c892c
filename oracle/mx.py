"""MX activations for the matrix-core prefill of MXFP4 experts: MXFP8 blocks (E4M3 elements).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages serve the DeepSeek-V4-Flash experts in MXFP4 ([FT-KR] "실험 환경") and leave the
activation format of the expert GEMMs open.  Reading taken here, for the prefill path
that feeds MXFP4 weights to the matrix cores as they are stored: the activation operand
of each GEMM (the token rows x for gate/up, the SwiGLU intermediate a for down) is
converted to MXFP8 as the OCP Microscaling Formats v1.0 specification defines it:

  * blocks of 32 consecutive elements along the reduction dimension share one E8M0
    scale 2^s, s = floor(log2(max |v|)) - 8 (8 is the largest E4M3 exponent), clamped to
    [-127, 127]; a block of zeros takes s = -127;
  * each element is v / 2^s rounded to the nearest E4M3 value, ties to the even code,
    magnitudes beyond 448 (the largest E4M3 value) saturating to 448.

The intermediate a is quantised from its fp32 value (the precision the kernel holds it
in), so both sides take each rounding decision on the same number.  Weights are the
MXFP4 records as stored (formats.dequant_mxfp4).  Everything else is the plain fp64
SwiGLU of ffn.expert_ffn.

Parity: pinned in tests/test_oracle_mx.py -- the E4M3 table from its bit fields against
the values the OCP 8-bit floating point specification names, the quantiser against a
brute-force nearest search over every code, round trips of representable blocks, the
scale rule's closed forms, and equality with the plain expert FFN on inputs MXFP8
represents exactly.
"""
import numpy as np

from .ffn import silu

E4M3_MAX = 448.0
MX_BLOCK = 32


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """8-bit E4M3 codes -> float64, from the bit fields: sign, 4 exponent bits (bias 7),
    3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN (no infinities)."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return sign * mag


# every finite non-negative code (0x00 .. 0x7E) and its value, ascending in both
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = e4m3_decode(_POS_CODES)


def _e4m3_nearest(q: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code of each value (ties to the even code), saturating at 448."""
    q = np.asarray(q, dtype=np.float64)
    mag = np.minimum(np.abs(q), E4M3_MAX)
    hi = np.clip(np.searchsorted(_POS_VALUES, mag, side="left"), 0, len(_POS_VALUES) - 1)
    lo = np.clip(hi - 1, 0, len(_POS_VALUES) - 1)
    d_lo = np.abs(mag - _POS_VALUES[lo])
    d_hi = np.abs(_POS_VALUES[hi] - mag)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((_POS_CODES[hi] & 1) == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    return (code | np.where(np.signbit(q), 0x80, 0)).astype(np.uint8)


def mxfp8_quantize(v: np.ndarray):
    """v [rows, n] (n a multiple of 32) -> (E4M3 codes uint8 [rows, n], E8M0 scale bytes
    uint8 [rows, n/32]) by the block rule above."""
    v = np.asarray(v, dtype=np.float64)
    rows, n = v.shape
    blocks = v.reshape(rows, n // MX_BLOCK, MX_BLOCK)
    amax = np.abs(blocks).max(axis=2)
    with np.errstate(divide="ignore"):
        s = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8.0, -127.0)
    s = np.clip(s, -127.0, 127.0)
    q = blocks / np.exp2(s)[:, :, None]
    codes = _e4m3_nearest(q).reshape(rows, n)
    return codes, (s + 127.0).astype(np.uint8)


def mxfp8_dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """E4M3 codes [rows, n] and E8M0 bytes [rows, n/32] -> float64 [rows, n]."""
    vals = e4m3_decode(codes)
    rows, n = vals.shape
    sc = np.exp2(np.asarray(scales).astype(np.float64) - 127.0)
    return (vals.reshape(rows, n // MX_BLOCK, MX_BLOCK) * sc[:, :, None]).reshape(rows, n)


def mxfp8_round(v: np.ndarray) -> np.ndarray:
    """The value MXFP8 represents for each element of v [rows, n]."""
    return mxfp8_dequant(*mxfp8_quantize(v))


def expert_ffn_mx(x64: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """x [n,H] (float64) through one expert with MXFP8 activations on both GEMMs -> [n,H]."""
    xq = mxfp8_round(x64)
    a = silu(xq @ w_gate.T) * (xq @ w_up.T)
    a32 = a.astype(np.float32).astype(np.float64)
    return mxfp8_round(a32) @ w_down.T
