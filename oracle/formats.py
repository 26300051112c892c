"""Weight and activation formats, widened exactly to float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

bf16: the upper 16 bits of an IEEE binary32.  e2m1 (OCP Microscaling spec,
"FP4 E2M1"): bit 3 sign, bits 2..1 exponent with bias 1, bit 0 mantissa;
exponent 0 is subnormal with value 0.5 * mantissa.  The DeepSeek-V4-Flash
experts on the pages are MXFP4 ([FT-KR] "실험 환경": routed experts quantised
to MXFP4); the workload stores one bf16 scale per 32 consecutive elements of a
row (the reduction dimension), a superset of the power-of-two MX scale.
MXFP4 keeps the MX scale itself: one E8M0 byte e per 32-element block, an
exponent with bias 127 and no sign or mantissa, so the scale is 2^(e - 127)
(OCP Microscaling spec, "E8M0"; e = 255 encodes NaN).
Parity: pinned by the exhaustive 16-code table test, by round trips, and MXFP4
by equality with the bf16-scale path fed the same powers of two as bf16 bits.
"""
import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exact."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """4-bit e2m1 codes (0..15, any integer dtype) -> float64 values, from the bit-field definition."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    exp = (c >> 1) & 3
    man = (c & 1).astype(np.float64)
    mag = np.where(exp == 0, 0.5 * man, (1.0 + 0.5 * man) * np.exp2(exp.astype(np.float64) - 1.0))
    return sign * mag


# The value of every 4-bit code, from the bit-field definition above (evaluated once;
# indexing it is the same map as calling e2m1_decode on each code).
_E2M1_TABLE = e2m1_decode(np.arange(16))


def _e2m1_values(codes: np.ndarray) -> np.ndarray:
    """Packed codes [rows, cols/2] (element 2i in the low nibble of byte i) -> float64 [rows, cols]."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows, half = codes.shape
    nib = np.empty((rows, half * 2), dtype=np.uint8)
    nib[:, 0::2] = codes & 0x0F
    nib[:, 1::2] = codes >> 4
    return _E2M1_TABLE[nib]


def dequant_fp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Packed codes [rows, cols/2] (element 2i in the low nibble of byte i) and bf16 scale
    bits [rows, cols/32] -> float64 [rows, cols]; w = e2m1(code) * scale of its 32-block."""
    vals = _e2m1_values(codes)                     # [rows, cols]
    sc = bf16_to_f64(scales)                       # [rows, cols/32]
    rows, cols = vals.shape
    return (vals.reshape(rows, cols // 32, 32) * sc[:, :, None]).reshape(rows, cols)


def e8m0_decode(e: np.ndarray) -> np.ndarray:
    """E8M0 scale bytes -> float64: 2^(e - 127); 255 is NaN."""
    e = np.asarray(e).astype(np.int64)
    return np.where(e == 255, np.nan, np.exp2((e - 127).astype(np.float64)))


def dequant_mxfp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Packed codes [rows, cols/2] (element 2i in the low nibble of byte i) and E8M0 scale
    bytes [rows, cols/32] -> float64 [rows, cols]; w = e2m1(code) * 2^(e - 127)."""
    vals = _e2m1_values(codes)
    rows, cols = vals.shape
    sc = e8m0_decode(scales)
    return (vals.reshape(rows, cols // 32, 32) * sc[:, :, None]).reshape(rows, cols)


def expert_weights_f64(workload, key: int):
    """(W_gate [I,H], W_up [I,H], W_down [H,I]) of expert `key` as float64.

    A slot holds every tensor needed to evaluate one (layer, expert) pair
    ([FT-KR] "FreeToken의 설계"); the expert's identity is the flattened id
    key = layer * E + expert ([FT-KR] "전문가 뱅크와 FTW 포맷").
    """
    from workloads import WFMT_F32, WFMT_BF16, WFMT_FP4
    out = []
    for t in range(3):
        v = workload.expert_tensor(key, t)
        if workload.wfmt == WFMT_F32:
            out.append(np.asarray(v, dtype=np.float64))
        elif workload.wfmt == WFMT_BF16:
            out.append(bf16_to_f64(v))
        elif workload.wfmt == WFMT_FP4:
            out.append(dequant_fp4(*v))
        else:
            out.append(dequant_mxfp4(*v))
    return tuple(out)


def activations_f64(x) -> np.ndarray:
    """Activation array from the workload (float32, or uint16 bf16 bits) -> float64."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_to_f64(x)
    return x.astype(np.float64)
