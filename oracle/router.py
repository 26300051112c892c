"""Router: logits, top-k selection and gates.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages say only that the router and the cache lookup run on the GPU and
pick k of E experts per token ([FT-KR] "decode 공동 설계" opening paragraph;
"MoE는 기회이면서 동시에 난제입니다": k << E, 6 of 256 for DeepSeek-V4-Flash).
The router function itself is not stated; the plainest reading, consistent
with the "top-k softmax routing" of the workload description, is:
  z = x W_r^T + bias          (fp32 router weights; bias is a workload input)
  p = softmax(z) over all E
  idx = the k largest z, highest first, ties to the lower expert index
  w_j = p[idx_j]              (renorm=1: w_j = p[idx_j] / sum_j' p[idx_j'])
The selection is decided on fp32 logits, the precision the GPU decides in.
Parity: pinned against an exhaustive rank count, brute force over all
k-subsets, scipy's softmax and transformers' Qwen3-MoE sparse block.
"""
import numpy as np


def router_logits(x64: np.ndarray, w_r: np.ndarray, bias=None) -> np.ndarray:
    """fp64 x [T,H] times fp32 router [E,H]^T (+ bias [T,E] or [E]) in fp64, rounded once to fp32."""
    z = np.asarray(x64, dtype=np.float64) @ np.asarray(w_r, dtype=np.float64).T
    if bias is not None:
        z = z + np.asarray(bias, dtype=np.float64)
    return z.astype(np.float32)


def topk_order(z_row: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest entries of one fp32 logit row, in rank order.

    Total order: e before e' iff z_e > z_e' or (z_e == z_e' and e < e');
    -0.0 and +0.0 compare equal.  Non-finite logits are rejected.
    """
    z = np.asarray(z_row, dtype=np.float32)
    if not np.all(np.isfinite(z)):
        raise ValueError("non-finite router logit")
    E = z.shape[0]
    order = sorted(range(E), key=lambda e: (-float(z[e]), e))
    return np.array(order[:k], dtype=np.int32)


def route(z: np.ndarray, k: int, renorm: int = 0):
    """fp32 logits [T,E] -> (idx [T,k] int32 in rank order, w [T,k] fp32 gates)."""
    z = np.asarray(z, dtype=np.float32)
    T, E = z.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    for t in range(T):
        sel = topk_order(z[t], k)
        zz = z[t].astype(np.float64)
        p = np.exp(zz - zz.max())
        p = p / p.sum()
        g = p[sel]
        if renorm:
            g = g / g.sum()
        idx[t] = sel
        w[t] = g.astype(np.float32)
    return idx, w
