"""SwiGLU expert FFN and the gate-weighted combine, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Each expert holds three weight tensors (the slot ring of [SPARK] copies
"three weight tensors" per swap); with the gate/up/down naming of SwiGLU:
  g = W_gate x,  u = W_up x,  a = silu(g) * u,  y = W_down a,
silu(z) = z / (1 + exp(-z)), no biases; W_gate, W_up are [I,H], W_down [H,I].
The layer output is the gate-weighted sum over the token's k experts taken in
rank order.  Wherever an expert runs (resident slot, fill, or host CPU) it
computes the same y_tj; the GPU and CPU partial sums merge exactly
([FT-KR] "측정된 대역폭이 분할을 결정합니다": each side computes a partial sum
and the two are added with no algorithmic approximation; [FT-CN] Figure 2
caption).  Parity: pinned against transformers' Qwen3-MoE sparse block and
dense SwiGLU MLP, zero-weight and single-expert special cases.
"""
import numpy as np


def silu(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def expert_ffn(x64: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """x [n,H] (float64) through one expert -> [n,H] float64."""
    g = x64 @ w_gate.T
    u = x64 @ w_up.T
    return (silu(g) * u) @ w_down.T


def moe_combine(expert_out: np.ndarray, w: np.ndarray, include: np.ndarray = None) -> np.ndarray:
    """expert_out [T,k,H] float64, gates w [T,k] -> y [T,H] float64, summed in rank order.

    include [T,k] bool restricts the sum to a subset of pairs (a partial sum).
    """
    T, k, H = expert_out.shape
    y = np.zeros((T, H), np.float64)
    for t in range(T):
        for j in range(k):
            if include is None or include[t, j]:
                y[t] += float(w[t, j]) * expert_out[t, j]
    return y


def moe_layer_dense(x64: np.ndarray, idx: np.ndarray, weights_of) -> np.ndarray:
    """All-resident reference: y[t] = sum_j w[t,j] * FFN_{idx[t,j]}(x_t).

    weights_of(expert) -> (W_gate, W_up, W_down) float64.  Returns [T,k,H]
    per-pair expert outputs; combine with moe_combine.
    """
    T, k = idx.shape
    H = x64.shape[1]
    out = np.zeros((T, k, H), np.float64)
    cache = {}
    for e in sorted(set(np.asarray(idx).reshape(-1).tolist())):
        if e not in cache:
            cache[e] = weights_of(e)
        rows = [(t, j) for t in range(T) for j in range(k) if idx[t, j] == e]
        xs = np.stack([x64[t] for t, _ in rows])
        ys = expert_ffn(xs, *cache[e])
        for (t, j), yy in zip(rows, ys):
            out[t, j] = yy
    return out
