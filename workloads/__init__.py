"""Seeded synthetic workloads for the routed-MoE layer over a bounded expert cache.

This module holds no step of the method: it names the workload shapes and turns
seeds into input arrays (activations, router weights, expert weights, routing
popularity biases, synthetic routing traces).  The oracle and the GPU path both
draw their inputs from here; neither imports the other.

Shapes follow the page descriptions of the two model families the method is
evaluated on (FreeToken summary, "MoE" section: 43 layers, 256 experts, 6
active for the DeepSeek-V4-Flash shape; Section "Results / prefill": a 64.4 GB
bf16 expert pool for the 35B-A3B shape).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libwlgen.so")
_lib = None

WFMT_F32, WFMT_BF16, WFMT_FP4, WFMT_MXFP4 = 0, 1, 2, 3
AFMT_F32, AFMT_BF16 = 0, 1

# Stream domains (high bits of the stream id); expert domains live in gen.c.
DOMAIN_ROUTER = 3 << 56
DOMAIN_X_DECODE = 4 << 56
DOMAIN_X_PREFILL = 5 << 56
DOMAIN_PERM = 6 << 56
DOMAIN_TRACE = 7 << 56


def host_march() -> str:
    """x86-64-v4 (AVX-512) when the build host has it, else x86-64-v3 (AVX2)."""
    try:
        flags = open("/proc/cpuinfo").read()
    except OSError:
        flags = ""
    return "x86-64-v4" if ("avx512dq" in flags and "avx512bw" in flags) else "x86-64-v3"


def build(force: bool = False) -> str:
    """Compile the generator with the host C compiler (idempotent unless force)."""
    src = os.path.join(_HERE, "gen.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O3", "-march=" + host_march(), "-fPIC", "-shared", "-ffp-contract=off",
                               src, "-o", tmp, "-lpthread", "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _WlCfg(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("wfmt", ctypes.c_int32), ("exact", ctypes.c_int32),
                ("seed", ctypes.c_uint64), ("alias_records", ctypes.c_int64),
                ("sigma", ctypes.c_float), ("fp4_scale_lo", ctypes.c_float),
                ("fp4_scale_hi", ctypes.c_float), ("pad2", ctypes.c_float),
                ("mx_exp_lo", ctypes.c_int32), ("mx_exp_hi", ctypes.c_int32)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        u64, i64, vp, f32 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
        L.wl_hash.restype = u64
        L.wl_hash.argtypes = [u64, u64, u64]
        for name in ("wl_normal_f32", "wl_normal_bf16"):
            getattr(L, name).argtypes = [vp, i64, u64, u64, u64, f32]
        L.wl_bytes.argtypes = [vp, i64, u64, u64, u64]
        L.wl_uniform_bf16.argtypes = [vp, i64, u64, u64, u64, f32, f32]
        L.wl_uniform_f64.argtypes = [vp, i64, u64, u64, u64]
        L.wl_expert_tensor.argtypes = [ctypes.POINTER(_WlCfg), i64, ctypes.c_int, vp, vp]
        L.wl_record_bytes.restype = i64
        L.wl_record_bytes.argtypes = [ctypes.POINTER(_WlCfg)]
        L.wl_pack_record.argtypes = [ctypes.POINTER(_WlCfg), i64, vp]
        L.wl_fill_pool.argtypes = [ctypes.POINTER(_WlCfg), vp, i64, i64, ctypes.c_int]
        L.wl_exact_act.argtypes = [vp, i64, ctypes.c_int, u64, u64, u64]
        L.wl_exact_router.argtypes = [vp, i64, i64, u64, u64]
        _lib = L
    return _lib


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: model shape, formats, cache budget and routing locality."""
    name: str
    seed: int
    n_layers: int
    n_experts: int
    top_k: int
    hidden: int
    inter: int
    wfmt: int
    afmt: int
    tokens: int              # decode batch (decode) or prompt length (prefill)
    steps: int               # decode steps
    n_slots: int             # GPU expert-cache slots
    sigma_w: float = 0.02    # expert weight std (F32 / BF16)
    sigma_r: float = 0.02    # router weight std
    sigma_x: float = 1.0     # activation std
    zipf_s: float = 1.1      # per-layer expert popularity exponent
    zipf_alpha: float = 0.0  # weight of ln Zipf in the logit bias (0 = no popularity bias)
    prev_bonus: float = 0.0  # logit bonus for the previous token's experts at the same layer
    renorm: int = 0
    alias_records: int = 0   # 0 = full pool; R > 0: key -> key % R backing record
    fp4_scale_lo: float = 0.5 * 0.02 / 2.926
    fp4_scale_hi: float = 1.5 * 0.02 / 2.926
    mx_exp_lo: int = 119     # MXFP4 scale exponents: 2^-8 .. 2^-6 (weight rms ~0.03)
    mx_exp_hi: int = 121
    resize_schedule: tuple = ()   # ((after_step, new_n_slots), ...)
    prefill_tokens: int = 0
    # exact-arithmetic inputs: sparse few-bit expert and router weights, activations in
    # {0, 1, 2} (gen.c, wl_exact_tensor): every sum of products is exact in fp32 and the
    # SwiGLU intermediate exact in bf16 / f16, so results can be compared bit for bit
    exact: bool = False

    # ---- derived sizes -------------------------------------------------
    @property
    def n_keys(self) -> int:
        return self.n_layers * self.n_experts

    @property
    def record_bytes(self) -> int:
        return int(lib().wl_record_bytes(ctypes.byref(self._cfg())))

    @property
    def pool_records(self) -> int:
        """Records that actually need host memory (aliased pools are smaller)."""
        return self.n_keys if self.alias_records <= 0 else min(self.alias_records, self.n_keys)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    def _cfg(self) -> _WlCfg:
        return _WlCfg(self.n_layers, self.n_experts, self.hidden, self.inter, self.wfmt, int(self.exact),
                      self.seed, self.alias_records, self.sigma_w,
                      self.fp4_scale_lo, self.fp4_scale_hi, 0.0, self.mx_exp_lo, self.mx_exp_hi)

    # ---- expert weights -------------------------------------------------
    def backing_key(self, key: int) -> int:
        return key % self.alias_records if self.alias_records > 0 else key

    def expert_tensor(self, key: int, t: int):
        """Logical values of tensor t (0 gate [I,H], 1 up [I,H], 2 down [H,I]) of expert `key`.

        F32 -> float32 array; BF16 -> uint16 bf16 bit patterns;
        FP4 -> (uint8 codes [rows, cols/2], uint16 bf16 scale bits [rows, cols/32]);
        MXFP4 -> (uint8 codes [rows, cols/2], uint8 E8M0 scale exponents [rows, cols/32]).
        """
        rows, cols = (self.inter, self.hidden) if t < 2 else (self.hidden, self.inter)
        cfg = self._cfg()
        if self.wfmt == WFMT_F32:
            out = np.empty((rows, cols), np.float32)
            rc = lib().wl_expert_tensor(ctypes.byref(cfg), key, t, out.ctypes.data, None)
        elif self.wfmt == WFMT_BF16:
            out = np.empty((rows, cols), np.uint16)
            rc = lib().wl_expert_tensor(ctypes.byref(cfg), key, t, out.ctypes.data, None)
        else:
            codes = np.empty((rows, cols // 2), np.uint8)
            scales = np.empty((rows, cols // 32), np.uint16 if self.wfmt == WFMT_FP4 else np.uint8)
            rc = lib().wl_expert_tensor(ctypes.byref(cfg), key, t, codes.ctypes.data, scales.ctypes.data)
            out = (codes, scales)
        if rc != 0:
            raise ValueError(f"wl_expert_tensor failed for key {key} tensor {t}")
        return out

    def pack_record(self, key: int) -> np.ndarray:
        buf = np.empty(self.record_bytes, np.uint8)
        if lib().wl_pack_record(ctypes.byref(self._cfg()), key, buf.ctypes.data) != 0:
            raise ValueError("wl_pack_record failed")
        return buf

    def fill_pool(self, ptr: int, first: int, count: int, threads: int | None = None) -> None:
        """Pack records for keys [first, first+count) contiguously at host address `ptr`."""
        threads = threads or min(16, len(os.sched_getaffinity(0)))
        if lib().wl_fill_pool(ctypes.byref(self._cfg()), ctypes.c_void_p(ptr), first, count, threads) != 0:
            raise ValueError("wl_fill_pool failed")

    # ---- router, activations, biases ------------------------------------
    def router_weight(self, layer: int) -> np.ndarray:
        out = np.empty((self.n_experts, self.hidden), np.float32)
        if self.exact:
            lib().wl_exact_router(out.ctypes.data, self.n_experts, self.hidden, self.seed, DOMAIN_ROUTER | layer)
        else:
            lib().wl_normal_f32(out.ctypes.data, out.size, self.seed, DOMAIN_ROUTER | layer, 0, self.sigma_r)
        return out

    def _act(self, domain: int, index: int, tokens: int):
        n = tokens * self.hidden
        if self.exact:
            out = np.empty((tokens, self.hidden), np.float32 if self.afmt == AFMT_F32 else np.uint16)
            lib().wl_exact_act(out.ctypes.data, n, int(self.afmt == AFMT_BF16), self.seed, domain | index, 0)
            return out
        if self.afmt == AFMT_F32:
            out = np.empty((tokens, self.hidden), np.float32)
            lib().wl_normal_f32(out.ctypes.data, n, self.seed, domain | index, 0, self.sigma_x)
        else:
            out = np.empty((tokens, self.hidden), np.uint16)
            lib().wl_normal_bf16(out.ctypes.data, n, self.seed, domain | index, 0, self.sigma_x)
        return out

    def decode_activations(self, step: int, layer: int, tokens: int | None = None):
        """x for decode step `step` at `layer`: [T, H] fp32 (F32 afmt) or bf16 bits (BF16 afmt)."""
        return self._act(DOMAIN_X_DECODE, step * self.n_layers + layer, tokens or self.tokens)

    def prefill_activations(self, layer: int, tokens: int | None = None, chunk: int = 0):
        return self._act(DOMAIN_X_PREFILL, chunk * self.n_layers + layer, tokens or self.prefill_tokens)

    def popularity_perm(self, layer: int) -> np.ndarray:
        """Seeded permutation pi_l: expert e has popularity rank pi_l[e] (0 = most popular)."""
        E = self.n_experts
        r = np.empty(E, np.float64)
        lib().wl_uniform_f64(r.ctypes.data, E, self.seed, DOMAIN_PERM | layer, 0)
        perm = np.arange(E)
        for i in range(E - 1, 0, -1):       # Fisher-Yates
            j = int(r[i] * (i + 1))
            perm[i], perm[j] = perm[j], perm[i]
        return perm

    def zipf_bias(self, layer: int) -> np.ndarray:
        """Per-layer logit bias alpha * ln Zipf_s(rank): float32 [E]."""
        E = self.n_experts
        if self.zipf_alpha == 0.0:
            return np.zeros(E, np.float32)
        rank = self.popularity_perm(layer).astype(np.float64) + 1.0
        harm = float(np.sum(np.arange(1, E + 1, dtype=np.float64) ** (-self.zipf_s)))
        return (self.zipf_alpha * (-self.zipf_s * np.log(rank) - math.log(harm))).astype(np.float32)

    def uniforms(self, stream: int, n: int) -> np.ndarray:
        out = np.empty(n, np.float64)
        lib().wl_uniform_f64(out.ctypes.data, n, self.seed, DOMAIN_TRACE | stream, 0)
        return out

    def synthetic_routing(self, steps: int, layer: int, tokens: int, reuse: float = 0.6) -> np.ndarray:
        """A routing trace with temporal locality, independent of any router: int32 [steps, T, k].

        Each rank slot of each token keeps one of the previous step's experts with
        probability `reuse`, else draws from the layer's Zipf popularity; experts of
        one token are distinct.  Used to drive cache-lookup tests with identical
        inputs on both sides.
        """
        E, k = self.n_experts, self.top_k
        perm = self.popularity_perm(layer)
        inv = np.argsort(perm)                       # rank -> expert
        w = np.arange(1, E + 1, dtype=np.float64) ** (-self.zipf_s)
        cdf = np.cumsum(w) / w.sum()
        u = self.uniforms(layer, steps * tokens * k * 3).reshape(steps, tokens, k, 3)
        out = np.empty((steps, tokens, k), np.int32)
        prev = [None] * tokens
        for s in range(steps):
            for t in range(tokens):
                chosen = []
                for j in range(k):
                    e = -1
                    if prev[t] is not None and u[s, t, j, 0] < reuse:
                        cand = [p for p in prev[t] if p not in chosen]
                        if cand:
                            e = cand[int(u[s, t, j, 1] * len(cand))]
                    tries = 0
                    while e < 0 or e in chosen:
                        x = (u[s, t, j, 2] + 0.618033988749895 * tries) % 1.0
                        e = int(inv[min(int(np.searchsorted(cdf, x)), E - 1)])
                        tries += 1
                        if tries > 4 * E:
                            e = next(ee for ee in range(E) if ee not in chosen)
                    chosen.append(e)
                out[s, t] = chosen
                prev[t] = chosen
        return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (a format conversion)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------
# The five workloads.  Shapes: tiny (tests), the 35B-A3B shape (L=40, E=256,
# k=8, H=2048, I=512, bf16 -> 64,424,509,440-byte pool) and the
# DeepSeek-V4-Flash shape (L=43, E=256, k=6, H=4096, I=2048, e2m1 + bf16
# scale per 32).

TINY = Workload(name="tiny_fp32", seed=1, n_layers=1, n_experts=8, top_k=2, hidden=64, inter=128,
                wfmt=WFMT_F32, afmt=AFMT_F32, tokens=1, steps=16, n_slots=4, prefill_tokens=16)

# Routing locality constants, frozen from workloads/calibration.json (written by
# `python -m workloads.calibrate`, which runs only the oracle): Zipf weight 0.5 keeps a
# 4096-token prompt routed to every expert; a 0.25 previous-token bonus puts the
# steady-state LRU miss rate at 1280 slots nearest the pages' 39%.
ZIPF_ALPHA = 0.5
PREV_BONUS = 0.25

A3B_DECODE = Workload(name="a3b_decode_bf16", seed=2, n_layers=40, n_experts=256, top_k=8, hidden=2048,
                      inter=512, wfmt=WFMT_BF16, afmt=AFMT_BF16, tokens=1, steps=512, n_slots=1280,
                      zipf_alpha=ZIPF_ALPHA, prev_bonus=PREV_BONUS)

A3B_PREFILL = A3B_DECODE.with_(name="a3b_prefill_bf16", seed=2, prefill_tokens=4096, prev_bonus=0.0)

DSV4 = Workload(name="dsv4_fp4", seed=4, n_layers=43, n_experts=256, top_k=6, hidden=4096, inter=2048,
                wfmt=WFMT_FP4, afmt=AFMT_BF16, tokens=1, steps=512, n_slots=1695,
                zipf_alpha=ZIPF_ALPHA, prev_bonus=PREV_BONUS, prefill_tokens=2048)

# The pages' DeepSeek-V4-Flash experts as MXFP4: the same codes with one E8M0 scale byte
# per 32 elements (13,369,344-byte records); the 24 GB cache then holds 1795 slots.
DSV4_MX = DSV4.with_(name="dsv4_mxfp4", wfmt=WFMT_MXFP4, n_slots=1795)

A3B_ELASTIC = A3B_DECODE.with_(name="a3b_elastic_hybrid", seed=5, tokens=4, steps=1024,
                               resize_schedule=((341, 640), (682, 960)))

WORKLOADS = {w.name: w for w in (TINY, A3B_DECODE, A3B_PREFILL, DSV4, DSV4_MX, A3B_ELASTIC)}
