"""Python binding of the routed-MoE C-ABI library (libroutedmoe.so, HIP for gfx950).

Argument marshalling only: every function here has the name of a C entry point
declared in include/routed_moe.h and forwards to it.  Device tensors are passed
as raw pointers (torch supplies device memory and the HIP stream); every step of
the hot path runs in the library's kernels.  There is no fallback: importing
this package fails when the compiled library is missing.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime the library links against)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libroutedmoe.so")

MOE_OK, MOE_EINVAL, MOE_ENOMEM, MOE_EHIP, MOE_ESTATE, MOE_ENOPIN, MOE_ENOTSUP, MOE_ETIMEDOUT = 0, -1, -2, -3, -4, -5, -6, -7
MOE_WFMT_F32, MOE_WFMT_BF16, MOE_WFMT_FP4, MOE_WFMT_MXFP4 = 0, 1, 2, 3
MOE_AFMT_F32, MOE_AFMT_BF16 = 0, 1
MOE_MODE_FUSED, MOE_MODE_OFFLOAD, MOE_MODE_CPU, MOE_MODE_HYBRID = 0, 1, 2, 3
MOE_KIND_HIT, MOE_KIND_FILL, MOE_KIND_CPU, MOE_KIND_BUF = 0, 1, 2, 3
MOE_FLAG_PROFILE = 1
MOE_FLAG_DEVICE_FILLS = 2
MOE_FLAG_MX_PREFILL = 4

_STATUS = {0: "MOE_OK", -1: "MOE_EINVAL", -2: "MOE_ENOMEM", -3: "MOE_EHIP", -4: "MOE_ESTATE",
           -5: "MOE_ENOPIN", -6: "MOE_ENOTSUP", -7: "MOE_ETIMEDOUT"}


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: {_STATUS.get(status, status)}: {msg}")
        self.status = status


class moe_config(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("wfmt", ctypes.c_int32),
                ("afmt", ctypes.c_int32), ("renorm", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
                ("mode", ctypes.c_int32), ("bw_pcie", ctypes.c_uint64), ("bw_host", ctypes.c_uint64),
                ("cpu_threads", ctypes.c_int32), ("flags", ctypes.c_int32)]


class moe_trace_rec(ctypes.Structure):
    _fields_ = [("key", ctypes.c_int32), ("kind", ctypes.c_int32), ("slot", ctypes.c_int32),
                ("evicted", ctypes.c_int32)]


class moe_stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in ("decode_calls", "prefill_calls", "lookups", "hits", "fills",
                                                 "cpu_experts", "evictions", "fill_bytes")] + [
        ("phase1_ms", ctypes.c_double), ("phase2_ms", ctypes.c_double),
        ("phase1_launches", ctypes.c_uint64), ("phase2_launches", ctypes.c_uint64),
        ("phase1_bytes", ctypes.c_uint64), ("phase2_bytes", ctypes.c_uint64),
        ("gemm1_ms", ctypes.c_double), ("gemm2_ms", ctypes.c_double),
        ("gemm1_launches", ctypes.c_uint64), ("gemm2_launches", ctypes.c_uint64),
        ("gemm_flops", ctypes.c_double), ("copy_ms", ctypes.c_double), ("copy_bytes", ctypes.c_uint64),
        ("cpu_ms", ctypes.c_double)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class moe_step_rec(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("layer", "misses", "fills", "cpu")] + [
        ("fill_ms", ctypes.c_double), ("cpu_ms", ctypes.c_double)]


MOE_PLACE_LRU, MOE_PLACE_PREFILL, MOE_PLACE_STATIC, MOE_PLACE_PINNED_RING = 0, 1, 2, 3


class moe_replay_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("n_layers", "n_experts", "pairs", "policy", "capacity",
                                              "ring_per_layer")]


class moe_replay_result(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in ("keys", "misses", "reads")]


class moe_bank_header(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("n_layers", "n_experts", "hidden", "inter", "wfmt", "pad")] + [
        ("record_bytes", ctypes.c_int64), ("n_records", ctypes.c_int64)]


class moe_bank_stats(ctypes.Structure):
    _fields_ = [("bytes", ctypes.c_uint64), ("seconds", ctypes.c_double), ("mode", ctypes.c_int32),
                ("threads", ctypes.c_int32), ("direct_errno", ctypes.c_int32), ("pad", ctypes.c_int32)]


BANK_READ_MODES = {0: "direct", 1: "direct_bounce", 2: "buffered"}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python routed_expert_ffn_02_amd/_build.py` "
                          "(hipcc, gfx950).  There is no CPU fallback.")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, U64, VP = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p
    sig = {
        "moe_create": (I32, [ctypes.POINTER(moe_config), ctypes.POINTER(P)]),
        "moe_destroy": (I32, [P]),
        "moe_last_error": (ctypes.c_char_p, [P]),
        "moe_record_bytes": (I64, [ctypes.POINTER(moe_config)]),
        "moe_pool_alloc": (I32, [P, I64, ctypes.POINTER(VP)]),
        "moe_pool_register": (I32, [P, VP, I64, I32]),
        "moe_bind": (I32, [P, VP, VP, ctypes.c_size_t, I32]),
        "moe_fused_load": (I32, [P, VP]),
        "moe_set_bandwidths": (I32, [P, U64, U64]),
        "moe_set_mode": (I32, [P, I32]),
        "moe_set_cpu_wait": (I32, [P, ctypes.c_double]),
        "moe_route": (I32, [P, I32, VP, I32, VP, VP, VP, VP, VP]),
        "moe_topk": (I32, [P, VP, I32, VP, VP, VP]),
        "expert_cache_lookup": (I32, [P, I32, VP, I32, VP, VP, VP, VP]),
        "moe_route_lookup": (I32, [P, I32, VP, I32, VP, VP, VP, VP, VP, VP, VP, VP]),
        "moe_decode_layer": (I32, [P, I32, VP, I32, VP, VP, VP, VP, VP, VP]),
        "moe_ffn_decode": (I32, [P, I32, VP, I32, VP, VP, VP, VP, VP]),
        "moe_prefill_begin": (I32, [P, VP]),
        "moe_ffn_prefill": (I32, [P, I32, VP, I32, VP, VP, VP, VP, VP, VP]),
        "moe_prefill_end": (I32, [P, VP]),
        "moe_permute": (I32, [P, VP, I32, VP, VP, VP, VP, VP]),
        "expert_cache_resize": (I32, [P, I32, VP, ctypes.c_size_t, VP]),
        "qstar_split": (I32, [I32, U64, U64, I32, I32]),
        "moe_bench_bw": (I32, [P, ctypes.POINTER(U64), ctypes.POINTER(U64)]),
        "moe_cache_snapshot": (I32, [P, VP, VP, VP, ctypes.POINTER(U64), ctypes.POINTER(I32)]),
        "moe_get_stats": (I32, [P, ctypes.POINTER(moe_stats)]),
        "moe_reset_stats": (I32, [P]),
        "moe_sync": (I32, [P, VP]),
        "moe_step_log": (I32, [P, VP, I32, ctypes.POINTER(I32)]),
        "moe_permute_noalloc": (I32, [VP, I32, I32, VP, VP, VP, VP, VP]),
        "moe_bench_hbm": (I32, [VP, ctypes.c_size_t, ctypes.c_size_t, I32, VP, VP]),
        "moe_placement_replay": (I32, [ctypes.POINTER(moe_replay_config), VP, I32, VP, I32, I32, VP,
                                       ctypes.POINTER(moe_replay_result)]),
        "moe_pool_check_f16": (I32, [ctypes.POINTER(moe_config), VP, I64, ctypes.POINTER(I64)]),
        "moe_bank_write": (I32, [ctypes.c_char_p, ctypes.POINTER(moe_config), VP, I64]),
        "moe_bank_info": (I32, [ctypes.c_char_p, ctypes.POINTER(moe_bank_header)]),
        "moe_bank_read": (I32, [ctypes.c_char_p, ctypes.POINTER(moe_config), VP, I64, I32,
                                ctypes.POINTER(moe_bank_stats)]),
        "moe_pool_load": (I32, [P, ctypes.c_char_p, I32, ctypes.POINTER(VP), ctypes.POINTER(moe_bank_stats)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


lib = _load()


# ---------------------------------------------------------------------------
def _ptr(t):
    """Device / host pointer of a tensor, an int address, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(s):
    if s is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


class Ctx:
    """Owner of a moe_ctx handle (destroyed with moe_destroy)."""

    def __init__(self, handle: int, cfg: moe_config):
        self.handle = handle
        self.cfg = cfg
        # held here so that a context collected at interpreter exit, after the
        # module globals are cleared, can still be destroyed
        self._destroy = lib.moe_destroy

    def __del__(self):
        if getattr(self, "handle", None):
            self._destroy(self.handle)
            self.handle = None


def _check(ctx, st, where):
    if st != MOE_OK:
        msg = lib.moe_last_error(ctx.handle if isinstance(ctx, Ctx) else ctx)
        raise MoeError(st, where, msg.decode() if msg else "")


def make_config(n_layers, n_experts, top_k, hidden, inter, wfmt, afmt, max_tokens, mode, renorm=0,
                bw_pcie=0, bw_host=0, cpu_threads=0, flags=0) -> moe_config:
    return moe_config(n_layers, n_experts, top_k, hidden, inter, wfmt, afmt, renorm, max_tokens, mode,
                      bw_pcie, bw_host, cpu_threads, flags)


def moe_create(cfg: moe_config) -> Ctx:
    h = ctypes.c_void_p()
    st = lib.moe_create(ctypes.byref(cfg), ctypes.byref(h))
    if st != MOE_OK:
        raise MoeError(st, "moe_create", "invalid configuration or device error")
    return Ctx(h.value, cfg)


def moe_destroy(ctx: Ctx) -> None:
    if ctx.handle:
        _check(ctx, lib.moe_destroy(ctx.handle), "moe_destroy")
        ctx.handle = None


def moe_last_error(ctx: Ctx) -> str:
    return lib.moe_last_error(ctx.handle).decode()


def moe_record_bytes(cfg: moe_config) -> int:
    return int(lib.moe_record_bytes(ctypes.byref(cfg)))


def moe_pool_check_f16(cfg: moe_config, pool, n_records: int) -> int:
    """Lowest record index whose block scales could take an FP4 / MXFP4 prefill weight out of
    f16's normal range, or -1 when every record passes."""
    bad = ctypes.c_int64(-1)
    st = lib.moe_pool_check_f16(ctypes.byref(cfg), _ptr(pool), n_records, ctypes.byref(bad))
    if st not in (MOE_OK, MOE_EINVAL) or (st == MOE_EINVAL and bad.value < 0):
        raise MoeError(st, "moe_pool_check_f16", "bad argument")
    return int(bad.value)


def moe_pool_alloc(ctx: Ctx, n_records: int) -> int:
    p = ctypes.c_void_p()
    _check(ctx, lib.moe_pool_alloc(ctx.handle, n_records, ctypes.byref(p)), "moe_pool_alloc")
    return p.value


def moe_pool_register(ctx: Ctx, host_pool, n_records: int, pinned: int) -> None:
    _check(ctx, lib.moe_pool_register(ctx.handle, _ptr(host_pool), n_records, pinned), "moe_pool_register")


def moe_bind(ctx: Ctx, router_w, arena, arena_bytes: int, n_slots: int) -> None:
    _check(ctx, lib.moe_bind(ctx.handle, _ptr(router_w), _ptr(arena), arena_bytes, n_slots), "moe_bind")


def moe_fused_load(ctx: Ctx, stream=None) -> None:
    _check(ctx, lib.moe_fused_load(ctx.handle, _stream(stream)), "moe_fused_load")


def moe_set_bandwidths(ctx: Ctx, bw_pcie: int, bw_host: int) -> None:
    _check(ctx, lib.moe_set_bandwidths(ctx.handle, int(bw_pcie), int(bw_host)), "moe_set_bandwidths")


def moe_set_mode(ctx: Ctx, mode: int) -> None:
    _check(ctx, lib.moe_set_mode(ctx.handle, mode), "moe_set_mode")


def moe_set_cpu_wait(ctx: Ctx, timeout_ms: float) -> None:
    _check(ctx, lib.moe_set_cpu_wait(ctx.handle, float(timeout_ms)), "moe_set_cpu_wait")


def moe_route(ctx: Ctx, layer, x, T, logit_bias, logits_out, topk_idx, topk_w, stream=None) -> None:
    _check(ctx, lib.moe_route(ctx.handle, layer, _ptr(x), T, _ptr(logit_bias), _ptr(logits_out), _ptr(topk_idx),
                              _ptr(topk_w), _stream(stream)), "moe_route")


def moe_topk(ctx: Ctx, logits, T, topk_idx, topk_w, stream=None) -> None:
    _check(ctx, lib.moe_topk(ctx.handle, _ptr(logits), T, _ptr(topk_idx), _ptr(topk_w), _stream(stream)),
           "moe_topk")


def expert_cache_lookup(ctx: Ctx, layer, topk_idx, T, slot_idx, trace=None, counts=None, stream=None) -> None:
    _check(ctx, lib.expert_cache_lookup(ctx.handle, layer, _ptr(topk_idx), T, _ptr(slot_idx), _ptr(trace),
                                        _ptr(counts), _stream(stream)), "expert_cache_lookup")


def moe_route_lookup(ctx: Ctx, layer, x, T, logit_bias, logits_out, topk_idx, topk_w, slot_idx, trace=None,
                     counts=None, stream=None) -> None:
    _check(ctx, lib.moe_route_lookup(ctx.handle, layer, _ptr(x), T, _ptr(logit_bias), _ptr(logits_out), _ptr(topk_idx),
                                     _ptr(topk_w), _ptr(slot_idx), _ptr(trace), _ptr(counts), _stream(stream)),
           "moe_route_lookup")


def moe_decode_layer(ctx: Ctx, layer, x, T, logit_bias, topk_idx, topk_w, slot_idx, y, stream=None) -> None:
    _check(ctx, lib.moe_decode_layer(ctx.handle, layer, _ptr(x), T, _ptr(logit_bias), _ptr(topk_idx), _ptr(topk_w),
                                     _ptr(slot_idx), _ptr(y), _stream(stream)), "moe_decode_layer")


def moe_ffn_decode(ctx: Ctx, layer, x, T, topk_idx, topk_w, slot_idx, y, stream=None) -> None:
    _check(ctx, lib.moe_ffn_decode(ctx.handle, layer, _ptr(x), T, _ptr(topk_idx), _ptr(topk_w), _ptr(slot_idx),
                                   _ptr(y), _stream(stream)), "moe_ffn_decode")


def moe_prefill_begin(ctx: Ctx, stream=None) -> None:
    _check(ctx, lib.moe_prefill_begin(ctx.handle, _stream(stream)), "moe_prefill_begin")


def moe_ffn_prefill(ctx: Ctx, layer, x, T, topk_idx, topk_w, y, trace=None, counts=None, stream=None) -> None:
    _check(ctx, lib.moe_ffn_prefill(ctx.handle, layer, _ptr(x), T, _ptr(topk_idx), _ptr(topk_w), _ptr(y),
                                    _ptr(trace), _ptr(counts), _stream(stream)), "moe_ffn_prefill")


def moe_prefill_end(ctx: Ctx, stream=None) -> None:
    _check(ctx, lib.moe_prefill_end(ctx.handle, _stream(stream)), "moe_prefill_end")


def moe_permute(ctx: Ctx, slot_idx, T, perm, offsets, group_slot, n_groups, stream=None) -> None:
    _check(ctx, lib.moe_permute(ctx.handle, _ptr(slot_idx), T, _ptr(perm), _ptr(offsets), _ptr(group_slot),
                                _ptr(n_groups), _stream(stream)), "moe_permute")


def expert_cache_resize(ctx: Ctx, new_n_slots, new_arena=None, new_arena_bytes=0, stream=None) -> None:
    _check(ctx, lib.expert_cache_resize(ctx.handle, new_n_slots, _ptr(new_arena), new_arena_bytes,
                                        _stream(stream)), "expert_cache_resize")


def qstar_split(m: int, bw_pcie: int, bw_host: int, mode: int, evictable: int) -> int:
    return int(lib.qstar_split(m, bw_pcie, bw_host, mode, evictable))


def moe_placement_replay(n_layers: int, n_experts: int, policy: int, capacity: int, decode, calib=None,
                         ring_per_layer: int = 0, want_miss: bool = False):
    """Replay a host routing trace (decode [steps, L, T*k], calib [tokens, L, k], int32
    NumPy arrays) against one placement policy.  Returns a dict with keys, misses, reads
    and, with want_miss, the per-pair miss flags [steps, L, T*k] (uint8)."""
    import numpy as np
    dec = np.ascontiguousarray(decode, dtype=np.int32)
    steps, L, pairs = dec.shape
    cal = None if calib is None else np.ascontiguousarray(calib, dtype=np.int32)
    cfg = moe_replay_config(n_layers, n_experts, pairs, policy, capacity, ring_per_layer)
    miss = np.zeros(dec.shape, np.uint8) if want_miss else None
    res = moe_replay_result()
    st = lib.moe_placement_replay(ctypes.byref(cfg), dec.ctypes.data, steps,
                                  None if cal is None else cal.ctypes.data,
                                  0 if cal is None else cal.shape[0], 1 if cal is None else cal.shape[2],
                                  None if miss is None else miss.ctypes.data, ctypes.byref(res))
    if st != MOE_OK:
        raise MoeError(st, "moe_placement_replay", "invalid shapes, ids or capacity")
    out = {"keys": res.keys, "misses": res.misses, "reads": res.reads}
    if want_miss:
        out["miss"] = miss
    return out


def _stats_dict(st: "moe_bank_stats") -> dict:
    return {"bytes": st.bytes, "seconds": st.seconds, "mode": BANK_READ_MODES.get(st.mode, st.mode),
            "threads": st.threads, "direct_errno": st.direct_errno}


def moe_bank_write(path: str, cfg: moe_config, pool, n_records: int) -> None:
    """Write n_records records from host memory `pool` (address or NumPy array) as a bank file."""
    st = lib.moe_bank_write(os.fsencode(path), ctypes.byref(cfg), _host_ptr(pool), n_records)
    if st != MOE_OK:
        raise MoeError(st, "moe_bank_write", f"cannot write {path}")


def moe_bank_info(path: str) -> dict:
    h = moe_bank_header()
    st = lib.moe_bank_info(os.fsencode(path), ctypes.byref(h))
    if st != MOE_OK:
        raise MoeError(st, "moe_bank_info", f"{path}: missing, malformed or truncated bank file")
    return {n: getattr(h, n) for n, _ in h._fields_ if n != "pad"}


def moe_bank_read(path: str, cfg, dst, dst_bytes: int, threads: int = 8) -> dict:
    """Read a bank file's records into host memory `dst` (address or NumPy array)."""
    out = moe_bank_stats()
    st = lib.moe_bank_read(os.fsencode(path), None if cfg is None else ctypes.byref(cfg), _host_ptr(dst), dst_bytes,
                           threads, ctypes.byref(out))
    if st != MOE_OK:
        raise MoeError(st, "moe_bank_read", f"{path}: header mismatch, short buffer or read error")
    return _stats_dict(out)


def moe_pool_load(ctx: Ctx, path: str, threads: int = 8):
    """Allocate the context's page-locked pool from a bank file and fill it; returns (pool address, stats)."""
    p = ctypes.c_void_p()
    out = moe_bank_stats()
    _check(ctx, lib.moe_pool_load(ctx.handle, os.fsencode(path), threads, ctypes.byref(p), ctypes.byref(out)),
           "moe_pool_load")
    return p.value, _stats_dict(out)


def _host_ptr(a):
    if a is None or isinstance(a, int):
        return a
    return a.ctypes.data


def moe_bench_bw(ctx: Ctx):
    bp, bh = ctypes.c_uint64(), ctypes.c_uint64()
    _check(ctx, lib.moe_bench_bw(ctx.handle, ctypes.byref(bp), ctypes.byref(bh)), "moe_bench_bw")
    return bp.value, bh.value


def moe_cache_snapshot(ctx: Ctx):
    """(slot_of [L*E], key_of [n_slots], stamp [n_slots], counter) as numpy arrays / int."""
    import numpy as np
    c = ctx.cfg
    slot_of = np.empty(c.n_layers * c.n_experts, np.int32)
    n = ctypes.c_int32()
    cnt = ctypes.c_uint64()
    _check(ctx, lib.moe_cache_snapshot(ctx.handle, slot_of.ctypes.data, None, None, ctypes.byref(cnt),
                                       ctypes.byref(n)), "moe_cache_snapshot")
    key_of = np.empty(max(n.value, 1), np.int32)
    stamp = np.empty(max(n.value, 1), np.uint64)
    _check(ctx, lib.moe_cache_snapshot(ctx.handle, None, key_of.ctypes.data, stamp.ctypes.data, None, None),
           "moe_cache_snapshot")
    return slot_of, key_of[: n.value], stamp[: n.value], cnt.value


def moe_get_stats(ctx: Ctx) -> dict:
    st = moe_stats()
    _check(ctx, lib.moe_get_stats(ctx.handle, ctypes.byref(st)), "moe_get_stats")
    return st.as_dict()


def moe_reset_stats(ctx: Ctx) -> None:
    _check(ctx, lib.moe_reset_stats(ctx.handle), "moe_reset_stats")


def moe_sync(ctx: Ctx, stream=None) -> None:
    _check(ctx, lib.moe_sync(ctx.handle, _stream(stream)), "moe_sync")


def moe_step_log(ctx: Ctx, capacity: int = 1 << 20):
    """The logged steps (oldest first) as a numpy record array; clears the log."""
    import numpy as np
    buf = (moe_step_rec * capacity)()
    n = ctypes.c_int32()
    _check(ctx, lib.moe_step_log(ctx.handle, ctypes.addressof(buf), capacity, ctypes.byref(n)), "moe_step_log")
    dt = np.dtype([("layer", np.int32), ("misses", np.int32), ("fills", np.int32), ("cpu", np.int32),
                   ("fill_ms", np.float64), ("cpu_ms", np.float64)])
    return np.frombuffer(bytes(buf)[: n.value * ctypes.sizeof(moe_step_rec)], dtype=dt).copy()


def moe_bench_hbm(buf, buf_bytes: int, read_bytes: int, reps: int, stream=None):
    """Per-pass kernel seconds of reps plain reads of read_bytes from the device buffer buf."""
    import numpy as np
    out = np.zeros(reps, np.float64)
    st = lib.moe_bench_hbm(_ptr(buf), buf_bytes, read_bytes, reps, out.ctypes.data, _stream(stream))
    if st != MOE_OK:
        raise MoeError(st, "moe_bench_hbm", "bad arguments or device error")
    return out


def moe_permute_noalloc(slot_idx, P: int, n_slot_range: int, perm, offsets, group_slot, n_groups, stream=None):
    st = lib.moe_permute_noalloc(_ptr(slot_idx), P, n_slot_range, _ptr(perm), _ptr(offsets), _ptr(group_slot),
                                 _ptr(n_groups), _stream(stream))
    if st != MOE_OK:
        raise MoeError(st, "moe_permute_noalloc", "sizes out of range, null pointer or launch failure")
