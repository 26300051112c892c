"""The host CPU branch and its worker pool, on the CPU: regression tests for the
pool's claim protocol and start-up, and the branch's numerics against the oracle."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
import workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.fixture(scope="module")
def shim(tmp_path_factory):
    from routed_expert_ffn_02_amd._build import host_cxx, rocm_root
    out = str(tmp_path_factory.mktemp("shim") / "libcpushim.so")
    cmd = [host_cxx(), "-O2", "-std=c++17", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm_root(), "include"),
           os.path.join(HERE, "native", "cpu_branch_shim.cpp"),
           os.path.join(ROOT, "routed_expert_ffn_02_amd", "csrc", "cpu_ffn.cpp"), "-o", out, "-lpthread"]
    subprocess.check_call(cmd)
    lib = ctypes.CDLL(out)
    i32, vp = ctypes.c_int, ctypes.c_void_p
    lib.shim_pool_stress.restype = ctypes.c_longlong
    lib.shim_pool_stress.argtypes = [i32, i32]
    lib.shim_pool_lifecycle.argtypes = [i32, i32]
    lib.shim_cpu_ffn.argtypes = [i32, i32, i32, i32, i32, ctypes.c_longlong, vp, vp, vp, vp, i32, vp, vp, i32]
    return lib


def test_pool_claims_each_task_once(shim):
    assert shim.shim_pool_stress(16, 20000) == 0


def test_pool_destroy_never_blocks(shim):
    # a pool destroyed before its threads first run used to wait forever in join
    assert shim.shim_pool_lifecycle(16, 200) == 0


@pytest.mark.parametrize("wl", [W.TINY, W.A3B_DECODE.with_(n_layers=1, n_experts=8, hidden=256, inter=128),
                                W.DSV4.with_(n_layers=1, n_experts=8, hidden=256, inter=128),
                                W.DSV4_MX.with_(n_layers=1, n_experts=8, hidden=256, inter=256)],
                         ids=["fp32", "bf16", "fp4", "mxfp4"])
@pytest.mark.parametrize("T", [1, 3])
def test_cpu_branch_matches_oracle(shim, wl, T):
    k, H, I = wl.top_k, wl.hidden, wl.inter
    rng = np.random.default_rng(T)
    idx = np.stack([rng.choice(wl.n_experts, size=k, replace=False) for _ in range(T)])
    w = rng.uniform(0.1, 1.0, size=(T, k)).astype(np.float32)
    # every other pair runs on the CPU; CPU list = distinct CPU experts in first-appearance order
    cpu_mask = (np.arange(T * k).reshape(T, k) % 2) == 0
    cpu_keys = []
    for t in range(T):
        for j in range(k):
            if cpu_mask[t, j] and idx[t, j] not in cpu_keys:
                cpu_keys.append(int(idx[t, j]))
    slot = np.where(cpu_mask, -1 - np.vectorize(lambda e: cpu_keys.index(e) if e in cpu_keys else 0)(idx), 5)
    slot = slot.astype(np.int32)
    recs = [wl.pack_record(e) for e in cpu_keys]
    ptrs = (ctypes.c_void_p * len(recs))(*[r.ctypes.data for r in recs])
    x = np.stack([oracle.formats.activations_f64(wl.decode_activations(0, 0, T))[t] for t in range(T)]).astype(np.float32)
    h = np.zeros((T * k, I), np.float32)
    y = np.zeros((T, H), np.float32)
    shim.shim_cpu_ffn(wl.wfmt, H, I, T, k, wl.record_bytes, x.ctypes.data, w.ctypes.data,
                      slot.ctypes.data, ptrs, len(recs), h.ctypes.data, y.ctypes.data, 4)
    outs = oracle.moe_layer_dense(x.astype(np.float64), idx, lambda e: oracle.expert_weights_f64(wl, e))
    ref = oracle.moe_combine(outs, w, cpu_mask)
    err = np.abs(y - ref).max() / np.abs(ref).max()
    assert err <= (1e-5 if wl.wfmt == W.WFMT_F32 else 1e-4), err
