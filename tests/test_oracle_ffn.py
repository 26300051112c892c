"""Pins for the expert FFN and the MoE layer output (oracle/ffn.py, oracle/layer.py)."""
import json
import os

import numpy as np
import pytest
import torch

import workloads as W
from oracle import (expert_ffn, moe_combine, moe_layer_dense, route, router_logits, e2m1_decode,
                    dequant_fp4, bf16_to_f64, OracleMoE, MODE_HYBRID, MODE_FUSED, MODE_OFFLOAD)

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _qwen3_block(E, k, H, I, renorm):
    from transformers.models.qwen3_moe.configuration_qwen3_moe import Qwen3MoeConfig
    from transformers.models.qwen3_moe.modeling_qwen3_moe import Qwen3MoeSparseMoeBlock
    cfg = Qwen3MoeConfig(hidden_size=H, moe_intermediate_size=I, num_experts=E, num_experts_per_tok=k,
                         norm_topk_prob=bool(renorm), hidden_act="silu")
    return Qwen3MoeSparseMoeBlock(cfg).double()


@pytest.mark.parametrize("renorm", [0, 1])
def test_layer_matches_transformers_qwen3_moe_block(renorm):
    """Route + SwiGLU experts + gate-weighted combine == transformers' Qwen3-MoE sparse block."""
    E, k, H, I, T = 8, 2, 64, 32, 6
    rng = np.random.default_rng(11 + renorm)
    wr = (rng.standard_normal((E, H)) * 0.3).astype(np.float32)
    wg = rng.standard_normal((E, I, H)) * 0.05
    wu = rng.standard_normal((E, I, H)) * 0.05
    wd = rng.standard_normal((E, H, I)) * 0.05
    x = rng.standard_normal((T, H)).astype(np.float32).astype(np.float64)
    blk = _qwen3_block(E, k, H, I, renorm)
    with torch.no_grad():
        blk.gate.weight.copy_(torch.from_numpy(wr.astype(np.float64)))
        blk.experts.gate_up_proj.copy_(torch.from_numpy(np.concatenate([wg, wu], axis=1)))
        blk.experts.down_proj.copy_(torch.from_numpy(wd))
        ref = blk(torch.from_numpy(x)[None]).numpy()[0]
    z = router_logits(x, wr)
    idx, w = route(z, k, renorm)
    outs = moe_layer_dense(x, idx, lambda e: (wg[e], wu[e], wd[e]))
    y = moe_combine(outs, w)
    np.testing.assert_allclose(y, ref, rtol=2e-6, atol=2e-7 * np.abs(ref).max())


def test_single_expert_reduces_to_dense_swiglu_mlp():
    from transformers.models.qwen3_moe.configuration_qwen3_moe import Qwen3MoeConfig
    from transformers.models.qwen3_moe.modeling_qwen3_moe import Qwen3MoeMLP
    H, I = 48, 80
    rng = np.random.default_rng(5)
    wg, wu, wd = (rng.standard_normal((I, H)), rng.standard_normal((I, H)), rng.standard_normal((H, I)))
    x = rng.standard_normal((3, H))
    mlp = Qwen3MoeMLP(Qwen3MoeConfig(hidden_size=H, intermediate_size=I, hidden_act="silu")).double()
    with torch.no_grad():
        mlp.gate_proj.weight.copy_(torch.from_numpy(wg))
        mlp.up_proj.weight.copy_(torch.from_numpy(wu))
        mlp.down_proj.weight.copy_(torch.from_numpy(wd))
        ref = mlp(torch.from_numpy(x)).numpy()
    # E = 1, k = 1: the gate is softmax over one logit = 1
    idx, w = route(np.zeros((3, 1), np.float32), 1)
    assert np.all(w == 1.0)
    y = moe_combine(moe_layer_dense(x, idx, lambda e: (wg, wu, wd)), w)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    assert np.all(expert_ffn(x, 0 * wg, wu, wd) == 0)
    # swapping gate and up changes the result (silu is not symmetric)
    assert not np.allclose(expert_ffn(x, wu, wg, wd), ref)


def test_e2m1_table_and_dequant():
    g = json.load(open(os.path.join(GOLD, "e2m1_ocp.json")))
    mags = np.array(g["magnitudes_by_code"])
    codes = np.arange(16)
    vals = e2m1_decode(codes)
    np.testing.assert_array_equal(vals[:8], mags)
    np.testing.assert_array_equal(vals[8:], -mags)
    # pack: element 2i in the low nibble; scale per 32 elements along the row
    rng = np.random.default_rng(0)
    nib = rng.integers(0, 16, size=(3, 64))
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    sc = np.array([[0x3F80, 0x4040]] * 3, np.uint16)        # 1.0 and 3.0 in bf16
    w = dequant_fp4(packed, sc)
    np.testing.assert_array_equal(w[:, :32], e2m1_decode(nib[:, :32]))
    np.testing.assert_array_equal(w[:, 32:], 3.0 * e2m1_decode(nib[:, 32:]))


def test_bf16_widening_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x4049, 0x0001], np.uint16)
    v = bf16_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -1.0 and v[2] == 0.0 and np.signbit(v[3])
    assert v[4] == np.float32(3.140625) and v[5] == 2.0 ** -133


def test_full_residency_bitwise_and_exact_merge():
    """At full residency the cached path's partial sum equals all-resident bitwise; the hybrid
    GPU + CPU partial sums merge to the same output within fp64 rounding."""
    wl = W.TINY.with_(n_experts=16, top_k=3)
    full = OracleMoE(wl, n_slots=wl.n_keys, mode=MODE_OFFLOAD)
    hyb = OracleMoE(wl, n_slots=4, mode=MODE_HYBRID, bw_pcie=1, bw_host=4)
    for step in range(10):
        x = wl.decode_activations(step, 0)
        rf = full.decode_layer(0, x)
        if step > 3:
            assert np.array_equal(rf["y_split"], rf["y_exact"])
        rh = hyb.decode_layer(0, x)
        np.testing.assert_allclose(rh["y_split"], rh["y_exact"], rtol=1e-13, atol=1e-15)
        np.testing.assert_array_equal(rh["y"], rf["y"])


def test_mxfp4_equals_bf16_scaled_path_on_powers_of_two():
    """An E8M0 byte e is the bf16 bit pattern e << 7 (bf16 has fp32's 8-bit exponent and
    a 7-bit mantissa), so MXFP4 must dequantise exactly like the bf16-scale path fed
    those bits; and the E8M0 definition's fixed points: 127 -> 1, 0 -> 2^-127, 255 -> NaN."""
    from oracle import dequant_mxfp4, e8m0_decode
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 256, size=(6, 64), dtype=np.uint8)     # 6 rows x 128 elements
    e = rng.integers(1, 255, size=(6, 4)).astype(np.uint8)
    e[0, 0], e[1, 1], e[2, 2] = 1, 127, 254
    assert np.array_equal(dequant_mxfp4(codes, e), dequant_fp4(codes, (e.astype(np.uint16) << 7)))
    assert e8m0_decode(np.array([127]))[0] == 1.0 and e8m0_decode(np.array([0]))[0] == 2.0 ** -127
    assert e8m0_decode(np.array([130]))[0] == 8.0 and np.isnan(e8m0_decode(np.array([255]))[0])


def test_mxfp4_workload_records():
    """MXFP4 records: the FP4 codes of the same seed, one scale byte per 32 elements in the
    configured exponent range, packed as [codes x3 | scale bytes x3]."""
    import workloads as W
    wl = W.DSV4_MX.with_(n_layers=1, n_experts=2, hidden=256, inter=256)
    fp = W.DSV4.with_(n_layers=1, n_experts=2, hidden=256, inter=256)
    n = wl.hidden * wl.inter
    assert wl.record_bytes == 3 * (n // 2) + 3 * (n // 32)
    rec = wl.pack_record(1)
    for t in range(3):
        codes, sc = wl.expert_tensor(1, t)
        assert np.array_equal(codes, fp.expert_tensor(1, t)[0])
        assert sc.dtype == np.uint8 and sc.min() >= wl.mx_exp_lo and sc.max() <= wl.mx_exp_hi
        assert np.array_equal(rec[t * (n // 2):(t + 1) * (n // 2)], codes.reshape(-1))
        assert np.array_equal(rec[3 * (n // 2) + t * (n // 32):3 * (n // 2) + (t + 1) * (n // 32)], sc.reshape(-1))
    assert W.DSV4_MX.record_bytes == 13369344
