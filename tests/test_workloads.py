"""The input generator: determinism, distributions, pool format sizes (no method arithmetic)."""
import json
import os

import numpy as np

import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_pool_sizes_match_pages():
    g = json.load(open(os.path.join(GOLD, "pool_sizes.json")))
    a3b = W.A3B_DECODE
    pool = a3b.record_bytes * a3b.n_keys
    assert pool == 40 * 256 * 3 * 2048 * 512 * 2
    assert abs(pool / 1e9 - g["a3b_pool_gb"]) < 0.05
    t = pool / (g["a3b_bw_pcie_gbs"] * 1e9)
    assert g["a3b_prefill_seconds"][0] - 0.01 <= t <= g["a3b_prefill_seconds"][1] + 0.01
    d = W.DSV4
    assert (d.n_layers, d.n_experts, d.top_k) == (g["dsv4_layers"], g["dsv4_experts"], g["dsv4_top_k"])
    assert d.record_bytes == 3 * 4096 * 2048 // 2 + 3 * 4096 * 2048 // 32 * 2


def test_generator_deterministic_and_distributed():
    w = W.A3B_DECODE
    a = W.bf16_bits_to_f32(w.expert_tensor(17, 2)).astype(np.float64)
    b = W.bf16_bits_to_f32(w.expert_tensor(17, 2)).astype(np.float64)
    c = W.bf16_bits_to_f32(w.expert_tensor(18, 2)).astype(np.float64)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    assert abs(a.mean()) < 1e-4 and abs(a.std() - 0.02) < 2e-4
    x = W.bf16_bits_to_f32(w.decode_activations(3, 5)).astype(np.float64)
    assert x.shape == (1, 2048) and abs(x.std() - 1.0) < 0.05
    f = W.TINY.expert_tensor(3, 0)
    assert f.dtype == np.float32 and abs(float(f.std()) - 0.02) < 2e-3


def test_record_packing_matches_logical_tensors():
    for wl in (W.TINY, W.A3B_DECODE.with_(hidden=64, inter=96), W.DSV4.with_(hidden=64, inter=96)):
        rec = wl.pack_record(5)
        off = 0
        parts = [wl.expert_tensor(5, t) for t in range(3)]
        if wl.wfmt == W.WFMT_FP4:
            for codes, _ in parts:
                assert np.array_equal(rec[off:off + codes.size], codes.reshape(-1)); off += codes.size
            for _, sc in parts:
                n = sc.size * 2
                assert np.array_equal(rec[off:off + n].view(np.uint16), sc.reshape(-1)); off += n
        else:
            for p in parts:
                n = p.nbytes
                assert np.array_equal(rec[off:off + n], p.reshape(-1).view(np.uint8)); off += n
        assert off == wl.record_bytes
        pool = np.zeros(3 * wl.record_bytes, np.uint8)
        wl.fill_pool(pool.ctypes.data, 4, 3, threads=2)
        assert np.array_equal(pool[wl.record_bytes:2 * wl.record_bytes], rec)


def test_alias_maps_to_backing_record():
    wl = W.A3B_DECODE.with_(hidden=64, inter=96, alias_records=10)
    assert np.array_equal(wl.expert_tensor(23, 1), wl.expert_tensor(3, 1))
    assert wl.pool_records == 10


def test_zipf_bias_shape():
    w = W.A3B_DECODE
    b = w.zipf_bias(0)
    p = np.exp(b.astype(np.float64) / w.zipf_alpha)
    assert abs(p.sum() - 1.0) < 1e-5          # exp(bias / alpha) is the Zipf(1.1) pmf over ranks
    ranks = w.popularity_perm(0) + 1.0
    np.testing.assert_allclose(p, ranks ** -1.1 / np.sum(np.arange(1, 257) ** -1.1), rtol=1e-5)
    assert sorted(w.popularity_perm(0).tolist()) == list(range(256))


def test_locality_constants_match_calibration():
    """The frozen routing constants are the ones the committed calibration chose."""
    cal = json.load(open(os.path.join(os.path.dirname(W.__file__), "calibration.json")))
    assert cal["chosen"]["zipf_alpha"] == W.ZIPF_ALPHA and cal["chosen"]["prev_bonus"] == W.PREV_BONUS
    assert cal["chosen"]["prefill_coverage"] >= 0.95
    assert W.A3B_DECODE.zipf_alpha == W.ZIPF_ALPHA and W.DSV4.prev_bonus == W.PREV_BONUS
