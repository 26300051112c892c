"""Expert bank file (no GPU needed): records written from the seeded generator come back
byte for byte through parallel direct and buffered reads, and malformed or mismatched
files are refused."""
import os

import numpy as np
import pytest

import workloads as W

WL = W.A3B_DECODE.with_(name="bank_bf16", n_layers=2, n_experts=8, hidden=256, inter=128)   # 192 KiB records
MX = W.DSV4_MX.with_(name="bank_mx", n_layers=2, n_experts=6, hidden=512, inter=256, alias_records=5)


def _cfg(R, wl):
    return R.make_config(wl.n_layers, wl.n_experts, wl.top_k, wl.hidden, wl.inter, wl.wfmt, wl.afmt, 1,
                         R.MOE_MODE_OFFLOAD)


def _pool(wl):
    buf = np.empty(wl.pool_records * wl.record_bytes, np.uint8)
    wl.fill_pool(buf.ctypes.data, 0, wl.pool_records)
    return buf


def _aligned(n, offset=0):
    raw = np.empty(n + 8192, np.uint8)
    start = (-raw.ctypes.data) % 4096 + offset
    return raw[start:start + n]


@pytest.mark.parametrize("wl", [WL, MX], ids=["bf16", "mxfp4_aliased"])
@pytest.mark.parametrize("threads", [1, 3, 8])
def test_bank_round_trip(tmp_path, wl, threads):
    import routed_expert_ffn_02_amd as R
    cfg = _cfg(R, wl)
    pool = _pool(wl)
    path = str(tmp_path / "experts.bank")
    R.moe_bank_write(path, cfg, pool, wl.pool_records)
    info = R.moe_bank_info(path)
    assert info == {"n_layers": wl.n_layers, "n_experts": wl.n_experts, "hidden": wl.hidden, "inter": wl.inter,
                    "wfmt": wl.wfmt, "record_bytes": wl.record_bytes, "n_records": wl.pool_records}
    assert os.path.getsize(path) == 4096 + pool.size
    # page-aligned destination: O_DIRECT where the file system allows it; the bytes must match either way
    dst = _aligned(pool.size)
    st = R.moe_bank_read(path, cfg, dst, dst.size, threads)
    assert np.array_equal(dst, pool) and st["bytes"] == pool.size and st["threads"] == threads
    # unaligned destination: O_DIRECT through the bounce buffers (or buffered reads)
    dst2 = _aligned(pool.size, offset=8)
    st2 = R.moe_bank_read(path, None, dst2, dst2.size, threads)
    assert np.array_equal(dst2, pool) and st2["mode"] in ("direct_bounce", "buffered")
    # every record is the generator's record of its key
    for key in range(wl.pool_records):
        rec = dst[key * wl.record_bytes:(key + 1) * wl.record_bytes]
        assert np.array_equal(rec, wl.pack_record(key))


def test_bank_refuses_mismatch_and_damage(tmp_path):
    import routed_expert_ffn_02_amd as R
    cfg = _cfg(R, WL)
    pool = _pool(WL)
    path = str(tmp_path / "experts.bank")
    R.moe_bank_write(path, cfg, pool, WL.pool_records)
    dst = _aligned(pool.size)
    other = R.make_config(WL.n_layers, WL.n_experts, WL.top_k, WL.hidden, WL.inter * 2, WL.wfmt, WL.afmt, 1,
                          R.MOE_MODE_OFFLOAD)
    with pytest.raises(R.MoeError):
        R.moe_bank_read(path, other, dst, dst.size, 2)                 # shape mismatch
    with pytest.raises(R.MoeError):
        R.moe_bank_read(path, cfg, dst, dst.size - 1, 2)               # short buffer
    with pytest.raises(R.MoeError):
        R.moe_bank_read(path, cfg, dst, dst.size, 0)                   # no reader threads
    trunc = str(tmp_path / "trunc.bank")
    with open(path, "rb") as f, open(trunc, "wb") as g:
        g.write(f.read()[:-1])
    with pytest.raises(R.MoeError):
        R.moe_bank_info(trunc)                                         # truncated records
    bad = str(tmp_path / "bad.bank")
    data = bytearray(open(path, "rb").read())
    data[0] ^= 0xFF
    open(bad, "wb").write(bytes(data))
    with pytest.raises(R.MoeError):
        R.moe_bank_info(bad)                                           # wrong magic
    with pytest.raises(R.MoeError):
        R.moe_bank_info(str(tmp_path / "missing.bank"))
