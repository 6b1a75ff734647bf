"""Pins for the oracle's E4M3 decoding of fp8 caches (CPU only).  The pages leave low-bit KV as future
work ([paper] Limitations, fp8); the format is the OCP 8-bit floating-point E4M3 (FN variant)."""
import numpy as np
import torch

from oracle import prr_oracle as orc

ALL = np.arange(256, dtype=np.uint8)


def test_decode_matches_torch_float8_e4m3fn():
    ours = orc.fp8_e4m3_decode(ALL)
    ref = torch.from_numpy(ALL.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])


def test_known_codes():
    vals = {0x00: 0.0, 0x38: 1.0, 0x40: 2.0, 0xC0: -2.0, 0x7E: 448.0, 0xFE: -448.0, 0x01: 2.0 ** -9,
            0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x3C: 1.5, 0x30: 0.5, 0x4B: 5.5}
    for code, v in vals.items():
        assert orc.fp8_e4m3_decode([code])[0] == v, hex(code)
    assert np.signbit(orc.fp8_e4m3_decode([0x80])[0]) and orc.fp8_e4m3_decode([0x80])[0] == 0.0
    assert np.isnan(orc.fp8_e4m3_decode([0x7F])[0]) and np.isnan(orc.fp8_e4m3_decode([0xFF])[0])


def test_positive_codes_increase_and_negatives_mirror():
    pos = orc.fp8_e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)
    neg = orc.fp8_e4m3_decode(np.arange(0x80, 0xFF, dtype=np.uint8))
    assert np.array_equal(neg, -pos)


def test_every_finite_code_is_a_bf16_value():
    """Converting an fp8 key or value to bf16 (as the GPU does before its bf16 products) is exact."""
    v = orc.fp8_e4m3_decode(ALL)
    v = v[~np.isnan(v)].astype(np.float32)
    trunc = (v.view(np.uint32) & 0xFFFF0000).view(np.float32)
    assert np.array_equal(trunc, v)


def test_upcast_of_an_fp8_cache():
    codes = np.array([[0x38, 0xC0], [0x01, 0x7E]], dtype=np.uint8)
    assert np.array_equal(orc.upcast(codes, "fp8"), [[1.0, -2.0], [2.0 ** -9, 448.0]])
    # queries and min/max metadata of an fp8 cache are bf16 bit patterns
    bf = np.array([0x3F80, 0xC000], dtype=np.uint16)
    assert np.array_equal(orc.upcast(bf, "fp8"), [1.0, -2.0])
