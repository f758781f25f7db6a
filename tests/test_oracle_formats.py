"""Pins for the oracle's storage formats (FP8 E4M3FN, bf16, fp16, packed codes).

The FP8 and bf16 encoders are checked against their definitions (known code
values, ties to even, saturation) and against torch's independent CPU casts.
"""

import numpy as np
import pytest
import torch

from oracle.formats import (
    FP8_E4M3FN_VALUES,
    bf16_round,
    fp16_round,
    fp8_e4m3fn_decode,
    fp8_e4m3fn_encode,
    pack_codes,
    unpack_codes,
)


def test_fp8_known_codes():
    v = FP8_E4M3FN_VALUES
    assert v[0x00] == 0.0
    assert v[0x01] == 2.0 ** -9  # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9  # largest subnormal
    assert v[0x08] == 2.0 ** -6  # smallest normal
    assert v[0x38] == 1.0
    assert v[0x39] == 1.125
    assert v[0x7E] == 448.0  # largest finite
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert v[0xFE] == -448.0 and v[0xB8] == -1.0
    finite = np.isfinite(v)
    assert finite.sum() == 254
    assert np.all(np.diff(v[:0x7F]) > 0)


def test_fp8_roundtrip_all_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    back = fp8_e4m3fn_encode(fp8_e4m3fn_decode(codes))
    assert np.array_equal(back, codes)


def test_fp8_ties_to_even_and_saturation():
    x = np.array([1.0625, 1.1875, 1.5 * 2 ** -9, 0.5 * 2 ** -9, 2.5 * 2 ** -9, 460.0, 1000.0, -1e9, -0.0, -1e-6])
    want = np.array([0x38, 0x3A, 0x02, 0x00, 0x02, 0x7E, 0x7E, 0xFE, 0x80, 0x80], dtype=np.uint8)
    assert np.array_equal(fp8_e4m3fn_encode(x), want)


def test_fp8_matches_torch_in_range():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(20000) * 4.0,
        rng.standard_normal(5000) * 0.01,
        rng.uniform(-440, 440, 5000),
        # exact midpoints between neighbouring codes
        (FP8_E4M3FN_VALUES[1:0x7E] + FP8_E4M3FN_VALUES[2:0x7F]) / 2.0,
    ]).astype(np.float32)
    ours = fp8_e4m3fn_encode(x)
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_bf16_matches_torch():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    # values exactly half way between two bf16 numbers
    base = torch.from_numpy(x[:1000]).to(torch.bfloat16).to(torch.float32).numpy()
    half = (base.view(np.uint32) + np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, half])
    ours = bf16_round(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), theirs.view(np.uint32))


def test_fp16_ties():
    # 1 + 2^-11 is half way between 1 and 1 + 2^-10: ties to even gives 1
    assert fp16_round(1.0 + 2.0 ** -11) == 1.0
    assert fp16_round(1.0 + 3 * 2.0 ** -11) == 1.0 + 2 * 2.0 ** -10


def test_pack_bit_order():
    assert pack_codes(np.array([1, 2]), 4).tolist() == [0x21]
    assert pack_codes(np.array([1, 2, 3, 0]), 2).tolist() == [0x39]
    rng = np.random.default_rng(0)
    for bits in (2, 4):
        q = rng.integers(0, 2 ** bits, size=(5, 64)).astype(np.uint8)
        b = pack_codes(q, bits)
        assert b.shape == (5, 64 * bits // 8)
        assert np.array_equal(unpack_codes(b, bits), q)


def test_pack_rejects_other_widths():
    with pytest.raises(ValueError):
        pack_codes(np.zeros(8), 3)
