"""Pins of the oracle's scalar formats against closed forms and independent library casts.

The pages fix: E4M3 maximum 448 and the static P scale 1/448 ("SageAttention2 Technical
Report", 3.4 "FP8 Quantization for P~V"); the E2M1 value set and the 1x32 E8M0 MX block
("SageAttention3" summary, 3.4 "The NVFP4 Microscaling Format and Quantization Operator").
"""
import numpy as np
import pytest
import torch

import oracle

L = None


def setup_module(module):
    global L
    L = oracle.lib()


def test_e4m3_closed_form_values():
    dec = oracle.e4m3_decode_table()
    assert dec[0x7E] == 448.0                     # largest finite magnitude
    assert dec[0x01] == 2.0 ** -9                 # smallest subnormal (not 2^-10 as one page says)
    assert dec[0x08] == 2.0 ** -6                 # smallest normal
    assert dec[0x38] == 1.0
    assert np.isnan(dec[0x7F]) and np.isnan(dec[0xFF])
    assert dec[0x80] == 0.0 and np.signbit(dec[0x80])
    finite = dec[:127]
    assert np.all(np.diff(finite) > 0)            # codes 0..126 are increasing magnitudes
    assert np.count_nonzero(np.isnan(dec)) == 2   # no infinities, two NaNs


def test_e4m3_decode_matches_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    dec = oracle.e4m3_decode_table()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(dec))
    assert np.array_equal(ref[~nan], dec[~nan])


def test_e4m3_encode_roundtrip_and_ties():
    dec = oracle.e4m3_decode_table()
    for c in range(256):
        if np.isnan(dec[c]):
            continue
        assert L.orc_e4m3_encode(dec[c]) == c
    # every midpoint between neighbouring codes rounds to the even code
    for c in range(126):
        mid = 0.5 * (dec[c] + dec[c + 1])
        even = c if c % 2 == 0 else c + 1
        assert L.orc_e4m3_encode(mid) == even
        assert L.orc_e4m3_encode(-mid) == 0x80 | even


def test_e4m3_saturation_and_nan():
    assert L.orc_e4m3_encode(448.00003) == 0x7E
    assert L.orc_e4m3_encode(463.99) == 0x7E
    assert L.orc_e4m3_encode(1e9) == 0x7E
    assert L.orc_e4m3_encode(float("inf")) == 0x7E
    assert L.orc_e4m3_encode(-1e9) == 0xFE
    assert L.orc_e4m3_encode(float("nan")) == 0x7F


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.uniform(-464, 464, 20000), rng.uniform(-1, 1, 20000) * 2.0 ** -5,
                        rng.standard_normal(20000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([L.orc_e4m3_encode(float(v)) for v in x], np.uint8)
    assert np.array_equal(ref, got)


def test_e5m2_matches_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e5m2).double().numpy()
    dec = np.array([L.orc_e5m2_decode(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(dec))
    assert np.array_equal(ref[~nan], dec[~nan])
    rng = np.random.default_rng(8)
    x = np.concatenate([rng.uniform(-57000, 57000, 5000), rng.standard_normal(5000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e5m2).view(torch.uint8).numpy()
    got = np.array([L.orc_e5m2_encode(float(v)) for v in x], np.uint8)
    assert np.array_equal(ref, got)


def test_e2m1_value_set_and_rounding():
    vals = [L.orc_e2m1_decode(c) for c in range(16)]
    assert vals[:8] == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert vals[8:] == [-0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    for c in range(16):
        assert L.orc_e2m1_encode(vals[c]) == (c if c != 8 else 8)
    # ties to the even mantissa (even code)
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for x, code in ties.items():
        assert L.orc_e2m1_encode(x) == code, x
        assert L.orc_e2m1_encode(-x) == 8 | code, x
    assert L.orc_e2m1_encode(7.0) == 7 and L.orc_e2m1_encode(100.0) == 7
    assert L.orc_e2m1_encode(0.2) == 0 and L.orc_e2m1_encode(0.3) == 1


def test_e8m0_scale_rule():
    f = L.orc_e8m0_exponent
    assert f(6.0) == 0 and f(6.0000001) == 1 and f(3.0) == -1 and f(3.0000001) == 0
    assert f(0.0) == -127 and f(1.0) == -2 and f(1e-40) == -127
    for amax in np.geomspace(1e-30, 1e30, 200):
        e = f(amax)
        assert amax <= 6.0 * 2.0 ** e
        assert e == -127 or amax > 6.0 * 2.0 ** (e - 1)


def test_widening_all_codes():
    codes = np.arange(65536, dtype=np.uint16)
    ref16 = codes.view(np.float16).astype(np.float32)
    got16 = np.array([L.orc_fp16_to_f32(int(c)) for c in codes], np.float32)
    nan = np.isnan(ref16)
    assert np.array_equal(nan, np.isnan(got16))
    assert np.array_equal(ref16[~nan].view(np.uint32), got16[~nan].view(np.uint32))
    refb = torch.from_numpy(codes.astype(np.int16)).view(torch.bfloat16).float().numpy()
    gotb = np.array([L.orc_bf16_to_f32(int(c)) for c in codes], np.float32)
    nan = np.isnan(refb)
    assert np.array_equal(nan, np.isnan(gotb))
    assert np.array_equal(refb[~nan].view(np.uint32), gotb[~nan].view(np.uint32))


def test_k_group_map_matches_accumulator_layout():
    """Key rows held by one lane half of a 32x32 accumulator tile: {8b + 4h + k}."""
    groups = {}
    for t in range(64):
        groups.setdefault(L.orc_k_group(t), []).append(t)
    assert sorted(groups) == [0, 1, 2, 3]
    for T in range(2):
        for h in range(2):
            keys = sorted(32 * T + 8 * b + 4 * h + k for b in range(4) for k in range(4))
            assert groups[2 * T + h] == keys
    assert L.orc_k_group(64 + 5) == L.orc_k_group(5)
