"""Pins of the oracle's number formats against the format specifications, torch's
own float8 / bf16 casts and hand-worked cases.  CPU only."""
import os

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _read(name):
    rows = []
    for line in open(os.path.join(GOLD, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append(line.split())
    return rows


def test_e2m1_table_matches_spec():
    for code, val in _read("e2m1_values.txt"):
        v = float(val)
        got = F.E2M1[int(code)]
        assert got == v and np.signbit(got) == np.signbit(v), (code, got, v)


def test_e4m3_specials_match_spec():
    for code, val in _read("e4m3_specials.txt"):
        got = F.E4M3[int(code, 16)]
        if val == "nan":
            assert np.isnan(got)
        else:
            assert got == float(val) and np.signbit(got) == np.signbit(float(val))
    assert np.isnan(F.E4M3).sum() == 2


def test_e4m3_table_matches_torch_cast():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    fin = ~np.isnan(ref)
    assert np.array_equal(F.E4M3[fin], ref[fin])
    assert np.array_equal(np.isnan(F.E4M3), ~fin)


def test_e4m3_encode_roundtrip_all_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    back = F.e4m3_encode(F.E4M3[codes])
    # -0.0 encodes to 0x80, so every finite code round-trips
    assert np.array_equal(back, codes)


def test_e4m3_encode_rne_matches_torch():
    rng = np.random.default_rng(0)
    # values inside the finite range, on many binades, including subnormals
    x = (rng.uniform(-1, 1, 200000) * np.exp2(rng.integers(-14, 9, 200000))).astype(np.float32)
    x = x[np.abs(x) < 464.0]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.e4m3_encode(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_e4m3_encode_ties_and_saturation():
    cases = {
        448.0: 0x7E, 464.0: 0x7E, 500.0: 0x7E, 1e9: 0x7E, -1e4: 0xFE,
        2.0 ** -10: 0x00,            # half the smallest subnormal: tie to even (0)
        1.5 * 2.0 ** -9: 0x02,       # 1.5 steps: tie to even (2 steps)
        2.5 * 2.0 ** -9: 0x02,       # 2.5 steps: tie to even (2 steps)
        1.0625: 0x38,                # halfway between 1 and 1.125 -> even mantissa (1.0)
        1.1875: 0x3A,                # halfway between 1.125 and 1.25 -> 1.25
        240.0: 0x77, 0.0: 0x00,
    }
    for v, c in cases.items():
        assert int(F.e4m3_encode(np.array([v]))[0]) == c, (v, c)


def test_e8m0_values():
    assert F.e8m0_value(np.array([127]))[0] == 1.0
    assert F.e8m0_value(np.array([120]))[0] == 2.0 ** -7
    assert F.e8m0_value(np.array([130]))[0] == 8.0
    assert F.e8m0_value(np.array([0]))[0] == 2.0 ** -127
    assert np.isnan(F.e8m0_value(np.array([255]))[0])


def test_bf16_encode_matches_torch():
    rng = np.random.default_rng(1)
    x = (rng.normal(0, 1, 100000) * np.exp2(rng.integers(-20, 20, 100000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.bf16_encode(x.astype(np.float64)), ref)
    # and decoding is the float32 with the low 16 bits cleared
    back = torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(F.bf16_value(ref), back)


def test_mx_quantize_worked_blocks():
    # amax 448: floor(log2 448) = 8 -> X = 8 - 8 + 127 = 127, elements unchanged
    v = np.zeros(32); v[0] = 448.0; v[1] = -3.0
    c, X = F.mx_e4m3_quantize(v.astype(np.float32).astype(np.float64))
    assert X.tolist() == [127] and c[0] == 0x7E and c[1] == F.e4m3_encode(np.array([-3.0]))[0]
    # amax 5: floor(log2 5) = 2 -> X = 121, 5 * 2^6 = 320 = 1.25 * 2^8 -> code 0x7A
    v = np.zeros(32); v[3] = 5.0
    c, X = F.mx_e4m3_quantize(v)
    assert X.tolist() == [121] and c[3] == 0x7A
    assert F.mx_e4m3_dequant_act(c, X)[3] == 5.0
    # all-zero block -> X = 0, zero codes
    c, X = F.mx_e4m3_quantize(np.zeros(64))
    assert X.tolist() == [0, 0] and not c.any()
    # amax 7.5: floor(log2) = 2, X = 121, 7.5 * 64 = 480 > 448 saturates (the OCP MX rule)
    v = np.zeros(32); v[0] = 7.5
    c, X = F.mx_e4m3_quantize(v)
    assert X.tolist() == [121] and c[0] == 0x7E


def test_mx_quantize_exact_on_grid():
    rng = np.random.default_rng(2)
    codes = rng.integers(0, 256, size=(4, 128)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x30
    blockscale = rng.integers(100, 140, size=(4, 4))
    v = F.E4M3[codes] * np.repeat(np.exp2(blockscale - 127.0), 32, axis=1)
    c2, X2 = F.mx_e4m3_quantize(v)
    np.testing.assert_array_equal(F.mx_e4m3_dequant_act(c2, X2), v)


def test_dequant_mxfp4_hand():
    packed = np.array([[0x7A, 0x21] + [0x00] * 14], dtype=np.uint8)  # 32 values
    s = np.array([[129]], dtype=np.uint8)  # x4
    v = F.dequant_mxfp4(packed, s)
    assert v.shape == (1, 32)
    # byte 0x7A: low nibble 0xA = -1.0 (even k), high 0x7 = 6.0 (odd k)
    assert v[0, :4].tolist() == [-4.0, 24.0, 2.0, 4.0]
    assert not v[0, 4:].any()


def test_dequant_tiles_against_torch_decode():
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 256, size=(64, 96)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0
    s8 = rng.integers(120, 135, size=(2, 3)).astype(np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for i in range(64):
        for j in range(96):
            ref[i, j] *= 2.0 ** (int(s8[i // 32, j // 32]) - 127)
    np.testing.assert_array_equal(F.dequant_mxfp8_weight(codes, s8), ref)
    codes = rng.integers(0, 256, size=(256, 128)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0
    sf = rng.uniform(0.5, 2, size=(2, 1)).astype(np.float32)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ref = ref * np.float64(sf[np.arange(256)[:, None] // 128, 0])
    np.testing.assert_array_equal(F.dequant_fp8_block128(codes, sf), ref)
