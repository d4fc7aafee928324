"""Pins of the oracle's storage codecs against the format definitions and torch's CPU
conversions (library routines): fp8-e4m3fn on all 256 codes, bf16 on all 65536 codes and on
a million random values with constructed ties, and the per-token fp8 quantizer."""
import math

import numpy as np
import pytest
import torch

import oracle
from synth.generate import to_bf16_bits, to_fp8_per_token


def test_fp8_table_matches_torch_all_codes():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    tab = oracle.fp8_e4m3_table()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(tab))
    assert nan.sum() == 2                               # 0x7F and 0xFF
    assert np.array_equal(tab[~nan], ref[~nan].astype(np.float64))
    # spot values straight from the definition
    assert tab[0x7E] == 448.0 and tab[0xFE] == -448.0
    assert tab[0x01] == 2.0 ** -9 and tab[0x07] == 7 * 2.0 ** -9
    assert tab[0x08] == 2.0 ** -6 and tab[0x38] == 1.0
    assert math.copysign(1.0, tab[0x80]) == -1.0 and tab[0x80] == 0.0


def test_fp8_encode_roundtrip_and_ties():
    tab = oracle.fp8_e4m3_table()
    finite = np.array([c for c in range(256) if not np.isnan(tab[c])], dtype=np.uint8)
    assert np.array_equal(oracle.encode_fp8_e4m3(tab[finite]), finite)
    # midpoints between neighbours go to the even code
    pos = tab[:127]
    mids = (pos[:-1] + pos[1:]) / 2
    codes = oracle.encode_fp8_e4m3(mids)
    lo = np.arange(126)
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(codes, expect.astype(np.uint8))
    # saturation and NaN
    assert oracle.encode_fp8_e4m3(np.array([1e6, -1e6, 449.0, 464.0]))[:4].tolist() == [0x7E, 0xFE, 0x7E, 0x7E]
    assert oracle.encode_fp8_e4m3(np.array([np.nan]))[0] == 0x7F


def test_fp8_encode_matches_torch_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000) * 50, rng.standard_normal(50000) * 1e-2,
                        rng.uniform(-448, 448, 50000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.encode_fp8_e4m3(x), ref)


def test_bf16_decode_all_codes():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    got = oracle.decode_bf16(bits)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(got[~nan], ref[~nan].astype(np.float64))


def test_bf16_encode_matches_torch_with_ties():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(1_000_000) * np.exp(rng.uniform(-30, 30, 1_000_000))).astype(np.float32)
    # exact ties: low 16 bits = 0x8000 with both parities of bit 16
    u = rng.integers(0, 2 ** 31, 20000, dtype=np.uint32) & np.uint32(0x7F7F0000)
    ties = (u | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    got = oracle.encode_bf16_rne(x)
    ref = to_bf16_bits(x)
    assert np.array_equal(got, ref)


def test_fp8_per_token_quantizer_matches_torch_route():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4096, 128)).astype(np.float32)
    x[5] = 0.0                                   # all-zero token gets scale 1
    x[6] *= 1e-30                                # tiny magnitudes
    codes, scale = oracle.quantize_fp8_per_token(x)
    c2, s2 = to_fp8_per_token(x)
    assert np.array_equal(scale, s2)
    assert np.array_equal(codes, c2)
    assert scale[5] == 1.0 and np.all(codes[5] == 0)
    # each token's largest magnitude maps to +-448 exactly
    big = np.abs(x[np.arange(4096) != 5]).argmax(axis=1)
    assert np.all(oracle.decode_fp8_e4m3(codes[np.arange(4096) != 5][np.arange(4095), big]) ** 2 == 448.0 ** 2)
