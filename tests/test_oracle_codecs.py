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


# ---- fp8 latent KV rows (per token, per 128-column tile, power-of-two scale) --------------

def test_kv_tile_scale_is_the_smallest_sufficient_power_of_two():
    """Checked in exact float64 arithmetic from the definition: 448 * s covers the tile's
    maximum, half of s does not (unless s is the floor 2^-126), and s is a power of two."""
    rng = np.random.default_rng(5)
    a = np.concatenate([
        (rng.standard_normal(200000) * np.exp(rng.uniform(-80, 80, 200000))),
        448.0 * np.ldexp(1.0, np.arange(-130, 120)),            # boundaries: 448 * 2^k
        1.75 * np.ldexp(1.0, np.arange(-130, 120)),              # mantissa exactly 1.75
        np.nextafter(np.float32(448.0) * np.ldexp(np.float32(1), np.arange(-20, 20)).astype(np.float32),
                     np.float32(np.inf)),                        # just above a boundary
        [1e-45, 1e-40, 1e-38, 3.4e38, 1.0, 448.0, 449.0],
    ]).astype(np.float32)
    a = np.abs(a[np.isfinite(a) & (a != 0)])
    s = oracle.kv_fp8_tile_scale(a).astype(np.float64)
    af = a.astype(np.float64)
    m, _ = np.frexp(s)
    assert np.all(m == 0.5)                                      # powers of two
    assert np.all(af <= 448.0 * s)
    floor = s == 2.0 ** -126
    assert np.all(floor | (af > 448.0 * s / 2))
    assert np.all(s >= 2.0 ** -126)
    assert oracle.kv_fp8_tile_scale(np.float32([0.0]))[0] == 1.0


def test_kv_fp8_rows_roundtrip_representable_values():
    """Rows built from e4m3 values times a power of two, each tile holding a +-448 code so
    that its scale is forced: quantizing the decoded row gives the same bytes back, and the
    byte layout (codes, bf16 rope, fp32 scales) is the documented one."""
    rng = np.random.default_rng(6)
    n = 64
    finite = np.arange(0, 127)                                   # +0 .. +448
    codes = rng.choice(finite, size=(n, 512)) | (rng.integers(0, 2, (n, 512)) << 7)
    codes[:, ::128] = 0x7E | (rng.integers(0, 2, (n, 4)) << 7)   # |448| in every tile
    e = rng.integers(-20, 20, size=(n, 4))
    scale = np.ldexp(1.0, e).astype(np.float32)
    nope = oracle.decode_fp8_e4m3(codes.astype(np.uint8)).reshape(n, 4, 128) * scale[:, :, None]
    rope_bits = to_bf16_bits(rng.standard_normal((n, 64)).astype(np.float32))
    x = np.concatenate([nope.reshape(n, 512), oracle.decode_bf16(rope_bits)], axis=1).astype(np.float32)
    rows = oracle.quantize_kv_fp8_rows(x)
    assert rows.shape == (n, oracle.KV_FP8_ROW_BYTES)
    assert np.array_equal(rows[:, :512], codes.astype(np.uint8))
    assert np.array_equal(rows[:, 512:640].copy().view("<u2"), rope_bits)
    assert np.array_equal(rows[:, 640:].copy().view("<f4"), scale)
    assert np.array_equal(oracle.decode_kv_fp8_rows(rows), x.astype(np.float64))


def test_kv_fp8_codes_are_the_nearest_e4m3_values():
    """Brute force over the 253 finite e4m3 values: every code decodes to a nearest value of
    x / scale (ties to the even code), and no tile saturates."""
    rng = np.random.default_rng(7)
    n = 200
    x = (rng.standard_normal((n, 576)) * np.exp(rng.uniform(-6, 6, (n, 1)))).astype(np.float32)
    x[3, :128] = 0.0                                             # all-zero tile: scale 1
    rows = oracle.quantize_kv_fp8_rows(x)
    scale = rows[:, 640:].copy().view("<f4").astype(np.float64)
    assert scale[3, 0] == 1.0 and np.all(rows[3, :128] == 0)
    q = x[:, :512].astype(np.float64).reshape(n, 4, 128) / scale[:, :, None]
    assert np.abs(q).max() <= 448.0
    table = oracle.fp8_e4m3_table()
    vals = table[np.isfinite(table)]
    got = oracle.decode_fp8_e4m3(rows[:, :512]).reshape(n, 4, 128)
    d = np.abs(q[..., None] - vals[None, None, None, :])
    best = d.min(axis=-1)
    assert np.array_equal(np.abs(q - got), best)
    # dequantized error bound: half the e4m3 spacing at the top binade, times the scale
    deq = oracle.decode_kv_fp8_rows(rows)
    err = np.abs(deq[:, :512] - x[:, :512]).reshape(n, 4, 128)
    assert np.all(err <= 16.0 * scale[:, :, None])
    assert np.array_equal(deq[:, 512:], oracle.decode_bf16(to_bf16_bits(x[:, 512:])))


# ---- MXFP8 (groups of 32, E8M0 power-of-two scales) -----------------------------------------

def test_mx_scale_byte_is_floor_log2_minus_8():
    """Checked in exact float64 from the definition: 2^(e + 8) <= amax < 2^(e + 9) for the
    scale 2^e, unless clamped at the ends of the E8M0 range; 0 for an all-zero group."""
    rng = np.random.default_rng(8)
    a = np.concatenate([
        np.abs(rng.standard_normal(100000) * np.exp(rng.uniform(-85, 85, 100000))),
        np.ldexp(1.0, np.arange(-149, 128)),                   # exact powers of two
        np.nextafter(np.ldexp(np.float32(1), np.arange(-100, 100)).astype(np.float32), np.float32(0)),
    ]).astype(np.float32)
    a = a[np.isfinite(a) & (a > 0)]
    e = oracle.mx_scale_bytes(a).astype(np.int64) - 127
    af = a.astype(np.float64)
    inner = (e > -127) & (e < 127)
    assert np.all(np.ldexp(1.0, e[inner] + 8) <= af[inner])
    assert np.all(af[inner] < np.ldexp(1.0, e[inner] + 9))
    assert np.all(af[e == -127] < 2.0 ** -118)
    assert oracle.mx_scale_bytes(np.float32([0.0]))[0] == 0


def test_mx_codes_are_the_nearest_clamped_e4m3_values():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((300, 128)) * np.exp(rng.uniform(-5, 5, (300, 1)))).astype(np.float32)
    x[7, :32] = 0.0
    codes, sb = oracle.quantize_mxfp8(x)
    assert codes.shape == x.shape and sb.shape == (300, 4)
    scale = np.ldexp(1.0, sb.astype(np.int64) - 127)
    q = np.clip(x.astype(np.float64).reshape(300, 4, 32) / scale[..., None], -448.0, 448.0)
    table = oracle.fp8_e4m3_table()
    vals = table[np.isfinite(table)]
    got = oracle.decode_fp8_e4m3(codes).reshape(300, 4, 32)
    best = np.abs(q[..., None] - vals).min(axis=-1)
    assert np.array_equal(np.abs(q - got), best)
    assert np.all(codes[7, :32] == 0)
    assert np.array_equal(oracle.decode_mxfp8(codes, sb), got.reshape(300, 128) * np.repeat(scale, 32, axis=1))


def test_mx_is_lossless_on_small_integers():
    """Integers in [-8, 8]: the group scale is at most 2^-5 and every value times 32 is an
    e4m3 value, so quantizing loses nothing."""
    rng = np.random.default_rng(10)
    x = rng.integers(-8, 9, size=(500, 128)).astype(np.float32)
    assert np.array_equal(oracle.decode_mxfp8(*oracle.quantize_mxfp8(x)), x.astype(np.float64))
