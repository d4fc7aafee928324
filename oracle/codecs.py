"""Exact decoding (and, for the cache-store helpers, encoding) of the stored formats.

TEST INFRASTRUCTURE (see the package header).

Formats:
* bf16: the upper 16 bits of an IEEE binary32; decoding shifts the bits up by 16.
* fp8-e4m3, OCP "fn" variant: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
  exponent field 0 encodes subnormals m * 2^-9; S.1111.111 is NaN; there is no infinity;
  the largest finite magnitude is 448.
* Per-token fp8 quantization of indexer keys (the quantized indexer path of "Day0
  Adaptation and Performance Optimization for Novel Long-Sequence Reasoning Models",
  section 3, with the per-token fp32 scale of this project's quantized workloads): the scale
  is the token's largest magnitude divided by 448 in fp32 (an all-zero token gets 1), the
  code is the fp32 quotient value/scale rounded to the nearest e4m3 value, ties to the even
  code, magnitudes above 448 saturating to 448.
* fp8 latent KV rows for SFA, quantized per token and per tile of 128 columns ("Day0
  Adaptation and Performance Optimization for Novel Long-Sequence Reasoning Models", section
  4; "Large Model Inference Acceleration: Day-0 Adaptation...", section 2.2).  The pages fix
  the granularity, not the scale's format; the reading taken here: the scale of a tile is the
  smallest power of two 2^e (e >= -126) with max|x| <= 448 * 2^e over the tile (1 for an
  all-zero tile), the code is x / scale (exact) rounded to the nearest e4m3 value, ties to
  the even code; the 64 rope columns of the 576-wide latent row stay in bf16.  A row is 656
  bytes: 512 codes, 64 bf16 (little-endian), then the four scales as fp32.
* MXFP8 with groups of 32 for the indexer's queries and keys ("Day0 Adaptation and
  Performance Optimization for Novel Long-Sequence Reasoning Models", section 4; "Day0
  Adaptation and Sparse Attention Optimization for Long-Sequence LLM Inference", section 5;
  "Optimizing and Deploying Ultra-Long Sequence Inference Architectures", section II), read
  as the OCP microscaling format: every 32 consecutive elements share an E8M0 scale byte s,
  the value 2^(s - 127); s = floor(log2(max|x|)) - 8 + 127 over the group (8 is the exponent
  of e4m3's largest power of two), clamped to [0, 254], and 0 for an all-zero group; each
  code is x / 2^(s - 127) (exact) rounded to the nearest e4m3 value, ties to the even code,
  saturating at +-448.
"""
from __future__ import annotations

import numpy as np


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bits -> float64 (exact)."""
    u32 = bits.astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u32.view(np.float32).astype(np.float64)


def fp8_e4m3_table() -> np.ndarray:
    """float64 value of each of the 256 e4m3fn codes, built from the format definition."""
    vals = np.empty(256, dtype=np.float64)
    for c in range(256):
        sign = -1.0 if (c >> 7) & 1 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = sign * m * 2.0 ** -9
        else:
            vals[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_FP8_TABLE = fp8_e4m3_table()


def decode_fp8_e4m3(codes: np.ndarray) -> np.ndarray:
    """uint8 e4m3fn codes -> float64 (exact)."""
    return _FP8_TABLE[codes.astype(np.intp)]


def decode(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Stored tensor -> float64, dtype in {f32, bf16, fp8} (fp8 without its scale), or
    fp8_rows for the tile-quantized latent rows (with their scales)."""
    if dtype == "f32":
        return arr.astype(np.float64)
    if dtype == "bf16":
        return decode_bf16(arr)
    if dtype == "fp8":
        return decode_fp8_e4m3(arr)
    if dtype == "fp8_rows":
        return decode_kv_fp8_rows(arr)
    raise ValueError(dtype)


def encode_bf16_rne(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest, ties to even (NaN -> quiet NaN)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) & np.uint64(0xFFFF)
    out = r.astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    out[nan] = np.uint16(0x7FC0) | (((u[nan] >> np.uint64(16)) & np.uint64(0x8000)).astype(np.uint16))
    return out


_POS_CODES = np.arange(0, 127, dtype=np.int64)          # +0 ... +448 (0x7E)
_POS_VALS = _FP8_TABLE[:127]                            # strictly increasing


def encode_fp8_e4m3(x: np.ndarray) -> np.ndarray:
    """float64/float32 -> e4m3fn codes: nearest value, ties to the even code, saturating
    magnitudes above 448 to 448; NaN -> 0x7F; the sign of zero is kept."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    hi = np.searchsorted(_POS_VALS, a, side="left")     # first value >= a
    hi = np.clip(hi, 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_hi = _POS_VALS[hi] - a
    d_lo = a - _POS_VALS[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    code = code | np.where(np.signbit(x), 0x80, 0)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)


def quantize_fp8_per_token(x: np.ndarray):
    """float32 [n, D] -> (uint8 codes [n, D], float32 scales [n])."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=1)
    scale = np.divide(amax, np.float32(448.0), dtype=np.float32)
    scale = np.where(amax == 0, np.float32(1.0), scale).astype(np.float32)
    quot = np.divide(x, scale[:, None], dtype=np.float32)
    return encode_fp8_e4m3(quot), scale


KV_FP8_ROW_BYTES = 656
KV_NOPE = 512
KV_TILE = 128


def kv_fp8_tile_scale(amax: np.ndarray) -> np.ndarray:
    """float32 tile maxima -> float32 scales: the smallest power of two 2^e, e >= -126, with
    amax <= 448 * 2^e; 1 where amax == 0.  With amax = f * 2^k, 0.5 <= f < 1 (frexp, exact):
    448 * 2^e = 0.875 * 2^(e + 9), so e = k - 9 when f <= 0.875 and k - 8 otherwise."""
    a = np.asarray(amax, dtype=np.float32).astype(np.float64)
    f, k = np.frexp(a)
    e = np.where(f > 0.875, k - 8, k - 9)
    e = np.maximum(e, -126)
    out = np.ldexp(1.0, e).astype(np.float32)
    return np.where(a == 0.0, np.float32(1.0), out).astype(np.float32)


def quantize_kv_fp8_rows(x: np.ndarray) -> np.ndarray:
    """float32 [n, 576] latent rows -> uint8 [n, 656] fp8 rows (format above)."""
    x = np.asarray(x, dtype=np.float32)
    n = x.shape[0]
    tiles = x[:, :KV_NOPE].reshape(n, KV_NOPE // KV_TILE, KV_TILE)
    scale = kv_fp8_tile_scale(np.max(np.abs(tiles), axis=2))
    quot = np.divide(tiles, scale[:, :, None], dtype=np.float32)
    out = np.empty((n, KV_FP8_ROW_BYTES), dtype=np.uint8)
    out[:, :KV_NOPE] = encode_fp8_e4m3(quot).reshape(n, KV_NOPE)
    out[:, KV_NOPE:640] = encode_bf16_rne(x[:, KV_NOPE:]).astype("<u2").view(np.uint8)
    out[:, 640:] = scale.astype("<f4").view(np.uint8)
    return out


def decode_kv_fp8_rows(rows: np.ndarray) -> np.ndarray:
    """uint8 [n, 656] fp8 rows -> float64 [n, 576] (exact: code * scale, bf16 rope)."""
    rows = np.ascontiguousarray(rows, dtype=np.uint8)
    n = rows.shape[0]
    scale = rows[:, 640:].copy().view("<f4").astype(np.float64)
    nope = decode_fp8_e4m3(rows[:, :KV_NOPE]).reshape(n, KV_NOPE // KV_TILE, KV_TILE)
    nope = (nope * scale[:, :, None]).reshape(n, KV_NOPE)
    rope = decode_bf16(rows[:, KV_NOPE:640].copy().view("<u2"))
    return np.concatenate([nope, rope], axis=1)


MX_GROUP = 32


def mx_scale_bytes(amax: np.ndarray) -> np.ndarray:
    """Group maxima (float32, >= 0) -> E8M0 bytes: floor(log2(amax)) - 8 + 127 clamped to
    [0, 254]; 0 where amax == 0.  floor(log2(amax)) = k - 1 for amax = f * 2^k, 0.5 <= f < 1
    (frexp, exact)."""
    a = np.asarray(amax, dtype=np.float32).astype(np.float64)
    _, k = np.frexp(a)
    b = np.clip(k - 1 - 8 + 127, 0, 254)
    return np.where(a == 0.0, 0, b).astype(np.uint8)


def quantize_mxfp8(x: np.ndarray):
    """float32 [..., D] (D % 32 == 0) -> (uint8 codes [..., D], uint8 E8M0 bytes [..., D/32])."""
    x = np.asarray(x, dtype=np.float32)
    D = x.shape[-1]
    g = x.reshape(x.shape[:-1] + (D // MX_GROUP, MX_GROUP))
    sb = mx_scale_bytes(np.max(np.abs(g), axis=-1))
    scale = np.ldexp(np.float32(1.0), sb.astype(np.int32) - 127).astype(np.float32)
    quot = np.divide(g, scale[..., None], dtype=np.float32)
    return encode_fp8_e4m3(quot).reshape(x.shape), sb


def decode_mxfp8(codes: np.ndarray, scale_bytes: np.ndarray) -> np.ndarray:
    """(uint8 codes [..., D], uint8 E8M0 bytes [..., D/32]) -> float64 [..., D] (exact)."""
    v = decode_fp8_e4m3(codes)
    D = v.shape[-1]
    g = v.reshape(v.shape[:-1] + (D // MX_GROUP, MX_GROUP))
    g = g * np.ldexp(1.0, scale_bytes.astype(np.int64) - 127)[..., None]
    return g.reshape(v.shape)
