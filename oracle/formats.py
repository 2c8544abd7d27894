"""Number formats of the decode layer, written from their bit definitions.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product path.

Formats named by the pages ("Mono decode layer for DeepSeek-V4.1-Flash on
MI355X", vLLM PR 60397, Design and Layout): fp8 e4m3 (weights, activations,
KV codes), MXFP4 = e2m1 elements with one E8M0 exponent per 32, MXFP8 with
32x32 E8M0 tiles, bf16 activations.  The bit layouts follow the OCP 8-bit
float and Microscaling (MX v1.0) specifications.  All arithmetic is float64
unless a rounding point says otherwise.
"""
from __future__ import annotations

import numpy as np


def e8m0_value(b: np.ndarray) -> np.ndarray:
    """E8M0 byte -> 2**(b-127); byte 255 is NaN."""
    b = np.asarray(b).astype(np.int64)
    v = np.ldexp(1.0, b - 127)
    return np.where(b == 255, np.nan, v)


def _e4m3_table() -> np.ndarray:
    """Value of each of the 256 E4M3FN codes: sign bit 7, exponent bits 6..3 (bias 7),
    mantissa bits 2..0; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN;
    there is no infinity."""
    t = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 7
        if e == 0xF and m == 7:
            t[c] = np.nan
        elif e == 0:
            t[c] = s * (m / 8.0) * 2.0 ** -6
        else:
            t[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


def _e2m1_table() -> np.ndarray:
    """Value of each of the 16 E2M1 codes: sign bit 3, exponent bits 2..1 (bias 1),
    mantissa bit 0; exponent 0 is subnormal (m * 0.5)."""
    t = np.empty(16, dtype=np.float64)
    for c in range(16):
        s = -1.0 if c & 8 else 1.0
        e = (c >> 1) & 3
        m = c & 1
        t[c] = s * (m * 0.5 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1))
    return t


E4M3 = _e4m3_table()
E2M1 = _e2m1_table()
E4M3_MAX = 448.0


def e4m3_value(codes: np.ndarray) -> np.ndarray:
    return E4M3[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even to E4M3FN with saturation to +-448 (finite inputs).
    Rounding is exact because x, given as float64 holding float32 values, is split
    into exponent and mantissa without loss."""
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x).astype(np.uint8) << 7
    a = np.abs(x)
    out = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # subnormal range: steps of 2^-9; a result of 8 is the smallest normal (code 8)
    out[sub] = np.rint(a[sub] / 2.0 ** -9).astype(np.int64)
    nrm = ~sub
    an = a[nrm]
    e = np.floor(np.log2(an)).astype(np.int64)
    # floor(log2) may be off by one at exact powers of two in floating point; fix it
    e = np.where(np.ldexp(1.0, e) > an, e - 1, e)
    e = np.where(np.ldexp(1.0, e + 1) <= an, e + 1, e)
    frac = an / np.ldexp(1.0, e) - 1.0  # in [0, 1), exact
    q = np.rint(frac * 8.0).astype(np.int64)  # 0..8, ties to even
    carry = q == 8
    e = np.where(carry, e + 1, e)
    q = np.where(carry, 0, q)
    code = ((e + 7) << 3) | q
    code = np.where((e + 7) > 15, 0x7E, code)
    code = np.minimum(code, 0x7E)  # saturate: 0x7F would be NaN
    out[nrm] = code
    return (out.astype(np.uint8) | sign).astype(np.uint8)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """bf16 code (uint16) -> float64: the top 16 bits of an IEEE float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f32(x: np.ndarray) -> np.ndarray:
    """Round to IEEE float32 (nearest even) and carry the result as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16_encode(x: np.ndarray) -> np.ndarray:
    """Round to float32, then to bf16 by round-to-nearest-even on the low 16 bits."""
    b = np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = (b + 0x7FFF + lsb) >> 16
    return (r & 0xFFFF).astype(np.uint16)


def bf16_round(x: np.ndarray) -> np.ndarray:
    return bf16_value(bf16_encode(x))


def mx_e4m3_quantize(v: np.ndarray):
    """OCP MX block quantization to MXFP8 (e4m3 elements), blocks of 32 along the last
    axis.  The shared exponent is floor(log2(amax)) read from the float32 exponent field,
    less e4m3's largest exponent (8), biased by 127 and clamped to [0, 254]; elements
    are v / 2^(X-127) rounded to nearest even with saturation.  An all-zero block gets
    X = 0 and zero codes.  v holds float32 values; returns (codes uint8, X uint8)."""
    v = np.asarray(v, dtype=np.float64)
    shp = v.shape
    blk = v.reshape(shp[:-1] + (shp[-1] // 32, 32))
    amax = np.abs(blk).max(axis=-1)
    efield = (amax.astype(np.float32).view(np.uint32) >> 23) & 0xFF
    X = np.clip(efield.astype(np.int64) - 8, 0, 254)
    scaled = blk / np.ldexp(1.0, X - 127)[..., None]
    codes = e4m3_encode(scaled).reshape(shp)
    return codes, X.astype(np.uint8)


def mx_e4m3_dequant_act(codes: np.ndarray, X: np.ndarray) -> np.ndarray:
    """Inverse of mx_e4m3_quantize: e4m3 value times 2^(X-127) per 32-block."""
    v = e4m3_value(codes)
    return v * np.repeat(e8m0_value(X), 32, axis=-1)


def dequant_mxfp8_weight(codes: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Row-major e4m3 [N, K] with one E8M0 per 32x32 tile [N/32, K/32]."""
    sc = np.repeat(np.repeat(e8m0_value(s), 32, axis=0), 32, axis=1)
    return e4m3_value(codes) * sc


def dequant_fp8_block128(codes: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Row-major e4m3 [N, K] with one float32 scale per 128x128 block [N/128, K/128]."""
    sc = np.repeat(np.repeat(np.asarray(s, dtype=np.float64), 128, axis=0), 128, axis=1)
    return e4m3_value(codes) * sc


def dequant_mxfp4(packed: np.ndarray, s: np.ndarray) -> np.ndarray:
    """e2m1 nibbles [N, K/2] (low nibble = even k, high nibble = odd k) with one E8M0
    per 32 along K [N, K/32] -> float64 [N, K]."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = E2M1[p & 0xF]
    hi = E2M1[p >> 4]
    v = np.stack([lo, hi], axis=-1).reshape(p.shape[:-1] + (p.shape[-1] * 2,))
    return v * np.repeat(e8m0_value(s), 32, axis=-1)
