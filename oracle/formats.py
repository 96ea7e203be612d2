"""Exact number formats of the layer (oracle side; test infrastructure only).

Definitions ("Native 1017 DSpark draft on the NVLink pair (N1-NATIVE)", section 2 "Official semantics"):

* E2M1 (FP4): magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 for codes 0..7, bit 3 is the sign (0b1000 is -0).
  Packed: byte j of a row holds input 2j in the low nibble and input 2j+1 in the high nibble.
* E8M0 scale: byte b means 2^(b-127); 255 is NaN (rejected here).
* FP8 E4M3 ("float8_e4m3fn", OCP): sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0
  is subnormal m/8 * 2^-6; 0x7F/0xFF are NaN (rejected); no infinities; max 448.
* bf16: the top 16 bits of an fp32; rounding is round-to-nearest-even everywhere (the page on the
  Gemma engine, "f32 to bf16" section, shows what truncation costs).
"""
from __future__ import annotations

import numpy as np

E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E4M3_MAX = 448.0


def e2m1_decode(nibbles: np.ndarray) -> np.ndarray:
    """E2M1 code (0..15) -> value (fp64). Pinned against the printed table and the x2 integer map."""
    n = np.asarray(nibbles).astype(np.int64)
    if n.size and (n.min() < 0 or n.max() > 15):
        raise ValueError("E2M1 code out of range")
    mag = E2M1_MAGNITUDES[n & 7]
    return np.where(n & 8, -mag, mag)


def e8m0_decode(b: np.ndarray) -> np.ndarray:
    """E8M0 byte -> 2^(b-127) (fp64). 255 (NaN) is rejected."""
    b = np.asarray(b).astype(np.int64)
    if b.size and b.max() >= 255:
        raise ValueError("E8M0 NaN code 255")
    return np.ldexp(1.0, b - 127)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """E4M3fn byte -> value (fp64). NaN codes are rejected. Pinned against torch's float8_e4m3fn cast."""
    c = np.asarray(codes).astype(np.int64)
    if c.size and np.any((c & 0x7F) == 0x7F):
        raise ValueError("E4M3 NaN code")
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), -9),
                   np.ldexp((8 + m).astype(np.float64), e - 10))
    return np.where(c & 0x80, -mag, mag)


def e4m3_encode_rne(v: np.ndarray) -> np.ndarray:
    """Value with |v| <= 448 -> nearest E4M3fn code, ties to even (the sign of zero is kept)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if a.size and a.max() > E4M3_MAX:
        raise ValueError("E4M3 encode: |v| > 448 (clamp first)")
    sub = a < 2.0 ** -6
    # subnormal range: quantum 2^-9; a result of 8 quanta is the smallest normal, code 0x08
    m_sub = np.rint(np.ldexp(a, 9)).astype(np.int64)
    # normal range: a = f * 2^p with f in [0.5, 1): leading bit 2^(p-1), quantum 2^(p-4)
    _, p = np.frexp(np.where(sub, 1.0, a))
    r = np.rint(np.ldexp(np.where(sub, 1.0, a), 4 - p)).astype(np.int64)  # in [8, 16]
    up = r == 16
    e_field = (p - 1 + 7) + up
    mant = np.where(up, 0, r - 8)
    code_norm = (e_field << 3) | mant
    code = np.where(sub, m_sub, code_norm)
    sign = np.signbit(v).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def bf16_rne(v: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value (ties to even), returned as fp64.

    Works directly from fp64 (no fp32 intermediate, so no double rounding). Values beyond the bf16
    range become +-inf, values below its subnormal quantum 2^-133 round on that quantum.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, p = np.frexp(np.where(a == 0, 1.0, a))          # leading bit of a is 2^(p-1)
    q = np.maximum(p - 8, -133)                          # 8 significant bits
    r = np.ldexp(np.rint(np.ldexp(a, -q)), q)
    r = np.where(a == 0, 0.0, r)
    r = np.where(r >= 2.0 ** 128, np.inf, r)
    return np.copysign(r, v)


def bf16_bits(v: np.ndarray) -> np.ndarray:
    """bf16-representable fp64 values -> uint16 bit patterns."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def bf16_from_bits(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> fp64 values (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def f32(v) -> np.ndarray:
    """Round to fp32 (RNE), as an fp32 array."""
    return np.asarray(v, dtype=np.float64).astype(np.float32)


def _e2m1_byte_table() -> np.ndarray:
    """[256, 2] fp64: the values of the low and the high nibble of every packed byte."""
    b = np.arange(256)
    return np.stack([e2m1_decode(b & 0xF), e2m1_decode(b >> 4)], axis=1)


_E2M1_BYTE = _e2m1_byte_table()


def decode_mxfp4(w: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Packed MXFP4 matrix -> fp64 values.

    ``w`` uint8 [rows, cols/2] (low nibble = even column), ``s`` uint8 E8M0 [rows, cols/32].
    Each value is ``e2m1(code) * 2^(b-127)``, exact ("Native 1017 DSpark draft on the NVLink pair (N1-NATIVE)", section 2). Byte j of a row
    looks up its two values (low nibble first) in a table of all 256 bytes.
    """
    rows, half = w.shape
    scale = e8m0_decode(s)
    if scale.shape != (rows, 2 * half // 32):
        raise ValueError("MXFP4 scale shape mismatch")
    vals = _E2M1_BYTE[w].reshape(rows, 2 * half // 32, 32)
    return (vals * scale[:, :, None]).reshape(rows, 2 * half)


def decode_fp8_blocks(w: np.ndarray, s: np.ndarray) -> np.ndarray:
    """FP8 E4M3 matrix with one E8M0 per 32x32 block -> fp64 values.

    ``w`` uint8 [rows, cols], ``s`` uint8 [ceil(rows/32), ceil(cols/32)] ("Native 1017 DSpark draft on the NVLink pair (N1-NATIVE)", section 2).
    """
    rows, cols = w.shape
    scale = e8m0_decode(s)
    if scale.shape != ((rows + 31) // 32, (cols + 31) // 32):
        raise ValueError("FP8 block-scale shape mismatch")
    full = np.repeat(np.repeat(scale, 32, axis=0), 32, axis=1)[:rows, :cols]
    return e4m3_decode(w) * full
