"""Pins of the oracle's number formats against printed tables and library routines."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import exact

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "printed_values.json")))


def test_e2m1_table_matches_printed_table():
    mags = GOLD["e2m1_magnitudes"]["value"]
    codes = np.arange(16)
    v = F.e2m1_decode(codes)
    assert list(v[:8]) == mags
    assert list(-v[8:]) == mags
    # 0b1000 is negative zero
    assert v[8] == 0 and np.signbit(v[8])


def test_e2m1_times_two_is_the_printed_integer_map():
    ints = GOLD["e2m1_times_two_integers"]["value"]
    v = F.e2m1_decode(np.arange(8)) * 2
    assert list(v.astype(int)) == ints
    # the brute force decodes from the integer map itself; both must agree on all 16 codes
    for n in range(16):
        iv, ex = exact.fp4_int(n)
        assert np.ldexp(iv, ex) == F.e2m1_decode(np.array([n]))[0]


def test_e8m0_formula_and_nan():
    b = np.arange(255)
    assert np.array_equal(F.e8m0_decode(b), 2.0 ** (b - GOLD["e8m0_bias"]["value"]))
    with pytest.raises(ValueError):
        F.e8m0_decode(np.array([GOLD["e8m0_nan"]["value"]]))


def test_e4m3_decode_matches_torch_float8_cast():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.e4m3_decode(codes)
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))
    assert got.max() == GOLD["e4m3_max"]["value"]
    with pytest.raises(ValueError):
        F.e4m3_decode(np.array([0x7F]))
    with pytest.raises(ValueError):
        F.e4m3_decode(np.array([0xFF]))


def _all_bf16_in(lo, hi):
    bits = np.arange(0, 0x8000, dtype=np.uint32)
    v = (bits << 16).view(np.float32).astype(np.float64)
    v = v[np.isfinite(v) & (v <= hi) & (v >= lo)]
    return np.concatenate([v, -v])


def test_e4m3_encode_rne_matches_torch_cast_on_every_bf16_value_in_range():
    v = _all_bf16_in(0.0, 448.0)
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.e4m3_encode_rne(v)
    assert np.array_equal(got, ref)


def test_e4m3_encode_rne_ties_and_midpoints():
    # exact midpoints between neighbouring codes go to the even code (fp64 midpoints)
    codes = np.array([c for c in range(0x7E)], dtype=np.uint8)
    lo = F.e4m3_decode(codes)
    hi = F.e4m3_decode(codes + 1)
    mid = (lo + hi) / 2
    got = F.e4m3_encode_rne(mid)
    want = np.where(codes % 2 == 0, codes, codes + 1).astype(np.uint8)
    assert np.array_equal(got, want)
    # brute-force nearest search agrees on a sweep of values
    xs = np.linspace(-448, 448, 2001)
    assert [exact.e4m3_nearest(float(x)) for x in xs] == list(F.e4m3_encode_rne(xs))


def test_bf16_rne_matches_torch_cast_on_fp32_values():
    rng = np.random.default_rng(0)
    a = rng.standard_normal(200000).astype(np.float32) * np.float32(1e3)
    # plant exact ties: low 16 bits = 0x8000 with both parities of bit 16
    bits = a.view(np.uint32)
    bits[:1000] = (bits[:1000] & 0xFFFF0000) | 0x8000
    a = bits.view(np.float32)
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(F.bf16_rne(a.astype(np.float64)), ref)


def test_bf16_rne_from_fp64_against_integer_rounding():
    rng = np.random.default_rng(1)
    v = rng.standard_normal(5000) * np.exp(rng.uniform(-30, 30, 5000))
    got = F.bf16_rne(v)
    for x, g in zip(v[:2000], got[:2000]):
        num, den = float(x).as_integer_ratio()
        # value = num / den with den a power of two; fixed point at 2^-EXP0
        S = num << (exact.EXP0 - (den.bit_length() - 1))
        assert exact.to_bf16(S) == g


def test_bf16_bits_roundtrip():
    bits = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    vals = F.bf16_from_bits(bits)
    fin = np.isfinite(vals)
    assert np.array_equal(F.bf16_bits(vals[fin]), bits[fin])


def test_mxfp4_decode_nibble_order_and_scale_blocks():
    # row of 64 inputs: byte j holds input 2j (low nibble) and 2j+1 (high nibble)
    w = np.zeros((2, 32), dtype=np.uint8)
    w[0, 0] = 0x52        # input 0 = code 2 (1.0), input 1 = code 5 (3.0)
    w[1, 31] = 0xA0       # input 62 = 0, input 63 = code 10 (-1.0)
    s = np.array([[127, 130], [120, 125]], dtype=np.uint8)
    d = F.decode_mxfp4(w, s)
    assert d.shape == (2, 64)
    assert d[0, 0] == 1.0 and d[0, 1] == 3.0 and np.count_nonzero(d[0]) == 2
    assert d[1, 63] == -1.0 * 2.0 ** (125 - 127) and np.count_nonzero(d[1]) == 1


def test_fp8_block_decode_uses_32x32_blocks():
    w = np.full((64, 64), 0x38, dtype=np.uint8)   # every value 1.0
    s = np.array([[127, 128], [129, 130]], dtype=np.uint8)
    d = F.decode_fp8_blocks(w, s)
    assert d[0, 0] == 1 and d[31, 31] == 1 and d[0, 32] == 2 and d[32, 0] == 4 and d[63, 63] == 8


def test_expert_storage_bytes_match_the_printed_memory_table():
    # one TP2 rank holds half of every routed matrix; a full layer is twice the printed figure
    shp = GOLD["mxfp4_expert_shapes"]["value"]
    per_expert = 2 * (shp["w1_i8"][0] * shp["w1_i8"][1] + shp["w1_e8m0"][0] * shp["w1_e8m0"][1]) \
        + shp["w2_i8"][0] * shp["w2_i8"][1] + shp["w2_e8m0"][0] * shp["w2_e8m0"][1]
    assert per_expert == 18_800_640
    mib = GOLD["expanded_bytes_mib"]["value"]["packed_per_stage_per_rank"]
    assert 128 * per_expert == 2 * mib * 2 ** 20
