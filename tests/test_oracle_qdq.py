"""Pins of the activation QDQ (act_quant per 32 with a power-of-two E8M0 scale)."""
from fractions import Fraction

import numpy as np

from oracle import formats as F
from oracle import moe
from oracle import exact


def _all_positive_finite_bf16():
    bits = np.arange(1, 0x7F80, dtype=np.uint32)
    return (bits << 16).view(np.float32)


def _ceil_log2_fraction(q: Fraction) -> int:
    # smallest E with 2^E >= q
    E = q.numerator.bit_length() - q.denominator.bit_length()
    while Fraction(2) ** E < q:
        E += 1
    while Fraction(2) ** (E - 1) >= q:
        E -= 1
    return E


def test_scale_rule_equals_exact_ceil_log2_for_every_bf16_amax():
    """fp32(amax * fp32(1/448)) with the ceil taken from the bits equals ceil(log2(amax/448)) exactly,
    for every finite bf16 amax (with the 1e-4 floor applied in fp32)."""
    a = _all_positive_finite_bf16()
    got = moe.qdq_scale_exponent(a)
    floor = Fraction(float(np.float32(1e-4)))
    bad = []
    for x, e in zip(a.astype(np.float64), got):
        q = max(Fraction(float(x)), floor) / 448
        if _ceil_log2_fraction(q) != e:
            bad.append(float(x))
    assert not bad, bad[:10]


def test_scale_rule_agrees_with_frexp_route_of_the_brute_force():
    a = _all_positive_finite_bf16()[::7]
    got = moe.qdq_scale_exponent(a)
    inv = exact.f32(1.0 / 448.0)
    for x, e in zip(a.astype(np.float64), got):
        v = exact.f32(max(float(x), exact.f32(1e-4)) * inv)
        fr, p = np.frexp(v)
        assert (p - 1 if fr == 0.5 else p) == e


def test_qdq_properties_on_random_rows():
    rng = np.random.default_rng(3)
    x = F.bf16_rne(rng.standard_normal((64, 512)) * np.exp(rng.uniform(-12, 12, (64, 1))))
    codes, sbytes, deq = moe.act_qdq(x)
    q = F.e4m3_decode(codes)
    assert np.abs(q).max() <= 448
    s = np.ldexp(1.0, sbytes.astype(np.int64) - 127)
    # dequantized values are exact in bf16 and equal q * s
    assert np.array_equal(F.bf16_rne(deq), deq)
    assert np.array_equal(deq, q * np.repeat(s, 32, axis=1))
    # each block's amax maps into (224, 448] before rounding (when above the 1e-4 floor)
    amax = np.abs(x.reshape(64, 16, 32)).max(axis=2)
    ratio = amax / s
    big = amax >= 1e-4
    assert np.all(ratio[big] > 224) and np.all(ratio[big] <= 448)
    # QDQ is idempotent in value
    _, _, deq2 = moe.act_qdq(deq)
    assert np.array_equal(deq2, deq)


def test_qdq_matches_brute_force_row():
    rng = np.random.default_rng(4)
    x = F.bf16_rne(rng.standard_normal((3, 128)) * 3)
    x[1, :32] = 0.0           # all-zero block: amax floor
    x[2, 40] = 300.0          # one large value in a block
    codes, sbytes, _ = moe.act_qdq(x)
    for r in range(3):
        c, s, _ = exact.qdq_row([float(v) for v in x[r]])
        assert list(codes[r]) == c
        assert list(sbytes[r]) == s


def test_qdq_of_zero_block_uses_the_floor():
    codes, sbytes, deq = moe.act_qdq(np.zeros((1, 32)))
    assert np.all(deq == 0) and np.all(codes == 0)
    # fp32(1e-4) * fp32(1/448) = 2.23e-7 -> ceil(log2) = -22
    assert sbytes[0, 0] == 127 - 22
