"""Pins of the oracle's linear layers, SwiGLU, combine and the whole tiny layer."""
import json
import os

import numpy as np
import pytest

import synth
from oracle import formats as F
from oracle import moe
from oracle import exact

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "printed_values.json")))


def test_whole_tiny_layer_equals_brute_force(tiny_cfg, tiny_inputs):
    o = moe.moe_forward(tiny_inputs, tiny_cfg)
    b = exact.layer(tiny_inputs, tiny_cfg)
    assert np.array_equal(o["ids"], np.array(b["ids"]))
    assert np.array_equal(o["xq"], np.array(b["xq"], dtype=np.uint8))
    assert np.array_equal(o["xs"], np.array(b["xs"], dtype=np.uint8))
    assert np.array_equal(o["g"], np.array(b["g"]))
    assert np.array_equal(o["u"], np.array(b["u"]))
    assert np.array_equal(o["h16"], np.array(b["h16"]))
    assert np.array_equal(o["slot_y"], np.array(b["slot_y"]))
    assert np.array_equal(o["out"], np.array(b["out"]))


def _tiny_with_shared(seed=7):
    cfg = synth.get_config(0, shared=True, seed=seed)
    return cfg, synth.make_inputs(cfg)


def test_tiny_layer_with_fp8_shared_expert_equals_brute_force():
    cfg, inp = _tiny_with_shared()
    o = moe.moe_forward(inp, cfg)
    b = exact.layer(inp, cfg)
    assert np.array_equal(o["shared_y"], np.array(b["shared_y"]))
    assert np.array_equal(o["out"], np.array(b["out"]))


def test_decoded_bf16_arm_equals_packed_arm(tiny_cfg, tiny_inputs):
    p = moe.moe_forward(tiny_inputs, tiny_cfg, arm="packed")
    d = moe.moe_forward(tiny_inputs, tiny_cfg, arm="decoded")
    for key in ("g", "u", "h16", "slot_y", "out"):
        assert np.array_equal(p[key], d[key]), key


def test_decoded_arm_weights_are_exact_in_bf16(tiny_inputs):
    W = moe.ExpertWeights(tiny_inputs, "decoded")
    for e in range(3):
        w1b, _, w2b = W.expand_bf16(e)
        assert np.array_equal(F.bf16_from_bits(w1b), F.decode_mxfp4(tiny_inputs["w1"][e], tiny_inputs["s1"][e]))
        assert np.array_equal(F.bf16_from_bits(w2b), F.decode_mxfp4(tiny_inputs["w2"][e], tiny_inputs["s2"][e]))


@pytest.mark.parametrize("n,kk,code,b", [(0, 0, 2, 127), (5, 1, 5, 120), (17, 63, 13, 124),
                                         (127, 254, 7, 118), (64, 255, 9, 130)])
def test_single_nibble_probe_fingerprints_layout(n, kk, code, b):
    """One nonzero nibble at (row n, input kk) with scale b gives y[n] = bf16(x[kk] e2m1(code) 2^(b-127))
    and zero elsewhere: fixes nibble order (even input = low nibble) and the scale's row/block index."""
    I, H = 128, 256
    w = np.zeros((I, H // 2), dtype=np.uint8)
    w[n, kk // 2] = code if kk % 2 == 0 else code << 4
    s = np.full((I, H // 32), 127, dtype=np.uint8)
    s[n, kk // 32] = b
    rng = np.random.default_rng(n + kk)
    x = F.bf16_rne(rng.standard_normal((1, H)))
    _, _, xhat = moe.act_qdq(x)
    y = F.bf16_rne(xhat @ F.decode_mxfp4(w, s).T)
    want = F.bf16_rne(xhat[0, kk] * F.e2m1_decode(np.array([code]))[0] * 2.0 ** (b - 127))
    assert y[0, n] == want
    assert np.count_nonzero(y[0]) == (1 if want != 0 else 0)


def test_fp8_block_probe():
    I, H = 64, 128
    w = np.zeros((I, H), dtype=np.uint8)
    w[40, 70] = 0x44            # 2^1 * 1.5 = 3.0
    s = np.full((I // 32, H // 32), 127, dtype=np.uint8)
    s[1, 2] = 125
    x = F.bf16_rne(np.linspace(-3, 3, H)[None, :])
    _, _, xhat = moe.act_qdq(x)
    y = F.bf16_rne(xhat @ F.decode_fp8_blocks(w, s).T)
    assert y[0, 40] == F.bf16_rne(xhat[0, 70] * 3.0 * 0.25)
    assert np.count_nonzero(y) == 1


def test_all_zero_weights_give_zero(tiny_cfg, tiny_inputs):
    inp = dict(tiny_inputs)
    for key in ("w1", "w3", "w2"):
        inp[key] = np.zeros_like(inp[key])
    o = moe.moe_forward(inp, tiny_cfg)
    assert np.all(o["out"] == 0)


def test_exact_integer_dot_equals_fp64_on_full_size_rows():
    """At the real shapes (H=5120, I=2304) the fp64 BLAS sums of the oracle are exact: sampled rows
    of g and y against exact integer sums."""
    cfg = synth.get_config(1, E=2)
    inp = synth.make_inputs(cfg)
    W = moe.ExpertWeights(inp)
    x = F.bf16_from_bits(inp["x"][:1])
    _, _, xhat = moe.act_qdq(x)
    w1, w3, w2 = W.get(0)
    o = moe.expert_ffn(xhat, np.array([0.25], dtype=np.float32), w1, w3, w2)
    _, _, xdeq = exact.qdq_row([float(v) for v in x[0]])
    for n in (0, 1, 777, 2303):
        row = exact.mxfp4_row(inp["w1"][0][n], inp["s1"][0][n])
        assert exact.to_bf16(exact.dot_fixed(xdeq, row)) == o["g"][0, n]
    _, _, hdeq = exact.qdq_row([float(v) for v in o["h16"][0]])
    for n in (0, 4095, 5119):
        row = exact.mxfp4_row(inp["w2"][0][n], inp["s2"][0][n])
        assert exact.to_bf16(exact.dot_fixed(hdeq, row)) == o["y"][0, n]


def test_swiglu_special_cases_and_bound():
    clamp = GOLD["up_clamp"]["value"]
    g = np.array([[0.0, 20.0, -200.0, 10.0, 3.0, -0.0]])
    u = np.array([[5.0, 50.0, 4.0, -50.0, 0.0, 7.0]])
    h = moe.swiglu(g, u, np.array([1.0], dtype=np.float32))[0]
    assert h[0] == 0                     # g = 0 -> silu = 0
    silu10 = 10.0 / (1.0 + np.exp(-10.0))
    assert h[1] == F.bf16_rne(np.float32(np.float32(silu10) * clamp))  # both clamps saturate
    assert h[2] == 0                     # exp overflows: silu -> -0
    assert h[3] == F.bf16_rne(np.float32(np.float32(silu10) * -clamp))
    assert h[4] == 0
    # the page's bound |h| <= silu(10) * 10 * rw
    rng = np.random.default_rng(0)
    G = F.bf16_rne(rng.standard_normal((4, 4096)) * 20)
    U = F.bf16_rne(rng.standard_normal((4, 4096)) * 20)
    rw = np.array([0.1, 0.5, 1.0, 1.5], dtype=np.float32)
    H = moe.swiglu(G, U, rw)
    bound = silu10 * clamp * rw.astype(np.float64)
    assert np.all(np.abs(H) <= F.bf16_rne(bound * (1 + 2 ** -20))[:, None])


def test_combine_adds_in_ascending_expert_id():
    """Order matters in fp32: with slots listed in descending id the oracle still adds ascending."""
    big, small = 2.0 ** 24, 1.0
    ids = np.array([[7, 3, 1]])
    # ascending id order: slot(1)= -big, slot(3)= small, slot(7)= big
    slot_y = np.array([[[big], [small], [-big]]])
    out = moe.combine(ids, slot_y, None)
    # ascending: (-big + 1) + big: -big + 1 = -16777215 exact in fp32, + big = 1
    assert out[0, 0] == 1.0
    # descending would give (big + 1) -> big (rounded), + (-big) = 0
    shared = np.array([[0.5]])
    assert moe.combine(ids, slot_y, shared)[0, 0] == 1.5


def test_permute_is_a_stable_counting_sort():
    rng = np.random.default_rng(2)
    ids = np.stack([rng.choice(16, size=4, replace=False) for _ in range(50)]).astype(np.int32)
    p = moe.permute(ids, 16)
    flat = ids.reshape(-1)
    assert p["offsets"][-1] == flat.size
    for e in range(16):
        seg = p["pairs"][p["offsets"][e]:p["offsets"][e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)
    assert np.array_equal(p["pairs"][p["inv"].reshape(-1)], np.arange(flat.size))
    act = p["active"][: p["n_active"]]
    assert np.array_equal(act, np.unique(flat)) and np.all(p["active"][p["n_active"]:] == -1)


def test_fp8_linear_one_hot_closed_form():
    """One nonzero E4M3 code c at (n, k) with block scale b: y[:, n] = bf16(xhat[:, k] * e4m3(c) * 2^(b-127)),
    every other output 0 (fingerprints the row/column roles and the 32x32 scale indexing)."""
    N, K = 96, 160
    for n, k, c, b in ((0, 0, 0x38, 127), (70, 131, 0xC9, 121), (95, 159, 0x7E, 124)):
        w = np.zeros((N, K), dtype=np.uint8)
        w[n, k] = c
        s = np.full((N // 32, K // 32), 127, dtype=np.uint8)
        s[n // 32, k // 32] = b
        x = synth.make_dense_inputs(N, K, 3, seed=n + k)["x"]
        o = moe.fp8_linear(x, w, s)
        _, _, xhat = moe.act_qdq(F.bf16_from_bits(x))
        want = F.bf16_rne(xhat[:, k] * F.e4m3_decode(np.array([c]))[0] * 2.0 ** (b - 127))
        assert np.array_equal(o["y"][:, n], want)
        assert np.count_nonzero(np.delete(o["y"], n, axis=1)) == 0


def test_fp8_linear_equals_exact_integer_sums():
    """Sampled outputs of a full-size projection (wo_b, K = 4096) against exact integer dot products."""
    N, K = 256, 4096
    inp = synth.make_dense_inputs(N, K, 2, seed=11)
    o = moe.fp8_linear(inp["x"], inp["w"], inp["s"])
    for t in range(2):
        _, _, xdeq = exact.qdq_row([float(v) for v in F.bf16_from_bits(inp["x"][t])])
        for n in (0, 31, 32, 255):
            row = exact.fp8_row(inp["w"][n], inp["s"][n // 32])
            assert exact.to_bf16(exact.dot_fixed(xdeq, row)) == o["y"][t, n]


@pytest.mark.parametrize("I, I_pad", [(96, 128), (160, 256), (64, 128)])
def test_zero_padding_of_the_intermediate_width_changes_no_output(I, I_pad):
    """Widening I with zero weight codes leaves every output value unchanged (the library takes I in
    multiples of 128; an I that is only a multiple of 32, e.g. a quarter of 2304, is padded this way)."""
    cfg = synth.get_config(0, I=I, shared=True, M=6, seed=11)
    inp = synth.make_inputs(cfg)
    pad = synth.pad_inter(inp, I, I_pad)
    pcfg = synth.get_config(0, I=I_pad, shared=True, M=6, seed=11)
    a, b = moe.moe_forward(inp, cfg), moe.moe_forward(pad, pcfg)
    assert np.array_equal(a["ids"], b["ids"])
    assert np.array_equal(b["g"][..., :I], a["g"]) and not np.any(b["g"][..., I:])
    assert np.array_equal(b["u"][..., :I], a["u"]) and not np.any(b["u"][..., I:])
    assert np.array_equal(b["h16"][..., :I], a["h16"]) and not np.any(b["h16"][..., I:])
    # values, not bits: an all-zero sum may come out as -0 on one side and +0 on the other
    assert np.array_equal(a["slot_y"], b["slot_y"])
    assert np.array_equal(a["shared_y"], b["shared_y"])
    assert np.array_equal(a["out"], b["out"])
