"""The seeded input generator: determinism, shapes, value ranges and structure of each config."""
import numpy as np
import pytest

import synth
from oracle import formats as F
from oracle import moe


def test_deterministic_and_seeded(tiny_cfg):
    a = synth.digest(synth.make_inputs(tiny_cfg))
    b = synth.digest(synth.make_inputs(tiny_cfg))
    c = synth.digest(synth.make_inputs(synth.get_config(0, seed=5)))
    assert a == b and a != c


def test_tiny_shapes_and_ranges(tiny_cfg, tiny_inputs):
    c, i = tiny_cfg, tiny_inputs
    assert i["x"].shape == (c.M, c.H) and i["x"].dtype == np.uint16
    assert i["gate_w"].shape == (c.E, c.H) and i["gate_w"].dtype == np.float32
    assert i["w1"].shape == (c.E, c.I, c.H // 2) and i["s1"].shape == (c.E, c.I, c.H // 32)
    assert i["w2"].shape == (c.E, c.H, c.I // 2) and i["s2"].shape == (c.E, c.H, c.I // 32)
    for s in ("s1", "s3", "s2"):
        assert i[s].min() >= c.e8m0_lo and i[s].max() <= c.e8m0_hi
    assert np.all(np.abs(i["gate_b"]) <= c.bias_half)


@pytest.mark.slow
def test_decode_config_distributions():
    cfg = synth.get_config(1)
    i = synth.make_inputs(cfg)
    x = F.bf16_from_bits(i["x"])
    assert abs(x.mean()) < 0.03 and abs(x.std() - 1) < 0.03   # 40,960 samples: 6 sigma
    assert abs(i["gate_w"].std() - cfg.gate_std) < 1e-4
    # uniform bytes: every nibble value equally likely
    nib = np.bincount((i["w1"][0] & 15).reshape(-1), minlength=16) / i["w1"][0].size
    assert np.all(np.abs(nib - 1 / 16) < 2e-3)
    assert set(np.unique(i["s2"][:4])) == set(range(cfg.e8m0_lo, cfg.e8m0_hi + 1))
    r = moe.route(i["x"], i["gate_w"], i["gate_b"], cfg.k, cfg.route_scale)
    assert 30 <= len(np.unique(r["ids"])) <= 48          # about 41 distinct experts at M=8


@pytest.mark.slow
def test_prefill_hot_rows_and_skewed_routing():
    c3 = synth.get_config(3)
    i3 = synth.make_inputs(c3)
    assert i3["hot_rows"].size == 410
    x = F.bf16_from_bits(i3["x"])
    hot = np.abs(x[i3["hot_rows"]]).mean()
    cold = np.abs(np.delete(x, i3["hot_rows"], axis=0)).mean()
    assert 7.5 < hot / cold < 8.5
    del i3, x
    c4 = synth.get_config(4)
    i4 = synth.make_inputs(c4)
    assert i4["hot_experts"].size == 8
    r = moe.route(i4["x"], i4["gate_w"], i4["gate_b"], c4.k, c4.route_scale)
    share = np.isin(r["ids"], i4["hot_experts"]).mean()
    assert 0.45 <= share <= 0.55
    # shared expert: only finite E4M3 codes
    for k in ("sw1", "sw3", "sw2"):
        assert not np.any((i4[k] & 0x7F) == 0x7F)
    assert i4["ss1"].shape == (c4.I // 32, c4.H // 32) and i4["ss2"].shape == (c4.H // 32, c4.I // 32)


def test_router_inputs_are_the_first_draws_of_make_inputs():
    for cid in (0, 4):
        cfg = synth.get_config(cid, M=16, H=256, E=16, I=128) if cid else synth.get_config(0)
        full = synth.make_inputs(cfg)
        r = synth.make_router_inputs(cfg)
        for k in ("x", "gate_w", "gate_b"):
            assert np.array_equal(r[k], full[k]), k
