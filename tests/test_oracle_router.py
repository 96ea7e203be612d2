"""Pins of the router: brute-force top-k, invariants, the fp32 logits against exact sums."""
import numpy as np
import pytest

import synth
from oracle import moe
from oracle import exact


def test_router_matches_brute_force_on_tiny(tiny_cfg, tiny_inputs):
    r = moe.route(tiny_inputs["x"], tiny_inputs["gate_w"], tiny_inputs["gate_b"], tiny_cfg.k,
                  tiny_cfg.route_scale)
    b = exact.layer(tiny_inputs, tiny_cfg)
    assert np.array_equal(r["ids"], np.array(b["ids"]))
    assert np.array_equal(r["rw"], np.array(b["rw"], dtype=np.float32))
    assert np.array_equal(r["logits"], np.array(b["logits"], dtype=np.float32))
    assert np.array_equal(r["scores"], np.array(b["scores"], dtype=np.float32))


@pytest.fixture(scope="module")
def c1_small():
    cfg = synth.get_config(1)
    rng = np.random.default_rng(11)
    x32 = rng.standard_normal((64, cfg.H)).astype(np.float32)
    import torch
    x = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    gate_w = (rng.standard_normal((cfg.E, cfg.H)) * cfg.gate_std).astype(np.float32)
    gate_b = rng.uniform(-cfg.bias_half, cfg.bias_half, cfg.E).astype(np.float32)
    return cfg, x, gate_w, gate_b


def test_logits_are_the_exact_sum_rounded_once_to_fp32(c1_small):
    cfg, x, gw, gb = c1_small
    l = moe.router_logits(x[:2], gw[:16])
    for t in range(2):
        xi = [exact.bf16_int(int(b)) for b in x[t]]
        for e in range(16):
            wi = [exact.f32_int(float(w)) for w in gw[e]]
            assert exact.to_f32(exact.dot_fixed(xi, wi)) == l[t, e]


def test_topk_is_a_full_sort_with_ties_to_lower_id(c1_small):
    cfg, x, gw, gb = c1_small
    r = moe.route(x, gw, gb, cfg.k, cfg.route_scale)
    for t in range(x.shape[0]):
        sel = r["sel"][t]
        ranked = sorted(range(cfg.E), key=lambda e: (-float(sel[e]), e))
        assert list(r["ids"][t]) == ranked[: cfg.k]
    # a planted exact tie resolves to the lower id
    gb2 = gb.copy()
    ids0 = r["ids"][0]
    s = r["scores"][0]
    a, b = int(ids0[0]), int(ids0[1])
    gb2[b] = np.float32(float(r["sel"][0][a]) - float(s[b]))
    r2 = moe.route(x[:1], gw, gb2, cfg.k, cfg.route_scale)
    if r2["sel"][0][a] == r2["sel"][0][b]:
        pos = list(r2["ids"][0])
        assert pos.index(min(a, b)) < pos.index(max(a, b))
        assert r2["tie"][0]


def test_route_invariants(c1_small):
    cfg, x, gw, gb = c1_small
    r = moe.route(x, gw, gb, cfg.k, cfg.route_scale)
    ids, rw = r["ids"], r["rw"]
    assert ids.dtype == np.int32 and ids.shape == (64, cfg.k)
    assert np.all((ids >= 0) & (ids < cfg.E))
    assert all(len(set(row)) == cfg.k for row in ids)
    # selection scores are non-increasing along the slots
    sel = np.take_along_axis(r["sel"], ids, axis=1)
    assert np.all(np.diff(sel, axis=1) <= 0)
    # route weights are positive and sum to the route scale (fp32: within (k + 2) ulp)
    assert np.all(rw > 0)
    tot = rw.astype(np.float64).sum(axis=1)
    ulp = np.spacing(np.float32(cfg.route_scale))
    assert np.all(np.abs(tot - cfg.route_scale) <= (cfg.k + 2) * ulp)
    # the gathered weights are the scores (bias only selects)
    w = np.take_along_axis(r["scores"], ids, axis=1).astype(np.float64)
    assert np.allclose(rw, cfg.route_scale * w / w.sum(axis=1, keepdims=True), rtol=1e-6, atol=0)


def test_scores_are_sqrt_softplus(c1_small):
    cfg, x, gw, gb = c1_small
    l = moe.router_logits(x[:4], gw)
    s = moe.router_scores(l)
    # closed form at a few points: softplus(0) = ln 2
    assert moe.router_scores(np.array([0.0], dtype=np.float32))[0] == np.float32(np.sqrt(np.log(2.0)))
    ref = np.sqrt(np.log(1.0 + np.exp(l.astype(np.float64))))
    assert np.allclose(s, ref, rtol=2 ** -23)
