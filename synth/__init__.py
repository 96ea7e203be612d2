"""Seeded synthetic inputs for the routed-MoE FFN layer (shared by the oracle and the GPU path).

This module only draws random numbers and arranges them in the storage formats the layer consumes.
It holds none of the layer's arithmetic: no decoding of the formats, no quantisation, no routing.

Storage formats (page "Native 1017 DSpark draft on the NVLink pair (N1-NATIVE)", section 2 "Official semantics" and
section 4 "Kernel contract"):

* activations ``x``: bf16 stored as ``uint16`` bit patterns, shape [M, H];
* gate weight: fp32 [E, H]; gate bias: fp32 [E];
* routed experts, MXFP4: ``w1``/``w3`` uint8 [E, I, H/2] (byte j of a row holds input 2j in the low
  nibble and 2j+1 in the high nibble) with E8M0 scales uint8 [E, I, H/32]; ``w2`` uint8 [E, H, I/2]
  with scales uint8 [E, H, I/32];
* shared expert, FP8 E4M3: ``sw1``/``sw3`` uint8 [I, H] with E8M0 32x32 block scales uint8
  [I/32, H/32]; ``sw2`` uint8 [H, I] with scales [H/32, I/32].

Draw order (one ``numpy.random.Generator(PCG64(seed))`` per config): x, (prefill: the scaled rows),
gate, bias, (skewed: the hot experts), w1, s1, w3, s3, w2, s2, then the shared tensors sw1, ss1,
sw3, ss3, sw2, ss2.
"""
from __future__ import annotations

import hashlib
import json
import os
from dataclasses import dataclass, field, asdict

import numpy as np

__all__ = ["LayerConfig", "CONFIGS", "get_config", "make_inputs", "make_router_inputs", "make_tokens", "digest",
           "c4_hot_bias", "pad_inter"]


@dataclass(frozen=True)
class LayerConfig:
    name: str
    M: int            # tokens
    H: int            # hidden size
    E: int            # routed experts
    I: int            # expert intermediate size
    k: int            # experts per token
    gate_std: float   # gate weight ~ N(0, gate_std)
    bias_half: float  # selection bias ~ U(-bias_half, bias_half)
    e8m0_lo: int      # E8M0 exponent bytes ~ U{e8m0_lo .. e8m0_hi}
    e8m0_hi: int
    route_scale: float = 1.5
    seed: int = 0
    hot_row_frac: float = 0.0    # fraction of token rows scaled by hot_row_mult
    hot_row_mult: float = 1.0
    shared: bool = False         # FP8 E4M3 shared expert present
    hot_experts: int = 0         # experts whose bias is raised by the calibrated delta

    @property
    def pairs(self) -> int:
        return self.M * self.k


_BIG = dict(H=5120, E=128, I=2304, k=6, gate_std=0.01, bias_half=0.05, e8m0_lo=118, e8m0_hi=124,
            route_scale=1.5)

CONFIGS = {
    0: LayerConfig(name="tiny_m4", M=4, H=256, E=8, I=128, k=2, gate_std=0.02, bias_half=0.1,
                   e8m0_lo=120, e8m0_hi=124, route_scale=1.5, seed=0),
    1: LayerConfig(name="decode_m8", M=8, seed=1, **_BIG),
    2: LayerConfig(name="batched_decode_m64", M=64, seed=2, **_BIG),
    3: LayerConfig(name="prefill_m8192", M=8192, seed=3, hot_row_frac=0.05, hot_row_mult=8.0, **_BIG),
    4: LayerConfig(name="prefill_shared_skew_m2048", M=2048, seed=4, shared=True, hot_experts=8, **_BIG),
}


def get_config(cid: int, **overrides) -> LayerConfig:
    """A config by index; keyword overrides (e.g. ``M=64``) give derived test shapes."""
    cfg = CONFIGS[cid]
    if overrides:
        d = asdict(cfg)
        d.update(overrides)
        cfg = LayerConfig(**d)
    return cfg


_HOT_BIAS_FILE = os.path.join(os.path.dirname(__file__), "c4_hot_bias.json")


def c4_hot_bias() -> float:
    """Bias increment of the hot experts in the skewed config.

    The value is stored in ``c4_hot_bias.json`` next to this file; it is written by
    ``oracle/calibrate_skew.py``, which bisects it with the oracle's router so that the hot experts
    take about half of all assignments on the generated activations.
    """
    with open(_HOT_BIAS_FILE) as f:
        return float(json.load(f)["delta"])


def _to_bf16_bits(a32: np.ndarray) -> np.ndarray:
    # Input preparation only: round the drawn fp32 samples to bf16 storage with torch's cast.
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _finite_e4m3_bytes(rng: np.random.Generator, shape) -> np.ndarray:
    # uniform over the 254 finite E4M3 codes: 0x00..0x7E and 0x80..0xFE
    v = rng.integers(0, 254, size=shape, dtype=np.uint16)
    v = v + (v >= 127)
    return v.astype(np.uint8)


def _draw_tokens(rng: np.random.Generator, cfg: LayerConfig):
    M, H = cfg.M, cfg.H
    x32 = rng.standard_normal((M, H), dtype=np.float32)
    hot_rows = np.zeros(0, dtype=np.int64)
    if cfg.hot_row_frac > 0:
        n_hot = int(round(cfg.hot_row_frac * M))
        hot_rows = np.sort(rng.choice(M, size=n_hot, replace=False))
        x32[hot_rows] *= np.float32(cfg.hot_row_mult)   # power of two: exact after bf16 rounding too
    return _to_bf16_bits(x32), hot_rows


def make_tokens(cfg: LayerConfig) -> np.ndarray:
    """Only the token rows x (bf16 bits [M, H]) of make_inputs(cfg), drawn the same way. Without hot rows,
    the first m rows for M = m' > m equal the rows for M = m (the normal draws fill x row by row)."""
    return _draw_tokens(np.random.Generator(np.random.PCG64(cfg.seed)), cfg)[0]


def _draw_router(rng: np.random.Generator, cfg: LayerConfig, hot_delta: float | None):
    """The first draws of a layer: tokens, gate weight and bias (with the hot experts' increment)."""
    E, H = cfg.E, cfg.H
    x, hot_rows = _draw_tokens(rng, cfg)
    gate_w = (rng.standard_normal((E, H)) * cfg.gate_std).astype(np.float32)
    gate_b = rng.uniform(-cfg.bias_half, cfg.bias_half, size=E).astype(np.float32)
    hot_experts = np.zeros(0, dtype=np.int64)
    if cfg.hot_experts > 0:
        hot_experts = np.sort(rng.choice(E, size=cfg.hot_experts, replace=False))
        delta = c4_hot_bias() if hot_delta is None else hot_delta
        gate_b[hot_experts] = (gate_b[hot_experts] + np.float32(delta)).astype(np.float32)
    return x, hot_rows, gate_w, gate_b, hot_experts


def make_router_inputs(cfg: LayerConfig) -> dict:
    """Only x, gate_w and gate_b of make_inputs(cfg), drawn the same way (no expert weights)."""
    x, _, gate_w, gate_b, _ = _draw_router(np.random.Generator(np.random.PCG64(cfg.seed)), cfg, None)
    return dict(x=x, gate_w=gate_w, gate_b=gate_b)


def make_inputs(cfg: LayerConfig, hot_delta: float | None = None) -> dict:
    """Draw every input tensor of one layer invocation (numpy arrays, host memory)."""
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    M, H, E, I = cfg.M, cfg.H, cfg.E, cfg.I
    x, hot_rows, gate_w, gate_b, hot_experts = _draw_router(rng, cfg, hot_delta)
    lo, hi = cfg.e8m0_lo, cfg.e8m0_hi + 1
    w1 = rng.integers(0, 256, size=(E, I, H // 2), dtype=np.uint8)
    s1 = rng.integers(lo, hi, size=(E, I, H // 32), dtype=np.uint8)
    w3 = rng.integers(0, 256, size=(E, I, H // 2), dtype=np.uint8)
    s3 = rng.integers(lo, hi, size=(E, I, H // 32), dtype=np.uint8)
    w2 = rng.integers(0, 256, size=(E, H, I // 2), dtype=np.uint8)
    s2 = rng.integers(lo, hi, size=(E, H, I // 32), dtype=np.uint8)
    out = dict(x=x, gate_w=gate_w, gate_b=gate_b, w1=w1, s1=s1, w3=w3, s3=s3, w2=w2, s2=s2,
               hot_rows=hot_rows, hot_experts=hot_experts)
    if cfg.shared:
        out["sw1"] = _finite_e4m3_bytes(rng, (I, H))
        out["ss1"] = rng.integers(lo, hi, size=(I // 32, H // 32), dtype=np.uint8)
        out["sw3"] = _finite_e4m3_bytes(rng, (I, H))
        out["ss3"] = rng.integers(lo, hi, size=(I // 32, H // 32), dtype=np.uint8)
        out["sw2"] = _finite_e4m3_bytes(rng, (H, I))
        out["ss2"] = rng.integers(lo, hi, size=(H // 32, I // 32), dtype=np.uint8)
    return out


def pad_inter(inp: dict, I: int, I_pad: int) -> dict:
    """The layer's weights with the intermediate width I (a multiple of 32) widened to I_pad by zero codes:
    w1 / w3 (and the shared sw1 / sw3) gain rows of code 0, w2 (and sw2) input columns of code 0; the new
    scale bytes are 127 (1.0). Layout only: the padded rows give g = u = 0, so h = 0, whose QDQ codes are 0,
    and the padded w2 inputs are 0, so every output is the same value as with width I."""
    assert I % 32 == 0 and I_pad >= I and I_pad % 32 == 0
    n = I_pad - I
    out = dict(inp)

    def rows(a, cnt, axis, fill):
        shape = list(a.shape)
        shape[axis] = cnt
        return np.concatenate([a, np.full(shape, fill, dtype=a.dtype)], axis=axis)

    out["w1"], out["w3"] = rows(inp["w1"], n, 1, 0), rows(inp["w3"], n, 1, 0)
    out["s1"], out["s3"] = rows(inp["s1"], n, 1, 127), rows(inp["s3"], n, 1, 127)
    out["w2"], out["s2"] = rows(inp["w2"], n // 2, 2, 0), rows(inp["s2"], n // 32, 2, 127)
    if "sw1" in inp:
        out["sw1"], out["sw3"] = rows(inp["sw1"], n, 0, 0), rows(inp["sw3"], n, 0, 0)
        out["ss1"], out["ss3"] = rows(inp["ss1"], n // 32, 0, 127), rows(inp["ss3"], n // 32, 0, 127)
        out["sw2"], out["ss2"] = rows(inp["sw2"], n, 1, 0), rows(inp["ss2"], n // 32, 1, 127)
    return out


# The dense FP8 projection family of the page "Native 1017 DSpark draft on the NVLink pair (N1-NATIVE)" (section 4 "Dense"), N x K per rank.
DENSE_SHAPES = {
    "wq_a": (1280, 5120),
    "wkv": (512, 5120),
    "wq_b": (16384, 1280),
    "wo_b": (5120, 4096),
    "main_proj": (5120, 15360),
}


def make_dense_inputs(N: int, K: int, M: int, seed: int = 7) -> dict:
    """One dense FP8 linear: x bf16 bits [M, K] = RNE(N(0, 1)); w uniform over the finite E4M3 codes
    [N, K]; s E8M0 uniform in [118, 124] per 32x32 block [N/32, K/32]. Draw order: x, w, s."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = _to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = _finite_e4m3_bytes(rng, (N, K))
    s = rng.integers(118, 125, size=(N // 32, K // 32), dtype=np.uint8)
    return dict(x=x, w=w, s=s)


def digest(inputs: dict) -> dict:
    """sha256 of every generated tensor (recorded beside results)."""
    return {k: hashlib.sha256(np.ascontiguousarray(v).tobytes()).hexdigest()[:16]
            for k, v in sorted(inputs.items())}
