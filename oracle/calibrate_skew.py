"""Write ``synth/c4_hot_bias.json``: the bias raise that gives the skewed prefill config's 8 hot
experts about half of all assignments (test infrastructure; calls only the oracle's router).

The generator adds this delta to the drawn selection bias of the hot experts. The bias only selects
experts ("Native 1017 DSpark draft on the NVLink pair (N1-NATIVE)", section 2 "Gate"), so the delta shifts routing without touching any
route weight. Bisection on delta until the hot share of the M*k assignments is within 0.5 +- 0.01.

    python -m oracle.calibrate_skew
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import synth  # noqa: E402
from oracle import moe  # noqa: E402


def hot_share(inp: dict, cfg, delta: float, base_bias: np.ndarray) -> float:
    b = base_bias.copy()
    hot = inp["hot_experts"]
    b[hot] = (b[hot] + np.float32(delta)).astype(np.float32)
    r = moe.route(inp["x"], inp["gate_w"], b, cfg.k, cfg.route_scale)
    return float(np.isin(r["ids"], hot).mean())


def calibrate(cid: int = 4, target: float = 0.5, tol: float = 0.01) -> dict:
    cfg = synth.get_config(cid)
    inp = synth.make_inputs(cfg, hot_delta=0.0)
    base = inp["gate_b"].copy()
    lo, hi = 0.0, 2.0
    share = hot_share(inp, cfg, hi, base)
    assert share > target, "upper bracket too small"
    delta = hi
    for _ in range(60):
        mid = 0.5 * (lo + hi)
        share = hot_share(inp, cfg, mid, base)
        delta = mid
        if abs(share - target) <= tol:
            break
        if share < target:
            lo = mid
        else:
            hi = mid
    delta = float(np.float32(delta))
    return dict(delta=delta, hot_share=hot_share(inp, cfg, delta, base), config=cfg.name,
                hot_experts=[int(e) for e in inp["hot_experts"]])


if __name__ == "__main__":
    res = calibrate()
    path = os.path.join(os.path.dirname(synth.__file__), "c4_hot_bias.json")
    with open(path, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    print(json.dumps(res))
