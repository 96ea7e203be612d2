"""Helpers shared by the GPU parity tests: upload seeded inputs, call the C ABI, compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import synth

# output tolerance of the layer against the oracle (max-abs relative to the reference's max-abs, and
# relative L2 norm)
MAX_ERR_RATIO = 2e-2
REL_L2 = 5e-3


def dev_tensor(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def upload(inp: dict) -> dict:
    return {k: dev_tensor(v) for k, v in inp.items() if isinstance(v, np.ndarray) and k not in ("hot_rows", "hot_experts")}


def dims_of(cfg, flags=0):
    import mxfp4_routed_expert_moe_amd as m
    return m.Dims(cfg.E, cfg.H, cfg.I, cfg.k, cfg.route_scale, flags)


def packed_of(d: dict):
    import mxfp4_routed_expert_moe_amd as m
    return m.MXFP4Experts(d["w1"], d["s1"], d["w3"], d["s3"], d["w2"], d["s2"])


def shared_of(d: dict):
    import mxfp4_routed_expert_moe_amd as m
    if "sw1" not in d:
        return None
    return m.FP8Expert(d["sw1"], d["ss1"], d["sw3"], d["ss3"], d["sw2"], d["ss2"])


def bf16_host(t: torch.Tensor) -> np.ndarray:
    """bf16 bit patterns on the device -> fp64 values on the host."""
    u = t.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def tiled_of(cfg, d: dict):
    """The packed experts with the prepared stage-major scales and the fragment-order copy of the codes (the
    layout the bench streams), with no row-major weight pointers."""
    import mxfp4_routed_expert_moe_amd as m
    pk = packed_of(d)
    st = m.moe_prepare_mxfp4_scales(dims_of(cfg), pk)
    tw = m.moe_prepare_mxfp4_weights(dims_of(cfg), pk)
    return m.MXFP4Experts(None, d["s1"], None, d["s3"], None, d["s2"], stage_scales=st, tiled_weights=tw)


def forward(cfg, d: dict, decoded=None, with_shared=True, M=None, packed=None, flags=0):
    """Run moe_forward; returns dict of host arrays (out, ids, rw, shared_out). packed: another form of the
    routed experts (e.g. tiled_of) instead of the row-major one; flags: moe_dims flags."""
    import mxfp4_routed_expert_moe_amd as m
    M = cfg.M if M is None else M
    dims = dims_of(cfg, flags)
    ws = m.workspace(dims, M)
    out = torch.empty((M, cfg.H), dtype=torch.int16, device="cuda")
    ids = torch.empty((M, cfg.k), dtype=torch.int32, device="cuda")
    rw = torch.empty((M, cfg.k), dtype=torch.float32, device="cuda")
    sh = shared_of(d) if with_shared else None
    sh_out = torch.empty((M, cfg.H), dtype=torch.int16, device="cuda") if sh is not None else None
    pk = None if decoded is not None else (packed if packed is not None else packed_of(d))
    m.moe_forward(dims, d["x"][:M], d["gate_w"], d["gate_b"], pk, decoded, sh, out, ids, rw, sh_out, ws)
    torch.cuda.synchronize()
    res = dict(out=bf16_host(out), ids=ids.cpu().numpy(), rw=rw.cpu().numpy(), out_bits=out.cpu().numpy(),
               rw_bits=rw.cpu().numpy().view(np.uint32))
    if sh_out is not None:
        res["shared_out"] = bf16_host(sh_out)
    return res


def tolerance(got: np.ndarray, ref: np.ndarray) -> tuple[float, float]:
    """(max|err| / max|ref|, ||err|| / ||ref||)."""
    err = np.abs(got - ref)
    return float(err.max() / max(np.abs(ref).max(), 1e-30)), float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-30))


def assert_within(got, ref, what=""):
    mx, l2 = tolerance(got, ref)
    assert mx <= MAX_ERR_RATIO and l2 <= REL_L2, f"{what}: max-err ratio {mx:.3g}, rel-L2 {l2:.3g}"
    return mx, l2


def check_routing(gpu_ids, gpu_rw, ref_route, cfg):
    """Routing parity: ids bit-exact except on tie-flagged tokens; rw within a few fp32 ulp.

    Returns the tokens whose ids differ (all tie-flagged) so the caller can condition the oracle."""
    ids_ref = ref_route["ids"]
    diff = np.nonzero(np.any(gpu_ids != ids_ref, axis=1))[0]
    untied = [int(t) for t in diff if not ref_route["tie"][t]]
    assert not untied, f"routing differs on tokens without a tie: {untied[:10]}"
    same = np.setdiff1d(np.arange(len(ids_ref)), diff)
    rel = np.abs(gpu_rw[same] - ref_route["rw"][same]) / np.abs(ref_route["rw"][same])
    assert rel.max(initial=0.0) <= 8 * 2.0 ** -23, f"route weights differ by {rel.max():.3g} relative"
    tot = gpu_rw.astype(np.float64).sum(axis=1)
    assert np.all(np.abs(tot - cfg.route_scale) <= (cfg.k + 2) * np.spacing(np.float32(cfg.route_scale)))
    return diff


def inputs(cid: int, **over):
    cfg = synth.get_config(cid, **over)
    return cfg, synth.make_inputs(cfg)
