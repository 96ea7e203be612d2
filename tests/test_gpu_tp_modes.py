"""fp32 partial outputs for a tensor-parallel split of the intermediate width (modes SLOT and COMBINE of the
kernel contract, and the exact-official combine after the all-reduce), through the C ABI.

Bars: the fp32 slot sums round to exactly the bf16 slot outputs; the fp32 COMBINE sum equals the same
fp32 adds done on the host in ascending expert id; the exact-official combine of one rank's partials
equals moe_combine bit for bit; a two-rank split of I (each rank holding half of every expert's w1/w3
rows and w2 inputs, the all-reduce done as an fp32 add) meets the layer tolerance against the oracle.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import moe as O

from gpu_helpers import assert_within, bf16_host, check_routing, dims_of, inputs, packed_of, shared_of, upload

pytestmark = pytest.mark.gpu

# prefill width (row-tiled GEMMs) and decode width (streamed: M * k below 6 rows per expert on average)
CASES = [dict(M=300, H=512, I=256, E=8, k=2, shared=True), dict(M=23, H=512, I=256, E=8, k=2, shared=True)]
IDS = ["prefill_width", "decode_width"]


def m():
    import mxfp4_routed_expert_moe_amd as lib
    return lib


def _route(cfg, d):
    """Device routing, QDQ'd x and permutation from the ABI's own calls."""
    M, k, E, H = cfg.M, cfg.k, cfg.E, cfg.H
    dims = dims_of(cfg)
    dev = dict(device="cuda")
    r = dict(dims=dims, ws=m().workspace(dims, M),
             ids=torch.empty((M, k), dtype=torch.int32, **dev), rw=torch.empty((M, k), dtype=torch.float32, **dev),
             xq=torch.empty((M, H), dtype=torch.uint8, **dev), xs=torch.empty((M, H // 32), dtype=torch.uint8, **dev),
             counts=torch.empty(E, dtype=torch.int32, **dev), offsets=torch.empty(E + 1, dtype=torch.int32, **dev),
             pairs=torch.empty(M * k, dtype=torch.int32, **dev), active=torch.empty(E, dtype=torch.int32, **dev))
    m().moe_route(dims, d["x"], d["gate_w"], d["gate_b"], r["ids"], r["rw"], r["xq"], r["xs"], r["ws"])
    m().moe_permute(dims, r["ids"], r["counts"], r["offsets"], r["pairs"], None, r["active"])
    return r


def _bf16_bits_of_f32(a: np.ndarray) -> np.ndarray:
    return F.bf16_bits(F.bf16_rne(a.astype(np.float64)))


@pytest.mark.parametrize("over", CASES, ids=IDS)
def test_slot_f32_rounds_to_the_bf16_slots(over):
    cfg, inp = inputs(0, **over)
    d = upload(inp)
    r = _route(cfg, d)
    M, k, H = cfg.M, cfg.k, cfg.H
    slot = torch.empty((M * k, H), dtype=torch.int16, device="cuda")
    slot32 = torch.empty((M * k, H), dtype=torch.float32, device="cuda")
    m().moe_expert_ffn(r["dims"], r["xq"], r["xs"], packed_of(d), None, r["rw"], r["offsets"], r["pairs"], r["active"],
                       slot, ws=r["ws"])
    m().moe_expert_ffn_f32(r["dims"], r["xq"], r["xs"], packed_of(d), None, r["rw"], r["offsets"], r["pairs"],
                           r["active"], slot32, r["ws"])
    torch.cuda.synchronize()
    got = _bf16_bits_of_f32(slot32.cpu().numpy())
    assert np.array_equal(got, slot.cpu().numpy().view(np.uint16))
    # the shared expert likewise
    sh = torch.empty((M, H), dtype=torch.int16, device="cuda")
    sh32 = torch.empty((M, H), dtype=torch.float32, device="cuda")
    m().moe_shared_expert(r["dims"], r["xq"], r["xs"], shared_of(d), sh, r["ws"])
    m().moe_shared_expert_f32(r["dims"], r["xq"], r["xs"], shared_of(d), sh32, r["ws"])
    torch.cuda.synchronize()
    assert np.array_equal(_bf16_bits_of_f32(sh32.cpu().numpy()), sh.cpu().numpy().view(np.uint16))


@pytest.mark.parametrize("over", CASES, ids=IDS)
def test_combine_modes_on_fp32_slots(over):
    cfg, inp = inputs(0, **over)
    d = upload(inp)
    r = _route(cfg, d)
    M, k, H = cfg.M, cfg.k, cfg.H
    slot = torch.empty((M * k, H), dtype=torch.int16, device="cuda")
    slot32 = torch.empty((M * k, H), dtype=torch.float32, device="cuda")
    m().moe_expert_ffn(r["dims"], r["xq"], r["xs"], packed_of(d), None, r["rw"], r["offsets"], r["pairs"], r["active"],
                       slot, ws=r["ws"])
    m().moe_expert_ffn_f32(r["dims"], r["xq"], r["xs"], packed_of(d), None, r["rw"], r["offsets"], r["pairs"],
                           r["active"], slot32, r["ws"])
    sh = torch.empty((M, H), dtype=torch.int16, device="cuda")
    sh32 = torch.empty((M, H), dtype=torch.float32, device="cuda")
    m().moe_shared_expert(r["dims"], r["xq"], r["xs"], shared_of(d), sh, r["ws"])
    m().moe_shared_expert_f32(r["dims"], r["xq"], r["xs"], shared_of(d), sh32, r["ws"])
    # mode COMBINE: fp32 sums in ascending expert id, then the fp32 add input
    out32 = torch.empty((M, H), dtype=torch.float32, device="cuda")
    m().moe_combine_sum_f32(r["dims"], r["ids"], slot32, sh32, out32)
    # exact-official combine: equals moe_combine on the bf16 slots, with the shared part in either form
    ref_bf = torch.empty((M, H), dtype=torch.int16, device="cuda")
    m().moe_combine(r["dims"], r["ids"], slot, sh, ref_bf)
    off_a = torch.empty_like(ref_bf)
    off_b = torch.empty_like(ref_bf)
    m().moe_combine_official_f32(r["dims"], r["ids"], slot32, off_a, shared_bf16=sh)
    m().moe_combine_official_f32(r["dims"], r["ids"], slot32, off_b, shared_f32=sh32)
    torch.cuda.synchronize()
    assert torch.equal(off_a, ref_bf)
    assert torch.equal(off_b, ref_bf)
    ids = r["ids"].cpu().numpy()
    s32 = slot32.cpu().numpy().reshape(M, k, H)
    acc = np.zeros((M, H), dtype=np.float32)
    order = np.argsort(ids, axis=1, kind="stable")
    for j in range(k):
        acc = acc + s32[np.arange(M), order[:, j]]
    acc = acc + sh32.cpu().numpy()
    assert np.array_equal(out32.cpu().numpy().view(np.uint32), acc.view(np.uint32))


def _rank_slices(inp, cfg, r, G):
    """Rank r of G: its share of every expert's w1/w3 rows and w2 inputs (and the shared expert's)."""
    I, Ig = cfg.I, cfg.I // G
    lo, hi = r * Ig, (r + 1) * Ig
    out = dict(inp)
    out["w1"], out["w3"] = inp["w1"][:, lo:hi], inp["w3"][:, lo:hi]
    out["s1"], out["s3"] = inp["s1"][:, lo:hi], inp["s3"][:, lo:hi]
    out["w2"], out["s2"] = inp["w2"][:, :, lo // 2:hi // 2], inp["s2"][:, :, lo // 32:hi // 32]
    out["sw1"], out["sw3"] = inp["sw1"][lo:hi], inp["sw3"][lo:hi]
    out["ss1"], out["ss3"] = inp["ss1"][lo // 32:hi // 32], inp["ss3"][lo // 32:hi // 32]
    out["sw2"], out["ss2"] = inp["sw2"][:, lo:hi], inp["ss2"][:, lo // 32:hi // 32]
    return {key: np.ascontiguousarray(v) if isinstance(v, np.ndarray) else v for key, v in out.items()}


@pytest.mark.parametrize("over", CASES, ids=IDS)
def test_two_rank_split_of_inter_meets_the_layer_tolerance(over):
    """Each rank holds I/2 of every expert (QDQ blocks never straddle the cut): fp32 SLOT partials and fp32
    shared partials, an fp32 add as the all-reduce, then the exact-official combine."""
    cfg, inp = inputs(0, **over)
    d = upload(inp)
    r = _route(cfg, d)
    M, k, H, G = cfg.M, cfg.k, cfg.H, 2
    rcfg = synth.get_config(0, **dict(over, I=cfg.I // G))
    rdims = dims_of(rcfg)
    rws = m().workspace(rdims, M)
    slot_sum = torch.zeros((M * k, H), dtype=torch.float32, device="cuda")
    sh_sum = torch.zeros((M, H), dtype=torch.float32, device="cuda")
    for rank in range(G):
        dr = upload(_rank_slices(inp, cfg, rank, G))
        part = torch.empty((M * k, H), dtype=torch.float32, device="cuda")
        shp = torch.empty((M, H), dtype=torch.float32, device="cuda")
        m().moe_expert_ffn_f32(rdims, r["xq"], r["xs"], packed_of(dr), None, r["rw"], r["offsets"], r["pairs"],
                               r["active"], part, rws)
        m().moe_shared_expert_f32(rdims, r["xq"], r["xs"], shared_of(dr), shp, rws)
        slot_sum += part
        sh_sum += shp
    out = torch.empty((M, H), dtype=torch.int16, device="cuda")
    m().moe_combine_official_f32(r["dims"], r["ids"], slot_sum, out, shared_f32=sh_sum)
    torch.cuda.synchronize()
    ids, rw = r["ids"].cpu().numpy(), r["rw"].cpu().numpy()
    ref = O.moe_forward(inp, cfg)
    diff = check_routing(ids, rw, ref["route"], cfg)
    if diff.size:
        ref = O.moe_forward(inp, cfg, ids=ids, rw=rw)
    mx, l2 = assert_within(bf16_host(out), ref["out"], f"TP2 {over}")
    print(f"TP2 {over}: max-err ratio {mx:.3g}, rel-L2 {l2:.3g}")
    # the routed part alone (the shared expert dominates the sum)
    routed = torch.empty_like(out)
    m().moe_combine_official_f32(r["dims"], r["ids"], slot_sum, routed)
    torch.cuda.synchronize()
    assert_within(bf16_host(routed), O.combine(ref["ids"], ref["slot_y"], None), f"TP2 routed part {over}")


@pytest.mark.parametrize("over", CASES, ids=IDS)
def test_four_rank_split_with_zero_padded_shares(over):
    """A split of I whose shares are multiples of 32 but not of 128 (I = 384 over four ranks: 96 each, as
    2304 over four gives 576): each rank's share is widened to 128 with zero codes (synth.pad_inter), which
    the library takes, and the four fp32 partials sum to the layer within the layer tolerance."""
    over = dict(over, I=384)
    cfg, inp = inputs(0, **over)
    d = upload(inp)
    r = _route(cfg, d)
    M, k, H, G = cfg.M, cfg.k, cfg.H, 4
    Ig, Ipad = cfg.I // G, 128
    rdims = dims_of(synth.get_config(0, **dict(over, I=Ipad)))
    rws = m().workspace(rdims, M)
    slot_sum = torch.zeros((M * k, H), dtype=torch.float32, device="cuda")
    sh_sum = torch.zeros((M, H), dtype=torch.float32, device="cuda")
    for rank in range(G):
        dr = upload(synth.pad_inter(_rank_slices(inp, cfg, rank, G), Ig, Ipad))
        part = torch.empty((M * k, H), dtype=torch.float32, device="cuda")
        shp = torch.empty((M, H), dtype=torch.float32, device="cuda")
        m().moe_expert_ffn_f32(rdims, r["xq"], r["xs"], packed_of(dr), None, r["rw"], r["offsets"], r["pairs"],
                               r["active"], part, rws)
        m().moe_shared_expert_f32(rdims, r["xq"], r["xs"], shared_of(dr), shp, rws)
        slot_sum += part
        sh_sum += shp
    out = torch.empty((M, H), dtype=torch.int16, device="cuda")
    m().moe_combine_official_f32(r["dims"], r["ids"], slot_sum, out, shared_f32=sh_sum)
    routed = torch.empty_like(out)
    m().moe_combine_official_f32(r["dims"], r["ids"], slot_sum, routed)
    torch.cuda.synchronize()
    ids, rw = r["ids"].cpu().numpy(), r["rw"].cpu().numpy()
    ref = O.moe_forward(inp, cfg)
    diff = check_routing(ids, rw, ref["route"], cfg)
    if diff.size:
        ref = O.moe_forward(inp, cfg, ids=ids, rw=rw)
    mx, l2 = assert_within(bf16_host(out), ref["out"], f"TP4 padded {over}")
    assert_within(bf16_host(routed), O.combine(ref["ids"], ref["slot_y"], None), f"TP4 padded routed part {over}")
    print(f"TP4 (shares of 96 padded to 128) {over}: max-err ratio {mx:.3g}, rel-L2 {l2:.3g}")
