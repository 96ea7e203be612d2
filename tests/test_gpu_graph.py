"""moe_forward captured in a HIP graph: every replay on changed inputs equals the eager call bit for bit.

The library enqueues kernels only (no allocation, no host synchronization, no memset), and launch
geometry depends only on (dims, M), so one captured graph serves every batch of the same M. Each replay
is checked against an eager call on the same inputs, with eager work and a synchronization between
replays.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import dev_tensor, dims_of, inputs, packed_of, shared_of, upload

pytestmark = pytest.mark.gpu


def m():
    import mxfp4_routed_expert_moe_amd as lib
    return lib


def _buffers(cfg, d, with_shared):
    M = cfg.M
    dims = dims_of(cfg)
    return dict(
        dims=dims,
        ws=m().workspace(dims, M),
        x=d["x"].clone(),
        out=torch.empty((M, cfg.H), dtype=torch.int16, device="cuda"),
        ids=torch.empty((M, cfg.k), dtype=torch.int32, device="cuda"),
        rw=torch.empty((M, cfg.k), dtype=torch.float32, device="cuda"),
        shared=shared_of(d) if with_shared else None,
    )


def _call(b, d):
    m().moe_forward(b["dims"], b["x"], d["gate_w"], d["gate_b"], packed_of(d), None, b["shared"], b["out"], b["ids"],
                    b["rw"], None, b["ws"])


@pytest.mark.parametrize("cid,over,with_shared", [
    (2, {}, False),                                            # decode width (M = 64)
    (0, dict(M=1000, H=512, I=256, E=8, k=2), False),          # prefill path (block-scaled MFMA)
    (0, dict(M=300, H=256, I=128, E=8, k=2, shared=True), True),  # prefill path + FP8 shared expert
])
def test_graph_replay_equals_eager_on_changed_inputs(cid, over, with_shared):
    cfg, inp = inputs(cid, **over)
    d = upload(inp)
    g_buf = _buffers(cfg, d, with_shared)
    e_buf = _buffers(cfg, d, with_shared)
    # warm up on a side stream, then capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _call(g_buf, d)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _call(g_buf, d)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    for it in range(4):
        # new activations: permuted rows of the seeded batch, some rows negated (changes routing and values)
        perm = rng.permutation(cfg.M)
        xb = inp["x"][perm].copy()
        flip = rng.random(cfg.M) < 0.3
        xb[flip] ^= np.uint16(0x8000)
        xt = dev_tensor(xb)
        g_buf["x"].copy_(xt)
        e_buf["x"].copy_(xt)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _call(e_buf, d)            # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(g_buf["ids"], e_buf["ids"]), f"replay {it}: routing differs from eager"
        assert torch.equal(g_buf["rw"], e_buf["rw"]), f"replay {it}: route weights differ from eager"
        assert torch.equal(g_buf["out"], e_buf["out"]), f"replay {it}: output differs from eager"


def test_graph_replay_of_the_fp32_slot_and_combine_modes():
    """route -> permute -> SLOT fp32 expert FFN -> COMBINE fp32 sum and exact-official combine, captured
    once and replayed on changed activations: every replay equals the eager calls bit for bit."""
    cfg, inp = inputs(0, M=300, H=256, I=128, E=8, k=2)
    d = upload(inp)
    M, k, H, E = cfg.M, cfg.k, cfg.H, cfg.E
    dims = dims_of(cfg)
    dev = dict(device="cuda")

    def bufs():
        return dict(ws=m().workspace(dims, M), x=d["x"].clone(),
                    ids=torch.empty((M, k), dtype=torch.int32, **dev), rw=torch.empty((M, k), dtype=torch.float32, **dev),
                    xq=torch.empty((M, H), dtype=torch.uint8, **dev), xs=torch.empty((M, H // 32), dtype=torch.uint8, **dev),
                    counts=torch.empty(E, dtype=torch.int32, **dev), offsets=torch.empty(E + 1, dtype=torch.int32, **dev),
                    pairs=torch.empty(M * k, dtype=torch.int32, **dev), active=torch.empty(E, dtype=torch.int32, **dev),
                    slot=torch.empty((M * k, H), dtype=torch.float32, **dev),
                    sum=torch.empty((M, H), dtype=torch.float32, **dev), out=torch.empty((M, H), dtype=torch.int16, **dev))

    def run(b):
        m().moe_route(dims, b["x"], d["gate_w"], d["gate_b"], b["ids"], b["rw"], b["xq"], b["xs"], b["ws"])
        m().moe_permute(dims, b["ids"], b["counts"], b["offsets"], b["pairs"], None, b["active"])
        m().moe_expert_ffn_f32(dims, b["xq"], b["xs"], packed_of(d), None, b["rw"], b["offsets"], b["pairs"],
                               b["active"], b["slot"], b["ws"])
        m().moe_combine_sum_f32(dims, b["ids"], b["slot"], None, b["sum"])
        m().moe_combine_official_f32(dims, b["ids"], b["slot"], b["out"])

    g_buf, e_buf = bufs(), bufs()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run(g_buf)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(g_buf)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    for it in range(4):
        xb = inp["x"][rng.permutation(M)].copy()
        xt = dev_tensor(xb)
        g_buf["x"].copy_(xt)
        e_buf["x"].copy_(xt)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        run(e_buf)
        torch.cuda.synchronize()
        for key in ("ids", "slot", "sum", "out"):
            assert torch.equal(g_buf[key], e_buf[key]), f"replay {it}: {key} differs from eager"


@pytest.mark.parametrize("N,K,M,tiled", [
    (5120, 4096, 8, False),    # wo_b: K split into runs + the run reduce
    (5120, 4096, 8, True),     # the same on the fragment-order weights
    (16384, 1280, 5, True),    # wq_b: one run, no reduce
])
def test_graph_replay_of_the_dense_fp8_linear(N, K, M, tiled):
    """moe_fp8_linear (or _tiled) captured once and replayed on changed activations: every replay equals an
    eager call on the same inputs bit for bit, with eager work and a synchronization between replays."""
    import synth
    inp = synth.make_dense_inputs(N, K, M, seed=31)
    w, s = dev_tensor(inp["w"]), dev_tensor(inp["s"])
    wl = m().moe_prepare_fp8_weights(w) if tiled else w

    def call(x, y, ws):
        if tiled:
            m().moe_fp8_linear_tiled(x, wl, N, s, y=y, ws=ws)
        else:
            m().moe_fp8_linear(x, wl, s, y=y, ws=ws)

    xg, xe = dev_tensor(inp["x"]), dev_tensor(inp["x"])
    yg, ye = (torch.empty((M, N), dtype=torch.int16, device="cuda") for _ in range(2))
    wsg, wse = m().fp8_linear_workspace(M, N, K), m().fp8_linear_workspace(M, N, K)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(xg, yg, wsg)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(xg, yg, wsg)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    for it in range(4):
        xb = inp["x"][rng.permutation(M)].copy()
        xb[rng.random(M) < 0.3] ^= np.uint16(0x8000)
        xt = dev_tensor(xb)
        xg.copy_(xt)
        xe.copy_(xt)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        call(xe, ye, wse)          # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(yg, ye), f"replay {it}: dense output differs from eager"
