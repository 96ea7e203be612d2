"""Throughput of the routed-MoE FFN layer (MXFP4 experts) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode_m8] [--replicas R]
                    [--no-prefill] [--no-cpu-baseline]

A step is one call of ``moe_forward`` (router + activation QDQ, permutation, grouped w1/w3 GEMM with
SwiGLU and QDQ of h, grouped w2 GEMM, fixed-order combine) over one batch of seeded synthetic tokens.
Inputs are resident in HBM before the timed region starts. The expert weights exist in R replicas and
step i uses replica i mod R, so the 256 MB last-level cache cannot serve them from a previous step.

Printed: one JSON line. ``value`` is tokens/s of the M=8 decode-width layer (hidden 5120, 128 MXFP4
experts, intermediate 2304, top-6). ``roofline`` describes the dominant kernel, the grouped w1/w3 GEMM.
``prefill`` holds the same figures for the M=8192 prefill layer. ``cpu_baseline`` is the CPU oracle timed
on a bounded sample of the decode workload on this host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_FP8_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 MFMA, published (E4M3 x E2M1 issues at the FP8 rate)

WORKLOADS = {"tiny_m4": 0, "decode_m8": 1, "batched_decode_m64": 2, "prefill_m8192": 3,
             "prefill_shared_skew_m2048": 4}

# L2<->memory bytes of the w1/w3 GEMM per launch, from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE runs (KiB per
# dispatch). A 1 GiB device copy reads FETCH_SIZE = 524300 KiB and WRITE_SIZE = 1048576 KiB on this GPU, so the
# fetch counter is scaled by 2.0 and the write counter by 1.0. The figures hold only for the kernel source they
# were measured on (sha256 prefix); after any change to it the traffic is reported as null until re-measured.
FETCH_SCALE, WRITE_SCALE = 1048576 / 524300.9, 1.0
MEASURED_TRAFFIC = {
    "decode_m8": dict(src="expert_gemm.hip", sha="129a4bb763d14ee8", fetch_kib=228000.9, write_kib=135.2),
    "prefill_m8192": dict(src="expert_mfma.hip", sha="2adfd3c215134d8e", fetch_kib=1784893.9, write_kib=166161.4),
}


def _measured_traffic(workload: str):
    import hashlib
    m = MEASURED_TRAFFIC.get(workload)
    if m is None:
        return None
    path = os.path.join(ROOT, "mxfp4_routed_expert_moe_amd", "csrc", m["src"])
    with open(path, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest()[:16] != m["sha"]:
            return None
    return int(round((m["fetch_kib"] * FETCH_SCALE + m["write_kib"] * WRITE_SCALE) * 1024))


def _bytes_per_expert(cfg):
    """Packed MXFP4 bytes (codes + E8M0 scales) of one expert: (w1 + w3, w2)."""
    H, I = cfg.H, cfg.I
    w13 = 2 * (I * H // 2 + I * H // 32)
    w2 = H * I // 2 + H * I // 32
    return w13, w2


def _flops_per_pair(cfg):
    """Multiply-add flops of one (token, expert) assignment: (w1 + w3, w2)."""
    return 2 * 2 * cfg.I * cfg.H, 2 * cfg.H * cfg.I


class Layer:
    """Device-resident inputs of one workload with R weight replicas, plus output buffers."""

    def __init__(self, cid: int, replicas: int, tiled: bool = True):
        import numpy as np
        import torch

        import mxfp4_routed_expert_moe_amd as moe
        import synth

        self.moe, self.torch, self.np = moe, torch, np
        self.cfg = cfg = synth.get_config(cid)
        inp = synth.make_inputs(cfg)
        self.digest = synth.digest({k: v for k, v in inp.items() if k in ("x", "gate_w", "gate_b", "w1", "w2")})

        def up(a):
            if a.dtype == np.uint16:
                a = a.view(np.int16)
            return torch.from_numpy(np.ascontiguousarray(a)).cuda()

        self.x, self.gate_w, self.gate_b = up(inp["x"]), up(inp["gate_w"]), up(inp["gate_b"])
        first = {n: up(inp[n]) for n in ("w1", "s1", "w3", "s3", "w2", "s2")}
        self.experts = [moe.MXFP4Experts(**first)]
        for _ in range(1, replicas):
            self.experts.append(moe.MXFP4Experts(**{n: t.clone() for n, t in first.items()}))
        self.shared = None
        if cfg.shared:
            self.shared = moe.FP8Expert(*(up(inp[n]) for n in ("sw1", "ss1", "sw3", "ss3", "sw2", "ss2")))
        del inp
        M, k, H, I, E = cfg.M, cfg.k, cfg.H, cfg.I, cfg.E
        self.dims = moe.Dims(E, H, I, k, cfg.route_scale)
        # one-time re-layouts at weight load: each replica's scales stage-major for the prefill-width kernels,
        # and (by default) its weight codes in fragment order, which then replace the stored row-major codes
        for w in self.experts:
            w.stage_scales = moe.moe_prepare_mxfp4_scales(self.dims, w)
            if tiled:
                w.tiled_weights = moe.moe_prepare_mxfp4_weights(self.dims, w)
                torch.cuda.synchronize()
                w.w1 = w.w3 = w.w2 = None
        self.weight_layout = "fragment-order" if tiled else "stored row-major"
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        self.ws = moe.workspace(self.dims, M)
        dev = dict(device="cuda")
        self.out = torch.empty((M, H), dtype=torch.int16, **dev)
        self.ids = torch.empty((M, k), dtype=torch.int32, **dev)
        self.rw = torch.empty((M, k), dtype=torch.float32, **dev)
        # buffers of the split entry points (kernel-level timing)
        self.xq = torch.empty((M, H), dtype=torch.uint8, **dev)
        self.xs = torch.empty((M, H // 32), dtype=torch.uint8, **dev)
        self.counts = torch.empty(E, dtype=torch.int32, **dev)
        self.offsets = torch.empty(E + 1, dtype=torch.int32, **dev)
        self.pairs = torch.empty(M * k, dtype=torch.int32, **dev)
        self.active = torch.empty(E, dtype=torch.int32, **dev)
        self.hq = torch.empty((M * k, I), dtype=torch.uint8, **dev)
        self.hs = torch.empty((M * k, I // 32), dtype=torch.uint8, **dev)
        self.slot = torch.empty((M * k, H), dtype=torch.int16, **dev)
        self.shared_out = torch.empty((M, H), dtype=torch.int16, **dev) if self.shared is not None else None

    def step(self, i: int):
        self.moe.moe_forward(self.dims, self.x, self.gate_w, self.gate_b, self.experts[i % len(self.experts)], None,
                             self.shared, self.out, self.ids, self.rw, None, self.ws)

    def gemm1_only(self, i: int):
        """GEMM1 alone on replica i, with the routing and activations left by the last split_step."""
        self.moe.moe_expert_gemm1(self.dims, self.xq, self.xs, self.experts[i % len(self.experts)], None, self.rw,
                                  self.offsets, self.pairs, self.active, self.hq, self.hs, self.ws)

    def split_step(self, i: int, ev):
        """The same layer through the split entry points, with events between the kernels."""
        m, w = self.moe, self.experts[i % len(self.experts)]
        ev[0].record()
        m.moe_route(self.dims, self.x, self.gate_w, self.gate_b, self.ids, self.rw, self.xq, self.xs, self.ws)
        ev[1].record()
        m.moe_permute(self.dims, self.ids, self.counts, self.offsets, self.pairs, None, self.active)
        ev[2].record()
        m.moe_expert_gemm1(self.dims, self.xq, self.xs, w, None, self.rw, self.offsets, self.pairs, self.active,
                           self.hq, self.hs, self.ws)
        ev[3].record()
        m.moe_expert_gemm2(self.dims, self.cfg.M, self.hq, self.hs, w, None, self.offsets, self.pairs, self.active,
                           self.slot, self.ws)
        ev[4].record()
        if self.shared is not None:
            m.moe_shared_expert(self.dims, self.xq, self.xs, self.shared, self.shared_out, self.ws)
        ev[5].record()
        m.moe_combine(self.dims, self.ids, self.slot, self.shared_out, self.out)
        ev[6].record()

    def distinct_experts(self) -> int:
        return int(self.torch.unique(self.ids).numel())


VERIFIER_WIDTHS = (1, 2, 4, 5, 10, 15, 20, 32)


def measure_widths(L: Layer, widths, steps: int, warmup: int) -> dict:
    """The same layer weights (all replicas) at the verifier widths M: moe_forward eager over rotated
    replicas, and the same steps replayed from a HIP graph. Token rows are the workload's own draw,
    extended (the first rows are the decode batch's)."""
    import dataclasses

    import numpy as np
    import torch

    import synth

    moe, cfg = L.moe, L.cfg
    Mx = max(widths)
    xw = torch.from_numpy(synth.make_tokens(dataclasses.replace(cfg, M=Mx)).view(np.int16)).cuda()
    dev = dict(device="cuda")
    ws = moe.workspace(L.dims, Mx)
    out = torch.empty((Mx, cfg.H), dtype=torch.int16, **dev)
    ids = torch.empty((Mx, cfg.k), dtype=torch.int32, **dev)
    rw = torch.empty((Mx, cfg.k), dtype=torch.float32, **dev)
    R = len(L.experts)
    w13_b, w2_b = _bytes_per_expert(cfg)
    res = {}
    for m in widths:
        def step(i):
            moe.moe_forward(L.dims, xw[:m], L.gate_w, L.gate_b, L.experts[i % R], None, L.shared, out[:m],
                            ids[:m], rw[:m], None, ws)
        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        us = float("inf")
        for _ in range(2):   # the better of two timed passes: one host stall should not set a width's figure
            t0 = time.perf_counter()
            for i in range(steps):
                step(warmup + i)
            torch.cuda.synchronize()
            us = min(us, (time.perf_counter() - t0) * 1e6 / steps)
        D = int(torch.unique(ids[:m]).numel())
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(R):
                step(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(R):
                step(i)
        graph.replay()
        torch.cuda.synchronize()
        n_rep = max(2, steps // R)
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(n_rep):
            graph.replay()
        g1.record()
        torch.cuda.synchronize()
        gus = g0.elapsed_time(g1) * 1e3 / (n_rep * R)
        del graph
        nbytes = D * (w13_b + w2_b)
        res[str(m)] = dict(us=round(us, 1), graph_us=round(gus, 1), tokens_per_s=round(m / (us * 1e-6), 1),
                           distinct_experts=D, weight_hbm_frac=round(nbytes / (us * 1e-6) / (HBM_PEAK_GBS * 1e9), 4))
    del ws, out, ids, rw, xw
    return res


def measure(cid: int, steps: int, warmup: int, replicas: int, widths=None, tiled: bool = True) -> dict:
    import torch

    L = Layer(cid, replicas, tiled)
    cfg = L.cfg
    for i in range(warmup):
        L.step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        L.step(warmup + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / steps
    D = L.distinct_experts()

    # kernel-level times: events between the split entry points, on the stream they launch on
    names = ["route", "permute", "gemm1", "gemm2", "shared", "combine"]
    tot = [0.0] * len(names)
    n_k = max(steps, 5)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(n_k)]
    for i in range(warmup):
        L.split_step(i, evs[0])
    torch.cuda.synchronize()
    for i in range(n_k):
        L.split_step(warmup + i, evs[i])
    torch.cuda.synchronize()
    for ev in evs:
        for j in range(len(names)):
            tot[j] += ev[j].elapsed_time(ev[j + 1])
    kern_us = {n: 1e3 * t / n_k for n, t in zip(names, tot)}
    if L.shared is None:
        kern_us.pop("shared")
    # GEMM1's own duration for the roofline: back-to-back launches over the weight replicas (same routing;
    # each launch streams another replica, so no launch finds its weights in cache), one event pair around
    # the batch, so the per-call event and dispatch gaps of the split pass do not enter it
    n_b = max(n_k, 2 * len(L.experts))
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    L.gemm1_only(0)
    torch.cuda.synchronize()
    b0.record()
    for i in range(n_b):
        L.gemm1_only(1 + i)
    b1.record()
    torch.cuda.synchronize()
    gemm1_us = b0.elapsed_time(b1) * 1e3 / n_b

    w13_b, w2_b = _bytes_per_expert(cfg)
    f13, f2 = _flops_per_pair(cfg)
    P = cfg.M * cfg.k
    gemm1_bytes = D * w13_b + cfg.M * (cfg.H + cfg.H // 32) + P * (cfg.I + cfg.I // 32)
    gemm1_flops = P * f13
    layer_bytes = D * (w13_b + w2_b) + cfg.E * cfg.H * 4
    # the same steps replayed from a HIP graph (one capture of R steps, one per weight replica): no host
    # launch work between the kernels
    R = len(L.experts)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(R):
            L.step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(R):
            L.step(i)
    graph.replay()
    torch.cuda.synchronize()
    n_rep = max(1, steps // R)
    g0, g1e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record()
    for _ in range(n_rep):
        graph.replay()
    g1e.record()
    torch.cuda.synchronize()
    graph_ms = g0.elapsed_time(g1e) / (n_rep * R)
    del graph

    res = dict(workload=cfg.name, M=cfg.M, ms_per_step=ms, tokens_per_s=cfg.M / (ms * 1e-3), distinct_experts=D,
               graph_ms_per_step=graph_ms,
               kernel_us=kern_us, layer_weight_bytes=layer_bytes,
               layer_hbm_frac=(layer_bytes / (ms * 1e-3)) / (HBM_PEAK_GBS * 1e9),
               layer_tflops=(P * (f13 + f2)) / (ms * 1e-3) / 1e12, replicas=replicas, inputs_sha256=L.digest)
    g1 = gemm1_us * 1e-6
    timing = dict(avg_us_timing=f"HIP events around {n_b} back-to-back launches on the launch stream",
                  avg_us_per_call_events=round(kern_us["gemm1"], 2))
    if cfg.M <= 64:
        ach = gemm1_bytes / g1 / 1e9
        res["roofline"] = dict(kernel="expert_gemm1 (w1/w3 + SwiGLU + QDQ)", bound="hbm", achieved=round(ach, 1),
                               peak=HBM_PEAK_GBS, unit="GB/s", frac=round(ach / HBM_PEAK_GBS, 4),
                               traffic=_measured_traffic(cfg.name),
                               algorithmic_bytes=gemm1_bytes, avg_us=round(gemm1_us, 2), **timing)
    else:
        ach = gemm1_flops / g1 / 1e12
        res["roofline"] = dict(kernel="expert_gemm1 (w1/w3 + SwiGLU + QDQ)", bound="mfma", achieved=round(ach, 1),
                               peak=MFMA_FP8_PEAK_TFLOPS, unit="TFLOP/s", frac=round(ach / MFMA_FP8_PEAK_TFLOPS, 4),
                               traffic=_measured_traffic(cfg.name), algorithmic_flops=gemm1_flops,
                               avg_us=round(gemm1_us, 2), **timing)
    if widths:
        res["widths"] = measure_widths(L, widths, steps, warmup)
    del L
    torch.cuda.empty_cache()
    return res


def measure_dense(M: int = 8, reps: int = 40, pool_bytes: int = 1 << 30, tiled: bool = True) -> dict:
    """The dense FP8 projection family at decode width: moe_fp8_linear per shape (by default on the
    fragment-order copy of the weights made at load, moe_fp8_linear_tiled), with the weights in as
    many replicas as fill about 1 GiB (rotated, so the 256 MB last-level cache cannot serve them). The
    calls are captured once in a HIP graph (the library is graph-safe) and the replays timed with HIP
    events, so host launch overhead does not enter the per-call time."""
    import numpy as np
    import torch

    import mxfp4_routed_expert_moe_amd as moe
    import synth

    out = {}
    for name, (N, K) in synth.DENSE_SHAPES.items():
        inp = synth.make_dense_inputs(N, K, M)
        x = torch.from_numpy(inp["x"].view(np.int16)).cuda()
        replicas = max(4, -(-pool_bytes // (N * K)))
        w0, s0 = torch.from_numpy(inp["w"]).cuda(), torch.from_numpy(inp["s"]).cuda()
        if tiled:
            ws_ = [(moe.moe_prepare_fp8_weights(w0), s0.clone()) for _ in range(replicas)]
        else:
            ws_ = [(w0.clone(), s0.clone()) for _ in range(replicas)]
        torch.cuda.synchronize()
        y = torch.empty((M, N), dtype=torch.int16, device="cuda")
        work = moe.fp8_linear_workspace(M, N, K)

        def call(i):
            w_i, s_i = ws_[i % replicas]
            if tiled:
                moe.moe_fp8_linear_tiled(x, w_i, N, s_i, y=y, ws=work)
            else:
                moe.moe_fp8_linear(x, w_i, s_i, y=y, ws=work)

        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(replicas):
                call(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        per_graph = replicas
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(per_graph):
                call(i)
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n_rep = max(2, reps // per_graph)
        e0.record()
        for _ in range(n_rep):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (n_rep * per_graph)
        del graph
        nbytes = N * K + (N // 32) * (K // 32) + M * K * 2 + M * N * 2
        out[name] = dict(N=N, K=K, replicas=replicas, us=round(us, 2), gbs=round(nbytes / (us * 1e-6) / 1e9, 1),
                         hbm_frac=round(nbytes / (us * 1e-6) / (HBM_PEAK_GBS * 1e9), 4))
        del ws_, work, w0, s0
    torch.cuda.empty_cache()
    return dict(workload=f"dense FP8 projections at M={M}", bound="hbm", unit="GB/s",
                weight_layout="fragment-order" if tiled else "stored row-major", shapes=out)


def calibrate_copy(gib: int = 1, reps: int = 5) -> dict:
    """A plain device-to-device copy of a known size (the reference for the L2 byte counters)."""
    import torch
    n = gib << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    return dict(bytes_read=n, bytes_written=n, us=round(dt * 1e6, 1), gbs=round(2 * n / dt / 1e9, 1))


def cpu_baseline(budget_tokens: int = 8) -> dict:
    """The CPU oracle, as it stands, on the first token(s) of the decode workload."""
    import synth
    from oracle import moe as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: the BLAS pool size is unknown, report the host count
        cores = os.cpu_count() or 1
    cfg = synth.get_config(1)
    inp = synth.make_inputs(cfg)
    toks = list(range(budget_tokens))
    t0 = time.perf_counter()
    O.moe_forward(inp, cfg, tokens=toks)
    dt = time.perf_counter() - t0
    return dict(value=round(len(toks) / dt, 5), unit="tokens/s", cores=cores, kind="oracle",
                sample=f"{len(toks)} token(s) of decode_m8 (router, QDQ, its {cfg.k} experts decoded from MXFP4, "
                       f"fp64 dot products, combine); {dt:.1f} s")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_m8", choices=sorted(WORKLOADS))
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--no-prefill", action="store_true", help="skip the M=8192 measurement")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense FP8 projection family")
    ap.add_argument("--no-widths", action="store_true", help="skip the verifier widths M = 1 .. 32")
    ap.add_argument("--stored-layout", action="store_true",
                    help="stream the weight codes (routed experts and the dense FP8 family) from their stored "
                         "row-major layout instead of the fragment-order copy made at load")
    ap.add_argument("--dense-only", action="store_true",
                    help="only the dense FP8 projection family (prints its object as the JSON line)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy (reference for the rocprof byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: the layer is measured on a single MI355X (asked for --gpus {args.gpus}); "
              "sharding across GPUs is not part of this library", file=sys.stderr)
        sys.exit(2)

    import torch
    import mxfp4_routed_expert_moe_amd  # noqa: F401  (fails loudly if libmoe.so is missing)

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        print(json.dumps({"calibrate_copy": calibrate_copy()}), flush=True)
        return
    if args.dense_only:
        print(json.dumps({"dense_fp8": measure_dense(tiled=not args.stored_layout)}), flush=True)
        return
    widths = VERIFIER_WIDTHS if (args.workload == "decode_m8" and not args.no_widths) else None
    tiled = not args.stored_layout
    main_res = measure(WORKLOADS[args.workload], args.steps, args.warmup, args.replicas, widths, tiled)
    print(f"# {main_res['workload']}: {main_res['ms_per_step'] * 1e3:.1f} us/step "
          f"(graph {main_res['graph_ms_per_step'] * 1e3:.1f}), kernels {main_res['kernel_us']}",
          file=sys.stderr, flush=True)
    if main_res.get("widths"):
        print("# widths: " + ", ".join(f"M={m}: {v['us']} us ({v['distinct_experts']} experts)"
                                       for m, v in main_res["widths"].items()), file=sys.stderr, flush=True)
    prefill = None
    if not args.no_prefill and args.workload != "prefill_m8192":
        p = measure(3, max(3, args.steps // 10), max(1, args.warmup // 5), 2, tiled=tiled)
        print(f"# {p['workload']}: {p['ms_per_step']:.3f} ms/step, kernels {p['kernel_us']}", file=sys.stderr,
              flush=True)
        prefill = dict(workload=p["workload"], value=round(p["tokens_per_s"], 1), unit="tokens/s",
                       ms_per_step=round(p["ms_per_step"], 4), kernel_us={k: round(v, 1) for k, v in
                                                                          p["kernel_us"].items()},
                       graph_ms_per_step=round(p["graph_ms_per_step"], 4),
                       layer_tflops=round(p["layer_tflops"], 1), roofline=p["roofline"])
    dense = None
    if not args.no_dense:
        dense = measure_dense(tiled=not args.stored_layout)
        summary = ", ".join(f"{k}: {v['us']} us" for k, v in dense["shapes"].items())
        print(f"# dense: {summary}", file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline()
    r = main_res
    line = {
        "metric": "MoE-layer tokens/s at M=8 and M=8192; % of HBM BW / MXFP4 MFMA roofline",
        "value": round(r["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 x mxfp4 (fp32 accumulate, bf16 out)",
        "data": "synthetic (seeded)",
        "config": {"workload": r["workload"], "M": r["M"], "hidden": 5120, "experts": 128, "inter": 2304,
                   "top_k": 6, "distinct_experts": r["distinct_experts"], "weight_replicas": r["replicas"],
                   "weight_layout": "stored row-major" if args.stored_layout else "fragment-order",
                   "parallelism": "none (1 GPU)"},
        "graph_ms_per_step": round(r["graph_ms_per_step"], 5),
        "kernel_us": {k: round(v, 2) for k, v in r["kernel_us"].items()},
        "layer_hbm_frac": round(r["layer_hbm_frac"], 4),
        "roofline": r["roofline"],
        "prefill": prefill,
        "verifier_widths": main_res.get("widths"),
        "dense_fp8": dense,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
