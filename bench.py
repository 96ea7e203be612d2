"""Throughput of the routed-MoE FFN layer (MXFP4 experts) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode_m8] [--replicas R]
                    [--no-prefill] [--no-cpu-baseline]

A step is one call of ``moe_forward`` (router + activation QDQ, permutation, grouped w1/w3 GEMM with
SwiGLU and QDQ of h, grouped w2 GEMM, fixed-order combine) over one batch of seeded synthetic tokens.
Inputs are resident in HBM before the timed region starts. The expert weights exist in R replicas and
step i uses replica i mod R, so the 256 MB last-level cache cannot serve them from a previous step.

Printed: one JSON line. ``value`` is tokens/s of the M=8 decode-width layer (hidden 5120, 128 MXFP4
experts, intermediate 2304, top-6) over the K timed steps. Without --warmup the timed steps follow 10 untimed
ones and then 0.5 s more of untimed steps, so that the GPU's clocks have left their idle state (``warmup``
reports all untimed steps). ``step_us`` holds the median, p10 and p90 of 200 per-step HIP-event samples taken
after another 0.5 s of the layer running, ``telemetry`` the GPU clock, power and temperature polled
meanwhile. ``roofline`` describes the dominant kernel, the grouped w1/w3 GEMM.
``prefill`` (8192 tokens), ``batched_decode_m64`` and ``prefill_shared_skew_m2048`` (2048 tokens with the FP8
shared expert and 8 hot experts) hold the same figures for the other workloads, each with its layer's
fractions of the HBM and MFMA peaks. ``peaks`` are this GPU's measured streaming-read and scaled-MFMA
rates. ``cpu_baseline`` is the CPU oracle timed on bounded samples on this host's cores (all, and one).
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
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published

WORKLOADS = {"tiny_m4": 0, "decode_m8": 1, "batched_decode_m64": 2, "prefill_m8192": 3,
             "prefill_shared_skew_m2048": 4}

# L2<->memory bytes of the w1/w3 GEMM per launch, from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE runs (KiB per
# dispatch). A 1 GiB device copy reads FETCH_SIZE = 524300 KiB and WRITE_SIZE = 1048576 KiB on this GPU, so the
# fetch counter is scaled by 2.0 and the write counter by 1.0. The figures hold only for the kernel source they
# were measured on (sha256 prefix); after any change to it the traffic is reported as null until re-measured.
FETCH_SCALE, WRITE_SCALE = 1048576 / 524300.9, 1.0
MEASURED_TRAFFIC = {
    "decode_m8": dict(src="expert_gemm.hip", sha="9d186bd42894c2f5", fetch_kib=227911.2, write_kib=135.1),
    "prefill_m8192": dict(src="expert_wide.hip", sha="e3b50cc018fcb773", fetch_kib=1492984.0, write_kib=114324.0),
}


# The fixed fp32 summation orders of the path (recorded so that routing and outputs are reproducible; the tie
# flags of each run are in cpu_baseline.routing_ties).
FP32_ORDERS = {
    "router_logits": "M <= 64: per 512-wide chunk of H, 64 lanes x an 8-FMA chain then a butterfly over the lanes, "
                     "chunks added in ascending order; M > 64 (and the batch-invariant flag): bf16 matrix cores over "
                     "each quarter of H, three exact split-gate products per 32-wide step in ascending order, quarters "
                     "added in ascending order",
    "route_weights": "rw_j = (s_j / ((((s_0 + s_1) + ...) + s_{k-1}) + 1e-20)) * route_scale in fp32, slots in "
                     "descending selection order, IEEE division",
    "expert_dot_products": "each 128-wide K step's exact block products summed inside one block-scaled MFMA, the steps "
                           "accumulated in fp32 in ascending order",
    "combine": "acc = 0; acc += float(slot) over the token's experts in ascending expert id; then + float(shared); "
               "out = bf16(acc)",
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


class Telemetry:
    """Clock, power and temperature of the GPU, polled from amdsmi in a background thread while the layer
    runs back to back (null fields where the library or a reading is unavailable)."""

    def __init__(self, period_s: float = 0.01):
        import threading

        self.samples = []
        self.period = period_s
        self._stop = threading.Event()
        self._thread = None
        self.handle = None
        try:
            import amdsmi
            import torch

            amdsmi.amdsmi_init()
            self.amdsmi = amdsmi
            props = torch.cuda.get_device_properties(torch.cuda.current_device())
            want = (props.pci_domain_id, props.pci_bus_id, props.pci_device_id)
            for h in amdsmi.amdsmi_get_processor_handles():
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)   # "dddd:bb:dd.f"
                dom, bus, rest = bdf.split(":")
                if (int(dom, 16), int(bus, 16), int(rest.split(".")[0], 16)) == want:
                    self.handle = h
                    break
        except Exception:   # amdsmi missing or not permitted: telemetry is reported as unavailable
            self.handle = None

    def _read(self):
        m = self.amdsmi.amdsmi_get_gpu_metrics_info(self.handle)
        def num(k):
            v = m.get(k)
            return v if isinstance(v, (int, float)) and v not in (0xFFFF, 0xFFFFFFFF) else None
        gfx = None
        if isinstance(m.get("current_gfxclks"), list):   # one clock per XCD: their mean
            vals = [v for v in m["current_gfxclks"] if isinstance(v, int) and 0 < v < 0xFFFF]
            gfx = sum(vals) / len(vals) if vals else None
        if gfx is None:
            gfx = num("current_gfxclk")
        return dict(gfx_mhz=gfx, avg_gfx_mhz=num("average_gfxclk_frequency"), gfx_activity_pct=num("average_gfx_activity"),
                    mem_mhz=num("current_uclk"), power_w=num("current_socket_power") or num("average_socket_power"),
                    hotspot_c=num("temperature_hotspot"))

    def _run(self):
        while not self._stop.is_set():
            try:
                self.samples.append(self._read())
            except Exception:
                return
            self._stop.wait(self.period)

    def __enter__(self):
        import threading
        if self.handle is not None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()

    def summary(self):
        if not self.samples:
            return None
        out = dict(samples=len(self.samples), period_ms=self.period * 1e3, source="amdsmi gpu metrics")
        for k in ("gfx_mhz", "avg_gfx_mhz", "gfx_activity_pct", "mem_mhz", "power_w", "hotspot_c"):
            v = sorted(x[k] for x in self.samples if x.get(k) is not None)
            out[k] = None if not v else dict(min=v[0], median=v[len(v) // 2], max=v[-1])
        return out


def _percentiles(us):
    import numpy as np
    a = np.asarray(us, dtype=np.float64)
    return dict(samples=int(a.size), median=round(float(np.median(a)), 2), p10=round(float(np.percentile(a, 10)), 2),
                p90=round(float(np.percentile(a, 90)), 2), min=round(float(a.min()), 2))


def settle(L: "Layer", seconds: float, first: int = 0) -> int:
    """Runs the layer back to back for at least `seconds` of wall time (untimed) and returns the steps run.
    From idle the GPU's clocks take a few hundred milliseconds of load to reach their sustained state (the SMU
    reports idle clocks when the load starts); measured on the decode layer, 100-step loops started from
    idle run about 2 % slower than after 0.4 s of load."""
    import torch
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(16):
            L.step(first + n)
            n += 1
        torch.cuda.synchronize()
    return n


def sample_steps(L: "Layer", n: int = 200, settle_s: float = 0.5) -> dict:
    """After a 0.5 s settle (the layer running back to back), n steps each bracketed by its own pair of HIP
    events on the launch stream (the weight replicas keep rotating): per-step microseconds as median, p10,
    p90."""
    import torch
    settle(L, settle_s)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i, (a, b) in enumerate(evs):
        a.record()
        L.step(i)
        b.record()
    torch.cuda.synchronize()
    return _percentiles([a.elapsed_time(b) * 1e3 for a, b in evs])


def measure(cid: int, steps: int, warmup: int, replicas: int, widths=None, tiled: bool = True,
            samples: int = 200, settle_s: float = 0.5) -> dict:
    """One workload: the timed K-step loop (whole-job rate), 200 event samples, graph replay, the split
    entry points' kernel times, GEMM1 back to back (roofline timing) and clock / power telemetry. The timed
    loop follows `warmup` untimed steps and then, with settle_s > 0, settle_s seconds more of untimed steps
    (the number of all untimed steps is returned as warmup_steps)."""
    import torch

    L = Layer(cid, replicas, tiled)
    cfg = L.cfg
    tel = Telemetry()
    if True:
        for i in range(warmup):
            L.step(i)
        torch.cuda.synchronize()
        warmup_steps = warmup + (settle(L, settle_s, warmup) if settle_s > 0 else 0)
        t0 = time.perf_counter()
        for i in range(steps):
            L.step(warmup_steps + i)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ms = (t1 - t0) * 1e3 / steps
        D = L.distinct_experts()
        ids_host = L.ids.cpu()
        samp = sample_steps(L, samples)

        # kernel-level times: events between the split entry points, on the stream they launch on
        names = ["route", "permute", "gemm1", "gemm2", "shared", "combine"]
        tot = [0.0] * len(names)
        n_k = max(min(steps, 50), 5)
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
        # clock, power and temperature while the layer runs back to back (graph replays for about 0.4 s)
        with tel:
            t_end = time.perf_counter() + 0.4
            while time.perf_counter() < t_end:
                graph.replay()
                torch.cuda.synchronize()
        del graph

    w13_b, w2_b = _bytes_per_expert(cfg)
    f13, f2 = _flops_per_pair(cfg)
    P = cfg.M * cfg.k
    gemm1_bytes = D * w13_b + cfg.M * (cfg.H + cfg.H // 32) + P * (cfg.I + cfg.I // 32)
    gemm1_flops = P * f13
    # the layer's algorithmic work: the touched experts' packed bytes (+ the fp32 gate, + the FP8 shared
    # expert's bytes), and the flops of every (token, expert) assignment (+ the shared expert on every token)
    layer_bytes = D * (w13_b + w2_b) + cfg.E * cfg.H * 4
    layer_flops = P * (f13 + f2)
    if cfg.shared:
        layer_bytes += 3 * cfg.I * cfg.H + 3 * (cfg.I // 32) * (cfg.H // 32)
        layer_flops += cfg.M * (f13 + f2)
    sec = ms * 1e-3
    res = dict(workload=cfg.name, M=cfg.M, ms_per_step=ms, tokens_per_s=cfg.M / sec, distinct_experts=D,
               warmup_steps=warmup_steps, settle_s=settle_s,
               graph_ms_per_step=graph_ms, step_us=samp, kernel_us=kern_us,
               layer_algorithmic_bytes=layer_bytes, layer_algorithmic_flops=layer_flops,
               layer_hbm_frac=(layer_bytes / sec) / (HBM_PEAK_GBS * 1e9),
               layer_mfma_frac=(layer_flops / sec) / (MFMA_FP8_PEAK_TFLOPS * 1e12),
               layer_tflops=layer_flops / sec / 1e12, replicas=replicas, weight_layout=L.weight_layout,
               inputs_sha256=L.digest, telemetry=tel.summary(), ids=ids_host)
    g1 = gemm1_us * 1e-6
    timing = dict(avg_us_timing=f"HIP events around {n_b} back-to-back launches on the launch stream",
                  avg_us_per_call_events=round(kern_us["gemm1"], 2))
    if cfg.M * cfg.k < 32 * cfg.E:   # decode width: the weight stream bounds GEMM1
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
        res["batch_invariant"] = measure_flagged(L, steps, warmup)
    del L
    torch.cuda.empty_cache()
    return res


def measure_decoded(cid: int, steps: int, warmup: int, packed_ms=None) -> dict:
    """The decoded-BF16 arm on one workload: the routed experts expanded once to bf16 (moe_expand_mxfp4) and
    the layer run on them (routed only, no shared expert), K timed steps after W warm-up steps, and GEMM1 /
    GEMM2 alone through the split entry points with HIP events, against the bf16 MFMA peak."""
    import numpy as np
    import torch

    import mxfp4_routed_expert_moe_amd as moe
    import synth

    cfg = synth.get_config(cid)
    inp = synth.make_inputs(cfg)
    E, H, I, k, M = cfg.E, cfg.H, cfg.I, cfg.k, cfg.M

    def up(a):
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    x, gw, gb = up(inp["x"]), up(inp["gate_w"]), up(inp["gate_b"])
    dims = moe.Dims(E, H, I, k, cfg.route_scale)
    dec = moe.BF16Experts(*(torch.empty(s, dtype=torch.int16, device="cuda") for s in [(E, I, H), (E, I, H), (E, H, I)]))
    for n, sn, dst in (("w1", "s1", dec.w1), ("w3", "s3", dec.w3), ("w2", "s2", dec.w2)):
        w, sc = up(inp[n]), up(inp[sn])
        moe.moe_expand_mxfp4(w, sc, dst)
        torch.cuda.synchronize()
        del w, sc
    del inp
    torch.cuda.empty_cache()
    dev = dict(device="cuda")
    ws = moe.workspace(dims, M)
    out = torch.empty((M, H), dtype=torch.int16, **dev)
    ids = torch.empty((M, k), dtype=torch.int32, **dev)
    rw = torch.empty((M, k), dtype=torch.float32, **dev)
    xq = torch.empty((M, H), dtype=torch.uint8, **dev)
    xs = torch.empty((M, H // 32), dtype=torch.uint8, **dev)
    counts = torch.empty(E, dtype=torch.int32, **dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, **dev)
    pairs = torch.empty(M * k, dtype=torch.int32, **dev)
    active = torch.empty(E, dtype=torch.int32, **dev)
    hq = torch.empty((M * k, I), dtype=torch.uint8, **dev)
    hs = torch.empty((M * k, I // 32), dtype=torch.uint8, **dev)
    slot = torch.empty((M * k, H), dtype=torch.int16, **dev)

    def layer():
        moe.moe_forward(dims, x, gw, gb, None, dec, None, out, ids, rw, None, ws)

    for _ in range(warmup):
        layer()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        layer()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    moe.moe_route(dims, x, gw, gb, ids, rw, xq, xs, ws)
    moe.moe_permute(dims, ids, counts, offsets, pairs, None, active)

    def timed(f, n):
        f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            f()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    n = max(3, steps // 2)
    g1_us = timed(lambda: moe.moe_expert_gemm1(dims, xq, xs, None, dec, rw, offsets, pairs, active, hq, hs, ws), n)
    g2_us = timed(lambda: moe.moe_expert_gemm2(dims, M, hq, hs, None, dec, offsets, pairs, active, slot, ws), n)
    f13, f2 = _flops_per_pair(cfg)
    P = M * k
    g1_tf = P * f13 / (g1_us * 1e-6) / 1e12
    res = dict(workload=cfg.name, M=M, arm="decoded-BF16 (expanded weights, bf16 MFMA grouped GEMM)",
               value=round(M / (ms * 1e-3), 1), unit="tokens/s", ms_per_step=round(ms, 5),
               steps=steps, warmup=warmup, decoded_weight_bytes=3 * E * H * I * 2,
               kernel_us=dict(gemm1=round(g1_us, 1), gemm2=round(g2_us, 1)),
               layer_tflops=round(P * (f13 + f2) / (ms * 1e-3) / 1e12, 1),
               roofline=dict(kernel="expert_gemm_bf16 GEMM1 (w1/w3 + SwiGLU + QDQ)", bound="mfma",
                             achieved=round(g1_tf, 1), peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s",
                             frac=round(g1_tf / MFMA_BF16_PEAK_TFLOPS, 4), traffic=None,
                             algorithmic_flops=P * f13, avg_us=round(g1_us, 1),
                             avg_us_timing=f"HIP events around {n} back-to-back launches"),
               note="routed experts only (the workload has no shared expert); same routing as the packed arm")
    if packed_ms:
        res["vs_packed_arm"] = round(packed_ms / ms, 4)
    del dec, ws
    torch.cuda.empty_cache()
    return res


def measure_flagged(L: Layer, steps: int, warmup: int) -> dict:
    """The same layer with MOE_FLAG_BATCH_INVARIANT (one router summation order at every M): eager loop over the
    weight replicas, against the default's loop timed the same way right before it."""
    import dataclasses

    import torch

    flagged = dataclasses.replace(L.dims, flags=L.moe.FLAG_BATCH_INVARIANT)

    def loop(dims):
        for i in range(warmup):
            L.moe.moe_forward(dims, L.x, L.gate_w, L.gate_b, L.experts[i % len(L.experts)], None, L.shared, L.out,
                              L.ids, L.rw, None, L.ws)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            L.moe.moe_forward(dims, L.x, L.gate_w, L.gate_b, L.experts[i % len(L.experts)], None, L.shared, L.out,
                              L.ids, L.rw, None, L.ws)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e6 / steps

    default_us = loop(L.dims)
    flagged_us = loop(flagged)
    return dict(us=round(flagged_us, 2), default_us=round(default_us, 2),
                note="router on the matrix-core kernel at every M, selection and permutation as separate kernels")


def leg(r: dict) -> dict:
    """The JSON object of one workload measured by measure() (value = tokens/s of the K-step loop)."""
    return dict(workload=r["workload"], M=r["M"], value=round(r["tokens_per_s"], 1), unit="tokens/s",
                ms_per_step=round(r["ms_per_step"], 5), step_us=r["step_us"],
                graph_ms_per_step=round(r["graph_ms_per_step"], 5), distinct_experts=r["distinct_experts"],
                kernel_us={k: round(v, 2) for k, v in r["kernel_us"].items()},
                layer_hbm_frac=round(r["layer_hbm_frac"], 4), layer_mfma_frac=round(r["layer_mfma_frac"], 4),
                layer_tflops=round(r["layer_tflops"], 1), roofline=r["roofline"], telemetry=r["telemetry"],
                inputs_sha256=r["inputs_sha256"], weight_replicas=r["replicas"], weight_layout=r["weight_layout"],
                warmup_steps=r["warmup_steps"], warmup_settle_s=r["settle_s"])


def measure_peaks() -> dict:
    """This GPU's achievable peaks for the two rooflines (libpeaks.so, built with the library): the best read of
    2 GiB over a sweep of block counts, loads in flight and the non-temporal hint, and dependency-free streams
    of the scaled 16x16x128 MFMA for the three operand-format pairs, on every SIMD (512 blocks of 4 waves)."""
    import ctypes

    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "mxfp4_routed_expert_moe_amd", "libpeaks.so"))
    lib.moe_peak_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_void_p, ctypes.c_void_p]
    lib.moe_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                  ctypes.c_void_p]
    st = torch.cuda.current_stream().cuda_stream
    n = 2 << 30
    buf = torch.empty(n, dtype=torch.uint8, device="cuda")
    buf.random_(0, 256)
    sink = torch.empty(lib.moe_peak_stream_blocks(), dtype=torch.int32, device="cuda")

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3 / reps

    sweep = {}
    for blocks in (1024, 2048, 4096, 8192):
        for unroll in (8, 16):
            for nt in (0, 1):
                t = timed(lambda: lib.moe_peak_stream_read(buf.data_ptr(), n, blocks, unroll, nt, sink.data_ptr(),
                                                           st), 10)
                sweep[f"b{blocks}_u{unroll}_{'nt' if nt else 'plain'}"] = round(n / t / 1e9, 1)
    best = max(sweep, key=sweep.get)
    lib.moe_peak_l2_read.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                     ctypes.c_void_p]
    l2 = {}
    for windows in (16, 32):   # 1 MB and 2 MB of windows: resident in each XCD's 4 MB L2
        for blocks in (1024, 2048):
            reps = 64
            t = timed(lambda: lib.moe_peak_l2_read(buf.data_ptr(), windows, blocks, reps, sink.data_ptr(), st), 5)
            l2[f"w{windows}_b{blocks}"] = round(blocks * 4 * reps * 65536 / t / 1e9, 1)
    out = dict(stream_read=dict(bytes=n, gbs=sweep[best], frac_of_8tbs=round(sweep[best] / 8000, 4), best=best,
                                sweep_gbs=sweep,
                                method="2 GiB read once per call, each wave a contiguous run of 1 KB loads "
                                       "(16-byte loads per lane); blocks x loads in flight x hint swept, "
                                       "the best kept; 10 calls each"),
               l2_read=dict(gbs=max(l2.values()), sweep_gbs=l2,
                            method="each wave re-reads a 64 KB window of a 1 or 2 MB buffer 64 times (L2-resident), "
                                   "1 KB per load instruction, 16 loads in flight"))
    del buf
    blocks, iters = 512, 4096
    fsink = torch.empty(4 * blocks, dtype=torch.float32, device="cuda")
    for name, fa, fb in (("e2m1_x_e4m3", 4, 0), ("e4m3_x_e4m3", 0, 0), ("e2m1_x_e2m1", 4, 4)):
        t = timed(lambda: lib.moe_peak_mfma(fa, fb, blocks, iters, fsink.data_ptr(), st), 5)
        flop = blocks * 4 * iters * 8 * 65536
        out[f"mfma_{name}"] = dict(tflops=round(flop / t / 1e12, 1))
    out["mfma_method"] = "v_mfma_scale_f32_16x16x128_f8f6f4, 8 independent accumulators per wave, 2 waves per SIMD"
    torch.cuda.empty_cache()
    return out


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


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(gpu_ids: dict | None = None) -> dict:
    """The CPU oracle, as it stands, timed on bounded samples on this host:
    - the decode workload's 8 tokens on all cores (the reported value), and 2 of them on one thread;
    - the tiny layer (4 tokens) on all cores and on one thread;
    - 4 tokens of the batched-decode workload on all cores.
    Each run is the whole oracle layer for those tokens: router, QDQ, their experts decoded from MXFP4, fp64
    dot products, SwiGLU, combine. Also reported: the oracle's routing of each measured workload, its
    tie-flagged tokens (selection scores within 1e-6) and whether the GPU's ids differ there."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import synth
    from oracle import moe as O

    pool = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count() or 1])

    inputs = {}

    def run(cid, ntok, threads):
        cfg = synth.get_config(cid)
        if cid not in inputs:
            inputs.clear()
            inputs[cid] = synth.make_inputs(cfg)
        inp = inputs[cid]
        toks = list(range(ntok))
        with threadpool_limits(limits=threads):
            t0 = time.perf_counter()
            O.moe_forward(inp, cfg, tokens=toks)
            dt = time.perf_counter() - t0
        return dict(workload=cfg.name, tokens=ntok, threads=threads, seconds=round(dt, 2),
                    tokens_per_s=round(ntok / dt, 4))

    runs = [run(1, 8, pool), run(1, 2, 1), run(0, 4, pool), run(0, 4, 1), run(2, 4, pool)]
    head = runs[0]
    ties = {}
    for name, ids in (gpu_ids or {}).items():
        cfg = synth.get_config(WORKLOADS[name])
        r = synth.make_router_inputs(cfg)
        ref = O.route(r["x"], r["gate_w"], r["gate_b"], cfg.k, cfg.route_scale)
        flagged = np.nonzero(ref["tie"])[0]
        g = np.asarray(ids)
        ties[name] = dict(flagged_tokens=[int(t) for t in flagged],
                          gpu_ids_differ_at=[int(t) for t in flagged if not np.array_equal(g[t], ref["ids"][t])],
                          untied_tokens_differing=int(np.sum(np.any(g != ref["ids"], axis=1) & ~ref["tie"])))
    return dict(value=head["tokens_per_s"], unit="tokens/s", cores=head["threads"], kind="oracle",
                sample=f"{head['tokens']} tokens of {head['workload']} (router, QDQ, their experts decoded from "
                       f"MXFP4, fp64 dot products, combine); {head['seconds']} s",
                cpu_model=_cpu_model(), host_cpus=os.cpu_count(), runs=runs, routing_ties=ties)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps before the timed ones (default: 10, then the layer keeps running untimed "
                         "until 0.5 s have passed, so that the clocks have left their idle state; an explicit "
                         "value runs exactly that many)")
    ap.add_argument("--workload", default="decode_m8", choices=sorted(WORKLOADS))
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--samples", type=int, default=200,
                    help="per-step HIP event samples after a 0.5 s settle (the layer running back to back)")
    ap.add_argument("--no-prefill", action="store_true", help="skip the 8192-token prefill measurement")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the 64-token and 2048-token (shared expert, skewed routing) workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense FP8 projection family")
    ap.add_argument("--no-widths", action="store_true", help="skip the verifier widths M = 1 .. 32")
    ap.add_argument("--no-peaks", action="store_true", help="skip the HBM-read and MFMA peak microbenchmarks")
    ap.add_argument("--no-decoded", action="store_true",
                    help="skip the decoded-BF16 arm at the 8192-token prefill workload")
    ap.add_argument("--stored-layout", action="store_true",
                    help="stream the weight codes (routed experts and the dense FP8 family) from their stored "
                         "row-major layout instead of the fragment-order copy made at load")
    ap.add_argument("--dense-only", action="store_true",
                    help="only the dense FP8 projection family (prints its object as the JSON line)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy (reference for the rocprof byte counters)")
    args = ap.parse_args()
    settle_s = 0.5 if args.warmup is None else 0.0
    if args.warmup is None:
        args.warmup = 10
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
    tiled = not args.stored_layout
    widths = VERIFIER_WIDTHS if (args.workload == "decode_m8" and not args.no_widths) else None
    main_res = measure(WORKLOADS[args.workload], args.steps, args.warmup, args.replicas, widths, tiled, args.samples,
                       settle_s)
    print(f"# {main_res['workload']}: {main_res['ms_per_step'] * 1e3:.1f} us/step, samples {main_res['step_us']}, "
          f"kernels {main_res['kernel_us']}", file=sys.stderr, flush=True)
    if main_res.get("widths"):
        print("# widths: " + ", ".join(f"M={m}: {v['us']} us ({v['distinct_experts']} experts)"
                                       for m, v in main_res["widths"].items()), file=sys.stderr, flush=True)
    gpu_ids = {main_res["workload"]: main_res.pop("ids").numpy()}
    others = {}
    plan = []
    if not args.no_others:
        plan.append(("batched_decode_m64", max(10, args.steps // 2), max(2, args.warmup // 2), args.replicas))
    if not args.no_prefill:
        plan.append(("prefill_m8192", max(20, args.steps // 5), max(4, args.warmup // 2), args.replicas))
    if not args.no_others:
        plan.append(("prefill_shared_skew_m2048", max(20, args.steps // 5), max(4, args.warmup // 2), args.replicas))
    for name, st, wu, rep in plan:
        if name == args.workload:
            continue
        r = measure(WORKLOADS[name], st, wu, rep, tiled=tiled, samples=args.samples, settle_s=settle_s)
        gpu_ids[name] = r.pop("ids").numpy()
        others[name] = leg(r)
        print(f"# {name}: {r['ms_per_step'] * 1e3:.1f} us/step, samples {r['step_us']}, kernels "
              f"{ {k: round(v, 1) for k, v in r['kernel_us'].items()} }", file=sys.stderr, flush=True)
    decoded = None
    if not args.no_decoded and not args.no_prefill:
        pre = others.get("prefill_m8192")
        decoded = measure_decoded(WORKLOADS["prefill_m8192"], max(10, args.steps // 10), max(2, args.warmup // 5),
                                  pre["ms_per_step"] if pre else None)
        print(f"# decoded-BF16 arm, prefill_m8192: {decoded['ms_per_step']:.3f} ms/step, kernels "
              f"{decoded['kernel_us']}", file=sys.stderr, flush=True)
    dense = None
    if not args.no_dense:
        dense = measure_dense(tiled=tiled)
        summary = ", ".join(f"{k}: {v['us']} us" for k, v in dense["shapes"].items())
        print(f"# dense: {summary}", file=sys.stderr, flush=True)
    peaks = None
    if not args.no_peaks:
        peaks = measure_peaks()
        print(f"# peaks: {peaks}", file=sys.stderr, flush=True)
        for o in [main_res] + list(others.values()):
            rf = o["roofline"]
            if rf["bound"] == "hbm":
                rf["measured_peak"] = peaks["stream_read"]["gbs"]
            else:
                rf["measured_peak"] = peaks["mfma_e2m1_x_e4m3"]["tflops"]
            rf["frac_of_measured_peak"] = round(rf["achieved"] / rf["measured_peak"], 4)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(gpu_ids)
    r = main_res
    line = {
        "metric": "MoE-layer tokens/s at M=8 and M=8192; % of HBM BW / MXFP4 MFMA roofline",
        "value": round(r["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": main_res["warmup_steps"],
        "warmup_settle_s": settle_s,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 x mxfp4 (fp32 accumulate, bf16 out)",
        "data": "synthetic (seeded)",
        "config": {"workload": r["workload"], "M": r["M"], "hidden": 5120, "experts": 128, "inter": 2304,
                   "top_k": 6, "distinct_experts": r["distinct_experts"], "weight_replicas": r["replicas"],
                   "weight_layout": r["weight_layout"], "parallelism": "none (1 GPU)"},
        "step_us": r["step_us"],
        "graph_ms_per_step": round(r["graph_ms_per_step"], 5),
        "kernel_us": {k: round(v, 2) for k, v in r["kernel_us"].items()},
        "layer_hbm_frac": round(r["layer_hbm_frac"], 4),
        "layer_algorithmic_bytes": r["layer_algorithmic_bytes"],
        "roofline": r["roofline"],
        "telemetry": r["telemetry"],
        "inputs_sha256": r["inputs_sha256"],
        "fp32_orders": FP32_ORDERS,
        "prefill": others.get("prefill_m8192"),
        "batched_decode_m64": others.get("batched_decode_m64"),
        "prefill_shared_skew_m2048": others.get("prefill_shared_skew_m2048"),
        "decoded_bf16_prefill_m8192": decoded,
        "verifier_widths": r.get("widths"),
        "decode_m8_batch_invariant": r.get("batch_invariant"),
        "dense_fp8": dense,
        "peaks": peaks,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
