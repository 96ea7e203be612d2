"""The device SwiGLU (the GEMM1 epilogue's fp32 chain in moe_device.h) against the oracle's.

The page's expert computes h = rw * silu(g) * u in fp32 with a full-precision exp ("Native 1017 DSpark draft on the NVLink pair (N1-NATIVE)",
section 4 "Kernel contract", math per (t, j)). The oracle evaluates that chain with a correctly rounded
exp and IEEE division. The device evaluates exp as 2^(x log2 e) on the hardware base-2 exponential with a
two-part log2 e, and the division as a hardware reciprocal plus one FMA correction. This test runs the
device function itself, through a test-only probe library, on every bf16 g in [-100, 10] crossed with a
grid of u and route weights, and bounds how far it moves h from the oracle's:

* in fp32 ulps of the oracle's h wherever |h| >= 2^-32;
* below that, both must stay below 2^-32: the QDQ of h that follows uses a scale of at least 2^-22 (the
  1e-4 amax floor over 448) and E4M3's smallest step is 2^-9 of the scale, so every |h| < 2^-32 becomes code
  0 whatever its exact value. (For g below about -87.3 the hardware reciprocal of 1 + e^-g >= 2^126 is
  flushed to zero, so the device gives h = 0 where the exact chain gives |h| < 2^-120.)
* as the fraction of elements whose bf16(h) differs from the oracle's bf16(h).
"""
import ctypes
import os

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import moe as O

pytestmark = pytest.mark.gpu

PROBE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libswiglu_probe.so")

# Bars. The device exp is within about 1 fp32 ulp of e^x and the corrected quotient within 1 ulp of g / d;
# the two multiplies that follow are correctly rounded on both sides. So h stays within a few ulp of the
# oracle's, and bf16(h) can only move where h lies within those ulp of a bf16 rounding boundary: about
# 2 * 4 / 2^16 (1.2e-4) of uniformly placed values.
MAX_ULP = 4
MAX_BF16_MISMATCH = 1e-3
# below this magnitude h always becomes E4M3 code 0 in the QDQ that follows (see the module docstring)
QDQ_ZERO = 2.0 ** -32


def _bf16_grid(lo: float, hi: float) -> np.ndarray:
    """Every bf16 value in [lo, hi] as fp32."""
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    v = (bits << 16).view(np.float32)
    v = v[np.isfinite(v)]
    v = np.unique(v[(v >= lo) & (v <= hi)])
    return v.astype(np.float32)


def _probe(g, u, rw):
    lib = ctypes.CDLL(PROBE)
    lib.swiglu_probe.restype = ctypes.c_int
    lib.swiglu_probe.argtypes = [ctypes.c_int] + [ctypes.c_void_p] * 5
    dg, du, dr = (torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda() for a in (g, u, rw))
    h = torch.empty_like(dg)
    st = torch.cuda.current_stream().cuda_stream
    rc = lib.swiglu_probe(int(g.size), dg.data_ptr(), du.data_ptr(), dr.data_ptr(), h.data_ptr(), st)
    assert rc == 0, rc
    torch.cuda.synchronize()
    return h.cpu().numpy()


def test_device_swiglu_against_oracle():
    g = _bf16_grid(-100.0, 10.0)
    # u: bf16 values over the clamp range and beyond it; rw: route weights of the workloads' range, and 1
    # (the shared expert, no route weight)
    u = np.concatenate([_bf16_grid(-12.0, 12.0)[::997], np.float32([-10.0, 10.0, 0.0, 1.0, -1.0])]).astype(np.float32)
    rw = np.float32([1.0, 1.5, 0.25, 0.3137, 0.0625, 0.7771, 1.2345, 0.01])
    G, U, R = np.meshgrid(g, u, rw, indexing="ij")
    G, U, R = G.ravel(), U.ravel(), R.ravel()
    h_dev = _probe(G, U, R)
    # the oracle's chain per element: rw is one value per row
    h_ref = O.swiglu_f32(G[:, None].astype(np.float64), U[:, None].astype(np.float64), R)[:, 0]
    assert h_dev.shape == h_ref.shape
    hd, hr = h_dev.astype(np.float64), h_ref.astype(np.float64)
    big = np.abs(hr) >= QDQ_ZERO
    err_ulp = np.abs(hd[big] - hr[big]) / np.spacing(np.abs(h_ref[big])).astype(np.float64)
    mismatch = float(np.mean(F.bf16_rne(hd) != F.bf16_rne(hr)))
    exact = float(np.mean(h_dev == h_ref))
    flushed = G[(h_dev == 0) & (h_ref != 0)]
    print(f"device SwiGLU over {G.size} (g, u, rw): fp32 h identical on {exact:.6f}; max error "
          f"{err_ulp.max():.2f} ulp where |h| >= 2^-32 ({big.sum()} elements); below it, device max |h| "
          f"{np.abs(hd[~big]).max(initial=0.0):.3g}; device zero where the oracle is not for g in "
          f"[{flushed.min(initial=0.0):.4g}, {flushed.max(initial=0.0):.4g}]; bf16(h) differs on {mismatch:.3g} "
          f"of elements")
    assert err_ulp.max() <= MAX_ULP
    assert np.all(np.abs(hd[~big]) < QDQ_ZERO)
    assert mismatch <= MAX_BF16_MISMATCH


def test_device_swiglu_special_cases():
    """g = 0 gives h = 0; g at and above the clamp gives silu(10) * clamp(u); very negative g gives |h| below
    the QDQ's zero threshold with the sign of the exact h (the device evaluates silu at max(g, -80))."""
    g = np.float32([0.0, -0.0, 10.0, 12.0, 1e4, -1e4, -88.0, -89.0, -30.0])
    u = np.float32([3.0, -3.0, 20.0, -20.0, 1.0, 5.0, 1.0, 1.0, 10.0])
    rw = np.float32([1.0] * 9)
    h = _probe(g, u, rw).astype(np.float64)
    ref = O.swiglu_f32(g[:, None].astype(np.float64), u[:, None].astype(np.float64), rw)[:, 0].astype(np.float64)
    assert h[0] == 0 and h[1] == 0
    assert abs(h[5]) < QDQ_ZERO and np.signbit(h[5]) == np.signbit(ref[5])
    big = np.abs(ref) >= QDQ_ZERO
    assert np.all(np.abs(h[big] - ref[big]) <= MAX_ULP * np.spacing(np.abs(ref[big]).astype(np.float32)))
    assert np.all(np.abs(h[~big]) < QDQ_ZERO)
