"""Build libmoe.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc.

    python mxfp4_routed_expert_moe_amd/build.py

Objects go to ``_build/`` at the repository root; the shared library is written next to this file.
Also builds the test-only probe libraries under ``tests/csrc`` (never linked into libmoe.so).
Always recompiles (cheap: a few seconds per source).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["route.hip", "permute.hip", "expert_gemm.hip", "expert_mfma.hip", "expert_wide.hip", "expert_bf16.hip",
           "combine.hip",
           "expand.hip", "dense.hip", "moe_abi.cpp"]

# test-only probes: source under tests/csrc -> tests/lib<name>.so
PROBES = ["swiglu_probe"]
# bench-only peak microbenchmarks: csrc/peaks.hip -> libpeaks.so next to libmoe.so
PEAKS = "peaks.hip"
PEAKS_LIB = os.path.join(PKG, "libpeaks.so")
TESTS = os.path.join(ROOT, "tests")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # exact fp32 steps: no contraction into FMAs, IEEE division and square root
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    # keep the compiler from forming packed fp32 ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(os.path.basename(src))[0] + ".o")
    path = src if os.path.isabs(src) else os.path.join(CSRC, src)
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    noise = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l]
    if any(l.strip() for l in noise):
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def _link(objs: list[str], lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    probes = [os.path.join(TESTS, "csrc", p + ".hip") for p in PROBES]
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(_compile, SOURCES + [PEAKS] + probes))
    n = len(SOURCES)
    _link(objs[:n], LIB)
    _link([objs[n]], PEAKS_LIB)
    for name, obj in zip(PROBES, objs[n + 1:]):
        _link([obj], os.path.join(TESTS, f"lib{name}.so"))
    if verbose:
        print(f"built {LIB}, {PEAKS_LIB} and {len(PROBES)} test probe(s)")
    return LIB


if __name__ == "__main__":
    build()
