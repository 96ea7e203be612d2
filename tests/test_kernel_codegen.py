"""Code-generation invariants of the prefill GEMMs' K loops (expert_wide.hip).

The wide GEMMs wait for their LDS-ring copies with one exact `s_waitcnt vmcnt(N)` per step: N is the number of
vector-memory operations the kernel issues after the copies it needs (the weight loads of the same step).
vmcnt counts outstanding operations, which complete in issue order, so the count is right only if every
load the source issues is in the loop as written: if the compiler dropped or merged one, the wait would let
a needed copy still be in flight. (An added operation, such as a register spill, only makes the wait
stricter; it is checked too because it costs time inside the loop.) This test builds the source to gfx950
assembly with the library's flags and counts, in every K loop (found through the compiler's loop
annotations), the weight loads and ring copies per barrier. CPU only: hipcc cross-compiles.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "mxfp4_routed_expert_moe_amd"))
import build  # noqa: E402  (the library's build script: its hipcc path and flags)

LABEL = re.compile(r"^(\.LBB\d+_\d+:|; %bb\.\d+:)")
HEADER = re.compile(r"Header=BB(\d+_\d+)|^\.LBB(\d+_\d+):.*Loop Header")
# per step of the wide GEMMs, every wave: 8 weight loads (16 bytes per lane into registers), 4 activation
# copies (16 bytes per lane into LDS) and 1 scale copy (16 bytes on waves 0-1, 4 bytes on waves 2-3: both
# forms are in the code, one on each side of a branch)
COUNTS = {
    "weight loads": (re.compile(r"buffer_load_dwordx4 v\["), 8),
    "16-byte ring copies (activations + weight scales)": (re.compile(r"buffer_load_dwordx4 v\d+,.*\blds"), 5),
    "4-byte ring copies (activation scales)": (re.compile(r"buffer_load_dword v\d+,.*\blds"), 1),
}
FORBIDDEN = re.compile(r"^\s+(scratch_\w+|buffer_store\w*|global_\w+|flat_\w+)\b")


def _assembly(src: str, tmp: str) -> str:
    out = os.path.join(tmp, os.path.basename(src) + ".s")
    flags = [f for f in build.FLAGS if f != "-fPIC"]
    cmd = [build.HIPCC, *flags, "-x", "hip", "--cuda-device-only", "-S", os.path.join(build.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


def _barrier_loops(asm: str):
    """{(function, loop header): [instruction lines]} for every loop whose blocks hold an s_barrier."""
    loops, func, header = {}, None, None
    for line in asm.splitlines():
        if re.match(r"^_Z\w+:", line):
            func, header = line.split(":")[0], None
            continue
        if line.startswith(".Lfunc_end"):
            func, header = None, None
            continue
        if LABEL.match(line):
            m = HEADER.search(line)
            header = (m.group(1) or m.group(2)) if m else None
            continue
        if func is not None and header is not None and line.startswith("\t") and not line.lstrip().startswith(";"):
            loops.setdefault((func, header), []).append(line)
    return {k: v for k, v in loops.items() if any("s_barrier" in l for l in v)}


@pytest.fixture(scope="module")
def wide_loops():
    if not os.path.exists(build.HIPCC):
        pytest.skip("hipcc not found")
    with tempfile.TemporaryDirectory() as tmp:
        loops = _barrier_loops(_assembly("expert_wide.hip", tmp))
    # the K loops: barrier loops that hold the block-scaled MFMAs
    return {k: v for k, v in loops.items() if any("v_mfma_scale_f32_16x16x128_f8f6f4" in l for l in v)}


def test_both_wide_gemms_have_k_loops(wide_loops):
    funcs = {k[0] for k in wide_loops}
    assert any("expert_gemm_wideILb1" in f for f in funcs), funcs   # GEMM1 (w1/w3)
    assert any("expert_gemm_wideILb0" in f for f in funcs), funcs   # GEMM2 (w2)


def test_k_loops_issue_exactly_the_counted_loads(wide_loops):
    for (func, header), lines in wide_loops.items():
        steps = sum("s_barrier" in l for l in lines)
        for what, (pat, per_step) in COUNTS.items():
            n = sum(bool(pat.search(l)) for l in lines)
            assert n == per_step * steps, f"{func[:60]} loop BB{header}: {n} {what} for {steps} steps"


def test_k_loops_hold_no_spills_or_other_memory_operations(wide_loops):
    for (func, header), lines in wide_loops.items():
        bad = [l.strip() for l in lines if FORBIDDEN.match(l)]
        assert not bad, f"{func[:60]} loop BB{header}: {bad[:4]}"
