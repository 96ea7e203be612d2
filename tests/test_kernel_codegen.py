"""Code-generation invariants of the prefill GEMMs' K loops (expert_wide.hip).

The wide GEMMs wait for their LDS-ring copies with one explicit `s_waitcnt vmcnt(8)` per step, before the
step's barrier: 8 is the number of vector-memory operations issued after the copies it needs (the weight
loads of that step). vmcnt counts outstanding operations, which complete in issue order, so the count is right
only if, on every path through a step, exactly the eight weight loads follow its last ring copy. Where the
loads go (a burst after the copies, or spread between the MFMAs) is the compiler's choice, and the K loop
branches (a scale copy of either size by wave, the MFMAs skipped past the last step), so this test builds
the source to gfx950 assembly with the library's flags, splits every K loop (found through the compiler's
loop annotations) into its blocks, and follows every path from one barrier to the next. It also checks that
no register spill or other memory operation sits inside the loops. CPU only: hipcc cross-compiles.
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
# copies (16 bytes per lane into LDS) and 1 scale copy (16 bytes on waves 0-1, 4 bytes on waves 2-3: the two
# forms sit in one-sided branches, so a path may show 0-2 of them; the count is checked as 4-6)
LOAD = re.compile(r"buffer_load_dwordx4 v\[")
COPY = re.compile(r"buffer_load_dword(x4)? v\d+,.*\blds")
LOADS_PER_STEP = 8
FORBIDDEN = re.compile(r"^\s+(scratch_\w+|buffer_store\w*|global_\w+|flat_\w+)\b")


def _assembly(src: str, tmp: str) -> str:
    out = os.path.join(tmp, os.path.basename(src) + ".s")
    flags = [f for f in build.FLAGS if f != "-fPIC"]
    cmd = [build.HIPCC, *flags, "-x", "hip", "--cuda-device-only", "-S", os.path.join(build.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


def _barrier_loops(asm: str):
    """{(function, loop header): [(block name, label line, [instruction lines])]} for every loop whose blocks
    hold an s_barrier, blocks in layout order."""
    loops, func, header, block = {}, None, None, None
    for line in asm.splitlines():
        if re.match(r"^_Z\w+:", line):
            func, header, block = line.split(":")[0], None, None
            continue
        if line.startswith(".Lfunc_end"):
            func, header, block = None, None, None
            continue
        if LABEL.match(line):
            m = HEADER.search(line)
            header = (m.group(1) or m.group(2)) if m else None
            name = line.split(":")[0].strip()
            block = None
            if func is not None and header is not None:
                block = (name, line, [])
                loops.setdefault((func, header), []).append(block)
            continue
        if block is not None and line.startswith("\t") and not line.lstrip().startswith(";"):
            block[2].append(line)
    return {k: v for k, v in loops.items() if any("s_barrier" in l for _, _, ls in v for l in ls)}


def _successors(blocks, i):
    """Indices of the blocks that block i of the loop can go to (-1: out of the loop)."""
    names = {name: j for j, (name, _, _) in enumerate(blocks)}
    out, falls = [], True
    for l in blocks[i][2]:
        t = l.split()
        if t[0].startswith("s_cbranch_") and not t[0].startswith("s_cbranch_join"):
            out.append(names.get(t[-1], -1))
        elif t[0] == "s_branch":
            out.append(names.get(t[-1], -1))
            falls = False
    if falls:
        out.append(i + 1 if i + 1 < len(blocks) else -1)
    return out


def _step_paths(blocks):
    """Every instruction path from an s_barrier of the loop to the next s_barrier (or out of the loop), as
    (lines after the starting barrier, ends at a barrier)."""
    paths = []

    def walk(i, start, acc):
        lines = blocks[i][2][start:]
        for k, l in enumerate(lines):
            if "s_barrier" in l:
                paths.append((acc + lines[:k], True))
                return
        for j in _successors(blocks, i):
            if j < 0:
                paths.append((acc + lines, False))
            else:
                walk(j, 0, acc + lines)

    for i, (_, _, lines) in enumerate(blocks):
        for k, l in enumerate(lines):
            if "s_barrier" in l:
                walk(i, k + 1, [])
    return paths


@pytest.fixture(scope="module")
def wide_loops():
    if not os.path.exists(build.HIPCC):
        pytest.skip("hipcc not found")
    with tempfile.TemporaryDirectory() as tmp:
        loops = _barrier_loops(_assembly("expert_wide.hip", tmp))
    # the K loops: barrier loops that hold the block-scaled MFMAs
    return {k: v for k, v in loops.items()
            if any("v_mfma_scale_f32_16x16x128_f8f6f4" in l for _, _, lines in v for l in lines)}


def test_both_wide_gemms_have_k_loops(wide_loops):
    funcs = {k[0] for k in wide_loops}
    assert any("expert_gemm_wideILb1" in f for f in funcs), funcs   # GEMM1 (w1/w3)
    assert any("expert_gemm_wideILb0" in f for f in funcs), funcs   # GEMM2 (w2)


def _covering_wait(lines, after):
    """(wait value, operations issued since line `after`) of the first s_waitcnt past line `after` whose
    vmcnt lets no operation issued up to line `after` stay in flight, or None."""
    issued = 0
    for l in lines[after + 1:]:
        if re.search(r"\bbuffer_load|\bglobal_load|\bscratch_|\bbuffer_store|\bglobal_store", l):
            issued += 1
        m = re.search(r"s_waitcnt.*vmcnt\((\d+)\)", l)
        if m and int(m.group(1)) <= issued:
            return int(m.group(1)), issued
    return None


def test_k_loops_wait_for_their_copies_exactly(wide_loops):
    # Every barrier-to-barrier path: 4-6 ring copies (the one-sided scale copies), then the weight loads. The
    # branches past the last step test one condition twice (the compiler keeps it in two registers), so the
    # enumeration also walks paths no run takes, with 0 or 16 loads; every path a run takes issues the step's
    # 8 (the source issues them on both sides of that branch), so those are the ones checked: a wait before
    # the barrier covers the last copy on each, and the schedule the kernel is written for is among them (the
    # copies covered first by exactly vmcnt(8); a stricter wait would stall on loads just issued). The path of
    # a step past the end may wait for everything where its register copies merge.
    for (func, header), blocks in wide_loops.items():
        where = f"{func[:60]} loop BB{header}"
        paths = [lines for lines, closed in _step_paths(blocks) if closed]   # (the exit: a full wait follows)
        assert paths, f"{where}: no barrier-to-barrier path"
        full, exact = 0, 0
        for lines in paths:
            copies = [k for k, l in enumerate(lines) if COPY.search(l)]
            loads = [k for k, l in enumerate(lines) if LOAD.search(l)]
            assert 4 <= len(copies) <= 6, f"{where}: {len(copies)} ring copies in a step"
            assert not loads or min(loads) > max(copies), f"{where}: a weight load issued before a ring copy"
            if len(loads) != LOADS_PER_STEP:
                continue
            full += 1
            cover = _covering_wait(lines, max(copies))
            assert cover is not None, f"{where}: no wait before the barrier covers the step's copies"
            exact += cover == (LOADS_PER_STEP, LOADS_PER_STEP)
        assert full, f"{where}: no path with the step's {LOADS_PER_STEP} weight loads"
        assert exact, f"{where}: no path whose copies are covered by exactly vmcnt({LOADS_PER_STEP})"


def test_k_loops_hold_no_spills_or_other_memory_operations(wide_loops):
    for (func, header), blocks in wide_loops.items():
        bad = [l.strip() for _, _, lines in blocks for l in lines if FORBIDDEN.match(l)]
        assert not bad, f"{func[:60]} loop BB{header}: {bad[:4]}"
