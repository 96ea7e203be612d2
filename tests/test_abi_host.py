"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every function that
include/moe.h declares, sizes workspaces, and refuses bad arguments before launching anything.

Every call here fails validation (or is an empty M = 0 call), so no kernel is ever launched: the
pointers passed are aligned stand-in addresses that are never dereferenced.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")
LIB = os.path.join(ROOT, "mxfp4_routed_expert_moe_amd", "libmoe.so")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(moe_[a-z_0-9]+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libmoe.so is not built (python mxfp4_routed_expert_moe_amd/build.py)")
    return ctypes.CDLL(LIB)


class Dims(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int32), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("route_scale", ctypes.c_float), ("flags", ctypes.c_uint32)]


class Six(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w1", "s1", "w3", "s3", "w2", "s2")]


class Packed(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w1", "s1", "w3", "s3", "w2", "s2", "stage_scales", "tiled_weights")]


class Three(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w1", "w3", "w2")]


FAKE = 0x10000000  # 256-byte aligned stand-in address, never dereferenced


def big():
    return Dims(128, 5120, 2304, 6, 1.5)


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ("moe_route", "moe_permute", "moe_expert_ffn", "moe_combine", "moe_forward"):
        assert n in names
    assert len(names) >= 10, names


def test_library_exports_every_declared_symbol(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_workspace_bytes(lib):
    f = lib.moe_workspace_bytes
    f.argtypes = [ctypes.POINTER(Dims), ctypes.c_int32]
    f.restype = ctypes.c_size_t
    d = big()
    w8, w64, w8192 = f(ctypes.byref(d), 8), f(ctypes.byref(d), 64), f(ctypes.byref(d), 8192)
    assert 0 < w8 < w64 < w8192
    assert w8 % 256 == 0
    # holds at least the per-slot bf16 outputs and the QDQ'd intermediates
    assert w8192 >= 8192 * 6 * (5120 * 2 + 2304 + 72)
    for bad in (Dims(0, 5120, 2304, 6, 1.5), Dims(128, 5120, 2304, 9, 1.5), Dims(300, 5120, 2304, 6, 1.5),
                Dims(128, 5000, 2304, 6, 1.5), Dims(128, 5120, 2300, 6, 1.5), Dims(4, 256, 128, 6, 1.5),
                Dims(8, 256, 128, 2, float("nan"))):
        assert f(ctypes.byref(bad), 8) == 0
    assert f(ctypes.byref(d), -1) == 0
    assert f(None, 8) == 0


def test_status_strings(lib):
    lib.moe_status_str.restype = ctypes.c_char_p
    assert lib.moe_status_str(OK) == b"MOE_OK"
    assert lib.moe_status_str(INVALID) == b"MOE_ERR_INVALID_ARG"
    assert lib.moe_status_str(UNSUPPORTED) == b"MOE_ERR_UNSUPPORTED"
    assert lib.moe_status_str(WORKSPACE) == b"MOE_ERR_WORKSPACE"
    assert lib.moe_status_str(-4) == b"MOE_ERR_HIP"


def _forward(lib, dims, M, x=FAKE, gw=FAKE, gb=FAKE, packed=True, decoded=False, shared=None, out=FAKE, ws=FAKE,
             ws_bytes=1 << 40, shared_out=None):
    f = lib.moe_forward
    f.restype = ctypes.c_int32
    if isinstance(packed, Packed):
        pk = ctypes.byref(packed)
    else:
        pk = ctypes.byref(Packed(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)) if packed else None
    dc = ctypes.byref(Three(FAKE, FAKE, FAKE)) if decoded else None
    sh = ctypes.byref(shared) if shared is not None else None
    return f(ctypes.byref(dims), ctypes.c_int32(M), ctypes.c_void_p(x), ctypes.c_void_p(gw), ctypes.c_void_p(gb), pk,
             dc, sh, ctypes.c_void_p(out), None, None, ctypes.c_void_p(shared_out), ctypes.c_void_p(ws),
             ctypes.c_size_t(ws_bytes), None)


def test_forward_refuses_before_launch(lib):
    d = big()
    assert _forward(lib, d, 0) == OK                                     # empty call: nothing enqueued
    assert _forward(lib, d, -1) == INVALID
    assert _forward(lib, d, 8, packed=False) == INVALID                  # neither weight set
    assert _forward(lib, d, 8, decoded=True) == INVALID                  # both weight sets
    assert _forward(lib, d, 8, x=0) == INVALID                           # null activation
    assert _forward(lib, d, 8, x=FAKE + 2) == INVALID                    # misaligned activation
    assert _forward(lib, d, 8, out=0) == INVALID
    assert _forward(lib, d, 8, ws=FAKE + 64) == INVALID                  # workspace not 256-byte aligned
    assert _forward(lib, d, 8, ws_bytes=1024) == WORKSPACE               # workspace too small
    assert _forward(lib, d, 8, shared=Six(FAKE, FAKE, FAKE, 0, FAKE, FAKE)) == INVALID   # partial shared set
    assert _forward(lib, d, 8, shared_out=FAKE) == INVALID               # shared_out without a shared expert
    assert _forward(lib, d, 8, packed=Packed(FAKE, FAKE + 4, FAKE, FAKE, FAKE, FAKE, None)) == INVALID   # misaligned scales
    assert _forward(lib, d, 8, packed=Packed(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 8)) == INVALID   # misaligned copy
    assert _forward(lib, d, 8, packed=Packed(0, FAKE, FAKE, FAKE, FAKE, FAKE, None, None)) == INVALID    # no w1 codes
    assert _forward(lib, d, 8, packed=Packed(0, FAKE, 0, FAKE, 0, FAKE, None, FAKE + 8)) == INVALID      # misaligned tiles
    assert _forward(lib, d, 8, packed=Packed(0, 0, 0, FAKE, 0, FAKE, None, FAKE)) == INVALID             # tiles, no s1
    assert _forward(lib, d, 8, shared=Six(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 8)) == INVALID  # misaligned scales
    assert _forward(lib, Dims(128, 5120, 2304, 9, 1.5), 8) == UNSUPPORTED
    assert _forward(lib, Dims(512, 5120, 2304, 6, 1.5), 8) == UNSUPPORTED
    assert _forward(lib, Dims(128, 5056, 2304, 6, 1.5), 8) == UNSUPPORTED
    assert _forward(lib, Dims(128, 5120, 2304, 6, 1.5), 1 << 25) == UNSUPPORTED
    assert _forward(lib, Dims(128, 5120, 2304, 0, 1.5), 8) == INVALID


def test_forward_noalloc_refuses_before_launch(lib):
    """moe_forward_noalloc validates like moe_forward and refuses a batch whose workspace exceeds its
    library-owned array (MOE_NOALLOC_SCRATCH_BYTES), all before touching the device."""
    f = lib.moe_forward_noalloc
    f.restype = ctypes.c_int32
    lib.moe_workspace_bytes.argtypes = [ctypes.POINTER(Dims), ctypes.c_int32]
    lib.moe_workspace_bytes.restype = ctypes.c_size_t
    d = big()

    def call(M, x=FAKE, out=FAKE, packed=True, decoded=False):
        pk = ctypes.byref(Packed(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)) if packed else None
        dc = ctypes.byref(Three(FAKE, FAKE, FAKE)) if decoded else None
        return f(ctypes.byref(d), ctypes.c_int32(M), ctypes.c_void_p(x), ctypes.c_void_p(FAKE),
                 ctypes.c_void_p(FAKE), pk, dc, None, ctypes.c_void_p(out), None, None, None, None)

    assert call(0) == OK
    assert call(-1) == INVALID
    assert call(8, x=0) == INVALID
    assert call(8, out=FAKE + 2) == INVALID
    assert call(8, packed=False) == INVALID
    assert call(8, decoded=True) == INVALID
    assert lib.moe_workspace_bytes(ctypes.byref(d), 64) <= 16 << 20 < lib.moe_workspace_bytes(ctypes.byref(d), 256)
    assert call(256) == WORKSPACE


def test_component_calls_refuse_before_launch(lib):
    d = big()
    r = lib.moe_route(ctypes.byref(d), 8, None, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
                      ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
                      ctypes.c_size_t(1 << 40), None)
    assert r == INVALID
    r = lib.moe_permute(ctypes.byref(d), 8, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), None, ctypes.c_void_p(FAKE),
                        None, ctypes.c_void_p(FAKE), None)
    assert r == INVALID
    r = lib.moe_combine(ctypes.byref(d), 8, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE + 8), None,
                        ctypes.c_void_p(FAKE), None)
    assert r == INVALID
    r = lib.moe_combine(ctypes.byref(d), 0, None, None, None, None, None)
    assert r == OK
    lib.moe_expand_mxfp4.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p]
    assert lib.moe_expand_mxfp4(16, 48, FAKE, FAKE, FAKE, None) == UNSUPPORTED
    assert lib.moe_expand_mxfp4(-1, 64, FAKE, FAKE, FAKE, None) == INVALID
    assert lib.moe_expand_mxfp4(0, 64, FAKE, FAKE, FAKE, None) == OK


def test_workspace_never_shrinks_as_m_grows(lib):
    """A workspace sized for max_tokens must serve every call with M <= max_tokens."""
    f = lib.moe_workspace_bytes
    f.argtypes = [ctypes.POINTER(Dims), ctypes.c_int32]
    f.restype = ctypes.c_size_t
    for d in (big(), Dims(8, 256, 128, 2, 1.5), Dims(256, 1024, 512, 8, 1.0)):
        prev = 0
        for M in list(range(0, 300)) + [1000, 4096, 8192, 8193]:
            w = f(ctypes.byref(d), M)
            assert w >= prev, (M, w, prev)
            prev = w


def test_stage_scales_size_and_refusals(lib):
    f = lib.moe_mxfp4_stage_scales_bytes
    f.argtypes = [ctypes.POINTER(Dims)]
    f.restype = ctypes.c_size_t
    assert f(ctypes.byref(big())) == 3 * 128 * 2304 * 5120 // 32
    assert f(ctypes.byref(Dims(128, 5000, 2304, 6, 1.5))) == 0
    prep = lib.moe_prepare_mxfp4_scales
    prep.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Packed), ctypes.c_void_p, ctypes.c_void_p]
    prep.restype = ctypes.c_int32
    ok = Packed(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert prep(ctypes.byref(big()), None, FAKE, None) == INVALID
    assert prep(ctypes.byref(big()), ctypes.byref(ok), FAKE + 4, None) == INVALID
    assert prep(ctypes.byref(big()), ctypes.byref(Packed(FAKE, 0, FAKE, FAKE, FAKE, FAKE, None)), FAKE, None) == INVALID
    assert prep(ctypes.byref(Dims(128, 5056, 2304, 6, 1.5)), ctypes.byref(ok), FAKE, None) == UNSUPPORTED


def test_prepare_tiled_weights_refuses_before_launch(lib):
    size = lib.moe_mxfp4_tiled_weights_bytes
    size.argtypes = [ctypes.POINTER(Dims)]
    size.restype = ctypes.c_size_t
    d = big()
    assert size(ctypes.byref(d)) == 3 * 128 * 2304 * 5120 // 2     # the three code matrices, same bytes
    assert size(ctypes.byref(Dims(128, 5000, 2304, 6, 1.5))) == 0
    f = lib.moe_prepare_mxfp4_weights
    f.restype = ctypes.c_int32
    f.argtypes = [ctypes.POINTER(Dims), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    w1, w3, w2 = FAKE, FAKE + (1 << 32), FAKE + (2 << 32)
    ok = Packed(w1, FAKE, w3, FAKE, w2, FAKE, None, None)
    assert f(ctypes.byref(d), ctypes.byref(ok), ctypes.c_void_p(FAKE + 8), None) == INVALID    # misaligned out
    assert f(ctypes.byref(d), ctypes.byref(ok), ctypes.c_void_p(w3 + 4096), None) == INVALID   # overlaps w3
    assert f(ctypes.byref(d), None, ctypes.c_void_p(FAKE + (3 << 32)), None) == INVALID
    assert f(ctypes.byref(d), ctypes.byref(Packed(w1, FAKE, 0, FAKE, w2, FAKE, None, None)),
             ctypes.c_void_p(FAKE + (3 << 32)), None) == INVALID                               # no w3
    assert f(ctypes.byref(Dims(128, 5120, 2300, 6, 1.5)), ctypes.byref(ok), ctypes.c_void_p(FAKE + (3 << 32)),
             None) == UNSUPPORTED


def test_dense_fp8_tiled_calls_refuse_before_launch(lib):
    size = lib.moe_fp8_tiled_weights_bytes
    size.argtypes = [ctypes.c_int32, ctypes.c_int32]
    size.restype = ctypes.c_size_t
    assert size(5120, 15360) == 5120 * 15360                     # same bytes, another order
    assert size(100, 128) == 0 and size(128, 100) == 0 and size(0, 128) == 0
    prep = lib.moe_prepare_fp8_weights
    prep.restype = ctypes.c_int32
    prep.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    w, out = FAKE, FAKE + (1 << 32)
    assert prep(1280, 5120, None, out, None) == INVALID
    assert prep(1280, 5120, w, None, None) == INVALID
    assert prep(1280, 5120, w + 8, out, None) == INVALID           # misaligned
    assert prep(1280, 5120, w, w + 1280 * 5120 - 16, None) == INVALID   # out overlaps w
    assert prep(1280, 5000, w, out, None) == UNSUPPORTED
    lin = lib.moe_fp8_linear_tiled
    lin.restype = ctypes.c_int32
    lin.argtypes = [ctypes.c_int32] * 3 + [ctypes.c_void_p] * 6 + [ctypes.c_size_t, ctypes.c_void_p]
    x, s, y, ws = FAKE, FAKE + (2 << 32), FAKE + (3 << 32), FAKE + (4 << 32)
    assert lin(65, 1280, 5120, x, w, s, y, None, ws, 1 << 30, None) == UNSUPPORTED   # decode widths only
    assert lin(8, 1280, 5120, x, w, s, y, y, ws, 1 << 30, None) == INVALID           # both outputs
    assert lin(8, 1280, 5120, x, w, s, y, None, ws, 16, None) == WORKSPACE
    assert lin(0, 1280, 5120, x, w, s, y, None, ws, 0, None) == OK                   # empty batch: nothing to do


def test_dense_plan_fits_lds_over_admitted_shapes(tmp_path):
    """The decode-width dense linear's launch plan (csrc/dense_plan.h), built with the host compiler and run
    over every admitted M <= 64 shape: dynamic LDS within the budget and every K step in exactly one run.
    N = 65536 with K = 5120 at M = 64 was the shape where the block-count rule alone asked for 338 KB."""
    import shutil
    import subprocess
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = tmp_path / "dense_plan_check"
    src = os.path.join(ROOT, "tests", "csrc", "dense_plan_check.cpp")
    inc = os.path.join(ROOT, "mxfp4_routed_expert_moe_amd", "csrc")
    subprocess.run([cxx, "-O2", "-std=c++17", "-I", inc, src, "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    print(r.stdout.strip())


def test_dense_workspace_holds_partials_of_split_plans(lib):
    """Where the LDS cap splits K although N alone fills the chip, the workspace grows by the fp32 partials."""
    lib.moe_fp8_linear_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_fp8_linear_workspace_bytes.argtypes = [ctypes.c_int32] * 3
    M, N, K = 64, 65536, 5120
    ws = lib.moe_fp8_linear_workspace_bytes(M, N, K)
    # 48 KB / (64 * 132 + 8) = 5 steps per run -> 8 runs of the 40 steps
    assert ws >= 8 * M * N * 4 + M * K + M * K // 32


def test_binding_constants_match_the_header():
    """The Python binding's copies of the header's constants."""
    import mxfp4_routed_expert_moe_amd as m
    text = open(HEADER).read()
    scratch = re.search(r"#define MOE_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    flag = re.search(r"#define MOE_FLAG_BATCH_INVARIANT (\d+)u", text)
    assert flag and m.FLAG_BATCH_INVARIANT == int(flag.group(1))
    tiled = re.search(r"#define MOE_TILED_ROWS_PER_EXPERT (\d+)", text)
    assert scratch and tiled
    assert m.NOALLOC_SCRATCH_BYTES == int(scratch.group(1)) << int(scratch.group(2))
    assert m.TILED_ROWS_PER_EXPERT == int(tiled.group(1))


def test_unknown_dims_flags_are_refused(lib):
    lib.moe_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_workspace_bytes.argtypes = [ctypes.POINTER(Dims), ctypes.c_int32]
    ok = Dims(128, 5120, 2304, 6, 1.5, 1)   # MOE_FLAG_BATCH_INVARIANT
    assert lib.moe_workspace_bytes(ctypes.byref(ok), 8192) > 0
    for flags in (2, 4, 0x80000000, 3):
        assert lib.moe_workspace_bytes(ctypes.byref(Dims(128, 5120, 2304, 6, 1.5, flags)), 64) == 0
        assert _forward(lib, Dims(128, 5120, 2304, 6, 1.5, flags), 8) == INVALID
