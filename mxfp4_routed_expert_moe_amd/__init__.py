"""Python binding of libmoe, the MI355X (gfx950) routed-MoE FFN layer library.

Argument marshalling only: every step of the layer runs in the library's HIP kernels. PyTorch
supplies device memory and streams; tensors are passed as raw device pointers to the C ABI declared
in ``include/moe.h`` (same function names, same argument order).

The library must be built (``python mxfp4_routed_expert_moe_amd/build.py``); importing this package
without it raises: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

__all__ = [
    "LIB_PATH", "MoeError", "Dims", "MXFP4Experts", "BF16Experts", "FP8Expert", "lib",
    "moe_workspace_bytes", "moe_status_str", "moe_route", "moe_permute", "moe_expert_ffn",
    "moe_expert_gemm1", "moe_expert_gemm2", "moe_shared_expert", "moe_combine", "moe_forward", "moe_expand_mxfp4", "workspace",
    "moe_mxfp4_stage_scales_bytes", "moe_prepare_mxfp4_scales", "moe_expert_ffn_f32", "moe_shared_expert_f32",
    "moe_combine_sum_f32", "moe_combine_official_f32", "moe_fp8_linear_workspace_bytes", "moe_fp8_linear",
    "moe_mxfp4_tiled_weights_bytes", "moe_prepare_mxfp4_weights", "moe_fp8_tiled_weights_bytes",
    "moe_prepare_fp8_weights", "moe_fp8_linear_tiled", "moe_forward_noalloc", "NOALLOC_SCRATCH_BYTES", "TILED_ROWS_PER_EXPERT", "FLAG_BATCH_INVARIANT",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libmoe.so is not built at {LIB_PATH}; run python mxfp4_routed_expert_moe_amd/build.py")

lib = ctypes.CDLL(LIB_PATH)

MOE_OK = 0


class MoeError(RuntimeError):
    """A libmoe entry point returned a non-zero status."""


class _Dims(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int32), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("route_scale", ctypes.c_float), ("flags", ctypes.c_uint32)]


class _MXFP4(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w1", "s1", "w3", "s3", "w2", "s2", "stage_scales", "tiled_weights")]


class _BF16(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w1", "w3", "w2")]


class _FP8(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w1", "s1", "w3", "s3", "w2", "s2")]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t

lib.moe_workspace_bytes.argtypes = [ctypes.POINTER(_Dims), _I32]
lib.moe_workspace_bytes.restype = _SZ
lib.moe_status_str.argtypes = [_I32]
lib.moe_status_str.restype = ctypes.c_char_p
lib.moe_route.argtypes = [ctypes.POINTER(_Dims), _I32, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]
lib.moe_route.restype = _I32
lib.moe_permute.argtypes = [ctypes.POINTER(_Dims), _I32, _P, _P, _P, _P, _P, _P, _P]
lib.moe_permute.restype = _I32
lib.moe_expert_ffn.argtypes = [ctypes.POINTER(_Dims), _I32, _P, _P, ctypes.POINTER(_MXFP4), ctypes.POINTER(_BF16),
                               _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]
lib.moe_expert_ffn.restype = _I32
lib.moe_expert_gemm1.argtypes = [ctypes.POINTER(_Dims), _I32, _P, _P, ctypes.POINTER(_MXFP4), ctypes.POINTER(_BF16),
                                 _P, _P, _P, _P, _P, _P, _P, _SZ, _P]
lib.moe_expert_gemm1.restype = _I32
lib.moe_expert_gemm2.argtypes = [ctypes.POINTER(_Dims), _I32, _P, _P, ctypes.POINTER(_MXFP4), ctypes.POINTER(_BF16),
                                 _P, _P, _P, _P, _P, _SZ, _P]
lib.moe_expert_gemm2.restype = _I32
lib.moe_shared_expert.argtypes = [ctypes.POINTER(_Dims), _I32, _P, _P, ctypes.POINTER(_FP8), _P, _P, _SZ, _P]
lib.moe_shared_expert.restype = _I32
lib.moe_combine.argtypes = [ctypes.POINTER(_Dims), _I32, _P, _P, _P, _P, _P]
lib.moe_combine.restype = _I32
lib.moe_forward.argtypes = [ctypes.POINTER(_Dims), _I32, _P, _P, _P, ctypes.POINTER(_MXFP4), ctypes.POINTER(_BF16),
                            ctypes.POINTER(_FP8), _P, _P, _P, _P, _P, _SZ, _P]
lib.moe_forward.restype = _I32
lib.moe_forward_noalloc.argtypes = [ctypes.POINTER(_Dims), _I32, _P, _P, _P, ctypes.POINTER(_MXFP4),
                                    ctypes.POINTER(_BF16), ctypes.POINTER(_FP8), _P, _P, _P, _P, _P]
lib.moe_forward_noalloc.restype = _I32
lib.moe_expert_ffn_f32.argtypes = [ctypes.POINTER(_Dims), _I32, _P, _P, ctypes.POINTER(_MXFP4), ctypes.POINTER(_BF16),
                                   _P, _P, _P, _P, _P, _P, _SZ, _P]
lib.moe_expert_ffn_f32.restype = _I32
lib.moe_shared_expert_f32.argtypes = [ctypes.POINTER(_Dims), _I32, _P, _P, ctypes.POINTER(_FP8), _P, _P, _SZ, _P]
lib.moe_shared_expert_f32.restype = _I32
lib.moe_combine_sum_f32.argtypes = [ctypes.POINTER(_Dims), _I32, _P, _P, _P, _P, _P]
lib.moe_combine_sum_f32.restype = _I32
lib.moe_combine_official_f32.argtypes = [ctypes.POINTER(_Dims), _I32, _P, _P, _P, _P, _P, _P]
lib.moe_combine_official_f32.restype = _I32
lib.moe_fp8_linear_workspace_bytes.argtypes = [_I32, _I32, _I32]
lib.moe_fp8_linear_workspace_bytes.restype = _SZ
lib.moe_fp8_linear.argtypes = [_I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _SZ, _P]
lib.moe_fp8_linear.restype = _I32
lib.moe_fp8_linear_tiled.argtypes = [_I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _SZ, _P]
lib.moe_fp8_linear_tiled.restype = _I32
lib.moe_fp8_tiled_weights_bytes.argtypes = [_I32, _I32]
lib.moe_fp8_tiled_weights_bytes.restype = _SZ
lib.moe_prepare_fp8_weights.argtypes = [_I32, _I32, _P, _P, _P]
lib.moe_prepare_fp8_weights.restype = _I32
lib.moe_mxfp4_stage_scales_bytes.argtypes = [ctypes.POINTER(_Dims)]
lib.moe_mxfp4_stage_scales_bytes.restype = _SZ
lib.moe_prepare_mxfp4_scales.argtypes = [ctypes.POINTER(_Dims), ctypes.POINTER(_MXFP4), _P, _P]
lib.moe_prepare_mxfp4_scales.restype = _I32
lib.moe_mxfp4_tiled_weights_bytes.argtypes = [ctypes.POINTER(_Dims)]
lib.moe_mxfp4_tiled_weights_bytes.restype = _SZ
lib.moe_prepare_mxfp4_weights.argtypes = [ctypes.POINTER(_Dims), ctypes.POINTER(_MXFP4), _P, _P]
lib.moe_prepare_mxfp4_weights.restype = _I32
lib.moe_expand_mxfp4.argtypes = [ctypes.c_int64, _I32, _P, _P, _P, _P]
lib.moe_expand_mxfp4.restype = _I32


@dataclass(frozen=True)
class Dims:
    num_experts: int
    hidden: int
    inter: int
    top_k: int
    route_scale: float = 1.5
    flags: int = 0   # MOE_FLAG_* bits (FLAG_BATCH_INVARIANT)

    def c(self) -> _Dims:
        return _Dims(self.num_experts, self.hidden, self.inter, self.top_k, self.route_scale, self.flags)


@dataclass
class MXFP4Experts:
    """Packed routed experts: w1/w3 uint8 [E, I, H/2], s1/s3 [E, I, H/32], w2 [E, H, I/2], s2 [E, H, I/32];
    optionally the moe_prepare_mxfp4_scales output of these scales and the moe_prepare_mxfp4_weights
    output of these weights (uint8, 16-byte aligned; with it, w1/w3/w2 may be None)."""
    w1: torch.Tensor | None
    s1: torch.Tensor
    w3: torch.Tensor | None
    s3: torch.Tensor
    w2: torch.Tensor | None
    s2: torch.Tensor
    stage_scales: torch.Tensor | None = None
    tiled_weights: torch.Tensor | None = None

    def c(self) -> _MXFP4:
        return _MXFP4(*(_ptr(getattr(self, n), torch.uint8)
                        for n in ("w1", "s1", "w3", "s3", "w2", "s2", "stage_scales", "tiled_weights")))


@dataclass
class BF16Experts:
    """Expanded routed experts (bf16 bit patterns as int16/bfloat16): w1/w3 [E, I, H], w2 [E, H, I]."""
    w1: torch.Tensor
    w3: torch.Tensor
    w2: torch.Tensor

    def c(self) -> _BF16:
        return _BF16(*(_ptr(getattr(self, n), (torch.bfloat16, torch.int16)) for n in ("w1", "w3", "w2")))


@dataclass
class FP8Expert:
    """Shared expert: E4M3 bytes w1/w3 [I, H], w2 [H, I]; E8M0 32x32 block scales s1/s3 [I/32, H/32], s2 [H/32, I/32]."""
    w1: torch.Tensor
    s1: torch.Tensor
    w3: torch.Tensor
    s3: torch.Tensor
    w2: torch.Tensor
    s2: torch.Tensor

    def c(self) -> _FP8:
        return _FP8(*(_ptr(getattr(self, n), torch.uint8) for n in ("w1", "s1", "w3", "s3", "w2", "s2")))


def _ptr(t, dtypes=None):
    """Device pointer of a contiguous CUDA tensor (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("libmoe takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libmoe takes contiguous tensors")
    if dtypes is not None:
        ok = dtypes if isinstance(dtypes, tuple) else (dtypes,)
        if t.dtype not in ok:
            raise TypeError(f"dtype {t.dtype} not in {ok}")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(status: int, what: str):
    if status != MOE_OK:
        raise MoeError(f"{what}: {moe_status_str(status)} ({status})")


_BF = (torch.bfloat16, torch.int16)


def moe_status_str(status: int) -> str:
    return lib.moe_status_str(status).decode()


def moe_workspace_bytes(dims: Dims, max_tokens: int) -> int:
    return int(lib.moe_workspace_bytes(ctypes.byref(dims.c()), max_tokens))


def workspace(dims: Dims, max_tokens: int, device="cuda") -> torch.Tensor:
    """A workspace tensor of moe_workspace_bytes(dims, max_tokens) bytes (256-byte aligned)."""
    n = moe_workspace_bytes(dims, max_tokens)
    if n == 0:
        raise MoeError("invalid dims for a workspace")
    ws = torch.empty(n + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws[off:off + n]


def moe_route(dims: Dims, x, gate_w, gate_b, ids, rw, x_q, x_s, ws, stream=None):
    M = x.shape[0]
    st = lib.moe_route(ctypes.byref(dims.c()), M, _ptr(x, _BF), _ptr(gate_w, torch.float32),
                       _ptr(gate_b, torch.float32), _ptr(ids, torch.int32), _ptr(rw, torch.float32),
                       _ptr(x_q, torch.uint8), _ptr(x_s, torch.uint8), _ptr(ws, torch.uint8), ws.numel(),
                       _stream(stream))
    _check(st, "moe_route")


def moe_permute(dims: Dims, ids, counts, offsets, pairs, inv, active, stream=None):
    M = ids.shape[0]
    st = lib.moe_permute(ctypes.byref(dims.c()), M, _ptr(ids, torch.int32), _ptr(counts, torch.int32),
                         _ptr(offsets, torch.int32), _ptr(pairs, torch.int32), _ptr(inv, torch.int32),
                         _ptr(active, torch.int32), _stream(stream))
    _check(st, "moe_permute")


def moe_expert_ffn(dims: Dims, x_q, x_s, packed: MXFP4Experts | None, decoded: BF16Experts | None, rw, offsets,
                   pairs, active, slot_out, h_q=None, h_s=None, ws=None, stream=None):
    M = x_q.shape[0]
    pk = ctypes.byref(packed.c()) if packed is not None else None
    dc = ctypes.byref(decoded.c()) if decoded is not None else None
    st = lib.moe_expert_ffn(ctypes.byref(dims.c()), M, _ptr(x_q, torch.uint8), _ptr(x_s, torch.uint8), pk, dc,
                            _ptr(rw, torch.float32), _ptr(offsets, torch.int32), _ptr(pairs, torch.int32),
                            _ptr(active, torch.int32), _ptr(slot_out, _BF), _ptr(h_q, torch.uint8),
                            _ptr(h_s, torch.uint8), _ptr(ws, torch.uint8), 0 if ws is None else ws.numel(),
                            _stream(stream))
    _check(st, "moe_expert_ffn")


def moe_expert_gemm1(dims: Dims, x_q, x_s, packed: MXFP4Experts | None, decoded: BF16Experts | None, rw, offsets,
                     pairs, active, h_q, h_s, ws, stream=None):
    M = x_q.shape[0]
    pk = ctypes.byref(packed.c()) if packed is not None else None
    dc = ctypes.byref(decoded.c()) if decoded is not None else None
    st = lib.moe_expert_gemm1(ctypes.byref(dims.c()), M, _ptr(x_q, torch.uint8), _ptr(x_s, torch.uint8), pk, dc,
                              _ptr(rw, torch.float32), _ptr(offsets, torch.int32), _ptr(pairs, torch.int32),
                              _ptr(active, torch.int32), _ptr(h_q, torch.uint8), _ptr(h_s, torch.uint8),
                              _ptr(ws, torch.uint8), ws.numel(), _stream(stream))
    _check(st, "moe_expert_gemm1")


def moe_expert_gemm2(dims: Dims, M: int, h_q, h_s, packed: MXFP4Experts | None, decoded: BF16Experts | None, offsets,
                     pairs, active, slot_out, ws, stream=None):
    pk = ctypes.byref(packed.c()) if packed is not None else None
    dc = ctypes.byref(decoded.c()) if decoded is not None else None
    st = lib.moe_expert_gemm2(ctypes.byref(dims.c()), M, _ptr(h_q, torch.uint8), _ptr(h_s, torch.uint8), pk, dc,
                              _ptr(offsets, torch.int32), _ptr(pairs, torch.int32), _ptr(active, torch.int32),
                              _ptr(slot_out, _BF), _ptr(ws, torch.uint8), ws.numel(), _stream(stream))
    _check(st, "moe_expert_gemm2")


def moe_shared_expert(dims: Dims, x_q, x_s, shared: FP8Expert, shared_out, ws, stream=None):
    M = x_q.shape[0]
    st = lib.moe_shared_expert(ctypes.byref(dims.c()), M, _ptr(x_q, torch.uint8), _ptr(x_s, torch.uint8),
                               ctypes.byref(shared.c()), _ptr(shared_out, _BF), _ptr(ws, torch.uint8), ws.numel(),
                               _stream(stream))
    _check(st, "moe_shared_expert")


def moe_combine(dims: Dims, ids, slot_out, shared_out, out, stream=None):
    M = ids.shape[0]
    st = lib.moe_combine(ctypes.byref(dims.c()), M, _ptr(ids, torch.int32), _ptr(slot_out, _BF),
                         _ptr(shared_out, _BF), _ptr(out, _BF), _stream(stream))
    _check(st, "moe_combine")


def moe_expert_ffn_f32(dims: Dims, x_q, x_s, packed: MXFP4Experts | None, decoded: BF16Experts | None, rw, offsets,
                       pairs, active, slot_f32, ws, stream=None):
    """Mode SLOT: fp32 [M*k, H] unrounded expert outputs (rows = pair ids)."""
    M = x_q.shape[0]
    pk = ctypes.byref(packed.c()) if packed is not None else None
    dc = ctypes.byref(decoded.c()) if decoded is not None else None
    st = lib.moe_expert_ffn_f32(ctypes.byref(dims.c()), M, _ptr(x_q, torch.uint8), _ptr(x_s, torch.uint8), pk, dc,
                                _ptr(rw, torch.float32), _ptr(offsets, torch.int32), _ptr(pairs, torch.int32),
                                _ptr(active, torch.int32), _ptr(slot_f32, torch.float32), _ptr(ws, torch.uint8),
                                ws.numel(), _stream(stream))
    _check(st, "moe_expert_ffn_f32")


def moe_shared_expert_f32(dims: Dims, x_q, x_s, shared: FP8Expert, shared_f32, ws, stream=None):
    M = x_q.shape[0]
    st = lib.moe_shared_expert_f32(ctypes.byref(dims.c()), M, _ptr(x_q, torch.uint8), _ptr(x_s, torch.uint8),
                                   ctypes.byref(shared.c()), _ptr(shared_f32, torch.float32), _ptr(ws, torch.uint8),
                                   ws.numel(), _stream(stream))
    _check(st, "moe_shared_expert_f32")


def moe_combine_sum_f32(dims: Dims, ids, slot_f32, add, out_f32, stream=None):
    M = ids.shape[0]
    st = lib.moe_combine_sum_f32(ctypes.byref(dims.c()), M, _ptr(ids, torch.int32), _ptr(slot_f32, torch.float32),
                                 _ptr(add, torch.float32), _ptr(out_f32, torch.float32), _stream(stream))
    _check(st, "moe_combine_sum_f32")


def moe_combine_official_f32(dims: Dims, ids, slot_f32, out, shared_f32=None, shared_bf16=None, stream=None):
    M = ids.shape[0]
    st = lib.moe_combine_official_f32(ctypes.byref(dims.c()), M, _ptr(ids, torch.int32),
                                      _ptr(slot_f32, torch.float32), _ptr(shared_f32, torch.float32),
                                      _ptr(shared_bf16, _BF), _ptr(out, _BF), _stream(stream))
    _check(st, "moe_combine_official_f32")


def moe_forward(dims: Dims, x, gate_w, gate_b, packed: MXFP4Experts | None, decoded: BF16Experts | None,
                shared: FP8Expert | None, out, ids_out=None, rw_out=None, shared_out=None, ws=None, stream=None):
    M = x.shape[0]
    pk = ctypes.byref(packed.c()) if packed is not None else None
    dc = ctypes.byref(decoded.c()) if decoded is not None else None
    sh = ctypes.byref(shared.c()) if shared is not None else None
    st = lib.moe_forward(ctypes.byref(dims.c()), M, _ptr(x, _BF), _ptr(gate_w, torch.float32),
                         _ptr(gate_b, torch.float32), pk, dc, sh, _ptr(out, _BF), _ptr(ids_out, torch.int32),
                         _ptr(rw_out, torch.float32), _ptr(shared_out, _BF), _ptr(ws, torch.uint8),
                         0 if ws is None else ws.numel(), _stream(stream))
    _check(st, "moe_forward")


# size of the library-owned workspace of moe_forward_noalloc (MOE_NOALLOC_SCRATCH_BYTES in moe.h)
NOALLOC_SCRATCH_BYTES = 16 << 20
# Dims.flags bit: one router summation order at every M, so a token's bits do not depend on the batch
# (MOE_FLAG_BATCH_INVARIANT)
FLAG_BATCH_INVARIANT = 1
# the routed GEMMs run over the row-tile list once M * top_k >= TILED_ROWS_PER_EXPERT * num_experts
# (MOE_TILED_ROWS_PER_EXPERT in moe.h)
TILED_ROWS_PER_EXPERT = 6


def moe_forward_noalloc(dims: Dims, x, gate_w, gate_b, packed: MXFP4Experts | None, decoded: BF16Experts | None,
                        shared: FP8Expert | None, out, ids_out=None, rw_out=None, shared_out=None, stream=None):
    """moe_forward with the library's own per-GPU workspace (no ws argument; see moe.h for the limit)."""
    M = x.shape[0]
    pk = ctypes.byref(packed.c()) if packed is not None else None
    dc = ctypes.byref(decoded.c()) if decoded is not None else None
    sh = ctypes.byref(shared.c()) if shared is not None else None
    st = lib.moe_forward_noalloc(ctypes.byref(dims.c()), M, _ptr(x, _BF), _ptr(gate_w, torch.float32),
                                 _ptr(gate_b, torch.float32), pk, dc, sh, _ptr(out, _BF),
                                 _ptr(ids_out, torch.int32), _ptr(rw_out, torch.float32), _ptr(shared_out, _BF),
                                 _stream(stream))
    _check(st, "moe_forward_noalloc")


def moe_expand_mxfp4(w, s, out, stream=None):
    """w uint8 [..., rows, cols/2], s uint8 [..., rows, cols/32] -> out bf16 [..., rows, cols]."""
    cols = w.shape[-1] * 2
    rows = w.numel() // w.shape[-1]
    st = lib.moe_expand_mxfp4(rows, cols, _ptr(w, torch.uint8), _ptr(s, torch.uint8), _ptr(out, _BF),
                              _stream(stream))
    _check(st, "moe_expand_mxfp4")


def moe_mxfp4_stage_scales_bytes(dims: Dims) -> int:
    return int(lib.moe_mxfp4_stage_scales_bytes(ctypes.byref(dims.c())))


def moe_prepare_mxfp4_scales(dims: Dims, packed: MXFP4Experts, out=None, stream=None) -> torch.Tensor:
    """The stage-major copy of packed's s1, s3, s2 (into out, or a new uint8 tensor on their device)."""
    n = moe_mxfp4_stage_scales_bytes(dims)
    if n == 0:
        raise MoeError("invalid dims for stage scales")
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device=packed.s1.device)
    st = lib.moe_prepare_mxfp4_scales(ctypes.byref(dims.c()), ctypes.byref(packed.c()), _ptr(out, torch.uint8),
                                      _stream(stream))
    _check(st, "moe_prepare_mxfp4_scales")
    return out


def moe_mxfp4_tiled_weights_bytes(dims: Dims) -> int:
    return int(lib.moe_mxfp4_tiled_weights_bytes(ctypes.byref(dims.c())))


def moe_prepare_mxfp4_weights(dims: Dims, packed: MXFP4Experts, out=None, stream=None) -> torch.Tensor:
    """The fragment-order copy of packed's w1, w3, w2 (into out, or a new uint8 tensor on their device)."""
    n = moe_mxfp4_tiled_weights_bytes(dims)
    if n == 0:
        raise MoeError("invalid dims for tiled weights")
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device=packed.w1.device)
    st = lib.moe_prepare_mxfp4_weights(ctypes.byref(dims.c()), ctypes.byref(packed.c()), _ptr(out, torch.uint8),
                                       _stream(stream))
    _check(st, "moe_prepare_mxfp4_weights")
    return out


def moe_fp8_linear_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib.moe_fp8_linear_workspace_bytes(M, N, K))


def fp8_linear_workspace(M: int, N: int, K: int, device="cuda") -> torch.Tensor:
    """A workspace tensor for moe_fp8_linear (256-byte aligned)."""
    n = moe_fp8_linear_workspace_bytes(M, N, K)
    if n == 0:
        raise MoeError("unsupported dense linear shape")
    ws = torch.empty(n + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws[off:off + n]


def moe_fp8_linear(x, w, s, y=None, y_f32=None, ws=None, stream=None):
    """y = bf16(act_qdq(x) W^T): x bf16 [M, K], w uint8 E4M3 [N, K], s uint8 E8M0 [N/32, K/32]; exactly
    one of y (bf16 [M, N]) or y_f32 (fp32 [M, N])."""
    M, K = x.shape
    N = w.shape[0]
    if ws is None:
        ws = fp8_linear_workspace(M, N, K, device=x.device)
    st = lib.moe_fp8_linear(M, N, K, _ptr(x, _BF), _ptr(w, torch.uint8), _ptr(s, torch.uint8), _ptr(y, _BF),
                            _ptr(y_f32, torch.float32), _ptr(ws, torch.uint8), ws.numel(), _stream(stream))
    _check(st, "moe_fp8_linear")


def moe_fp8_tiled_weights_bytes(N: int, K: int) -> int:
    return int(lib.moe_fp8_tiled_weights_bytes(N, K))


def moe_prepare_fp8_weights(w, out=None, stream=None) -> torch.Tensor:
    """The fragment-order copy of a dense FP8 weight matrix w uint8 [N, K] (into out, or a new uint8 tensor
    of N * K bytes on w's device)."""
    N, K = w.shape
    n = moe_fp8_tiled_weights_bytes(N, K)
    if n == 0:
        raise MoeError("unsupported dense linear shape")
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device=w.device)
    st = lib.moe_prepare_fp8_weights(N, K, _ptr(w, torch.uint8), _ptr(out, torch.uint8), _stream(stream))
    _check(st, "moe_prepare_fp8_weights")
    return out


def moe_fp8_linear_tiled(x, w_tiled, N, s, y=None, y_f32=None, ws=None, stream=None):
    """moe_fp8_linear with the moe_prepare_fp8_weights copy of the [N, K] weights (decode widths, M <= 64)."""
    M, K = x.shape
    if ws is None:
        ws = fp8_linear_workspace(M, N, K, device=x.device)
    st = lib.moe_fp8_linear_tiled(M, N, K, _ptr(x, _BF), _ptr(w_tiled, torch.uint8), _ptr(s, torch.uint8),
                                  _ptr(y, _BF), _ptr(y_f32, torch.float32), _ptr(ws, torch.uint8), ws.numel(),
                                  _stream(stream))
    _check(st, "moe_fp8_linear_tiled")
