"""ctypes binding of libw4a8.so (argument marshalling only)."""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libw4a8.so")

SCALE_ROW_MAJOR = 0
SCALE_M_MAJOR = 1

_STATUS = {0: "W4A8_OK", 1: "W4A8_ERR_NULL", 2: "W4A8_ERR_SHAPE", 3: "W4A8_ERR_LAYOUT",
           4: "W4A8_ERR_ALIGN", 5: "W4A8_ERR_CAPACITY", 6: "W4A8_ERR_DEVICE", 7: "W4A8_ERR_HIP"}

_lib = None


class W4A8Error(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        self.status = status
        super().__init__(f"{fn}: {_STATUS.get(status, status)}: {detail}")


def lib_path() -> str:
    return _LIB_PATH


def _declare(lib):
    i32, i64, sz, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
    lib.w4a8_route_prep.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp]
    lib.w4a8_route_prep.restype = i32
    lib.w4a8_route_prep_waves.argtypes = [i32, sz]
    lib.w4a8_route_prep_waves.restype = i32
    lib.w4a8_plan_bytes.argtypes = [i32, i64]
    lib.w4a8_plan_bytes.restype = sz
    lib.w4a8_plan.argtypes = [vp, i32, i32, i32, vp, sz, vp]
    lib.w4a8_plan.restype = i32
    lib.w4a8_grouped_gemm.argtypes = [vp, vp, i32, vp, vp, vp, i32, i32, i32, vp, vp]
    lib.w4a8_grouped_gemm.restype = i32
    lib.w4a8_grouped_gemm_planned.argtypes = [vp, vp, i32, vp, vp, vp, i32, i32, i32, vp, sz, vp, vp]
    lib.w4a8_grouped_gemm_planned.restype = i32
    lib.w4a8_grouped_gemm_planned_noalloc.argtypes = [vp, vp, i32, vp, vp, vp, i32, i32, i32, i64, vp, vp]
    lib.w4a8_grouped_gemm_planned_noalloc.restype = i32
    lib.w4a8_grouped_gemm_swiglu.argtypes = [vp, vp, i32, vp, vp, vp, i32, i32, i32, vp, vp, i32, vp]
    lib.w4a8_grouped_gemm_swiglu.restype = i32
    lib.w4a8_grouped_gemm_a16.argtypes = [vp, vp, vp, i32, vp, vp, i32, i32, i32, vp, vp]
    lib.w4a8_grouped_gemm_a16.restype = i32
    lib.w4a8_swiglu_quant.argtypes = [vp, i32, i32, vp, vp, i32, vp]
    lib.w4a8_swiglu_quant.restype = i32
    lib.w4a8_combine.argtypes = [vp, i32, i32, vp, vp, i32, i32, vp, vp]
    lib.w4a8_combine.restype = i32
    lib.w4a8_quantize_gather.argtypes = [vp, i32, i32, vp, i32, i32, vp, vp, i32, vp]
    lib.w4a8_quantize_gather.restype = i32
    lib.w4a8_plan_params.argtypes = [ctypes.POINTER(ctypes.c_int32), i32]
    lib.w4a8_plan_params.restype = i32
    lib.w4a8_status_string.argtypes = [i32]
    lib.w4a8_status_string.restype = ctypes.c_char_p
    lib.w4a8_last_error.argtypes = []
    lib.w4a8_last_error.restype = ctypes.c_char_p


def load(require_device: bool = True):
    """Load libw4a8.so (once).  Raises if it is missing, or -- when
    ``require_device`` -- if the current CUDA device is not gfx950."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m moe_grouped_precision_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        _declare(lib)
        _lib = lib
    if require_device:
        if not torch.cuda.is_available():
            raise RuntimeError("libw4a8 needs a visible MI355X (gfx950) GPU")
        arch = torch.cuda.get_device_properties(torch.cuda.current_device()).gcnArchName
        if not arch.startswith("gfx950"):
            raise RuntimeError(f"libw4a8 supports gfx950 only, current device is {arch}")
    return _lib


def _check(fn: str, status: int):
    if status != 0:
        raise W4A8Error(fn, status, _lib.w4a8_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, numel: Optional[int] = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")


def plan_params():
    """(GRAN, S_MAX, T_MAX, TN_STREAM, TN_MFMA, header words, tile words)."""
    lib = load(require_device=False)
    out = (ctypes.c_int32 * 7)()
    n = lib.w4a8_plan_params(out, 7)
    return tuple(out[i] for i in range(n))


def plan_bytes(E: int, max_total_rows: int) -> int:
    return int(load(require_device=False).w4a8_plan_bytes(E, max_total_rows))


def route_prep_waves(E: int, lds_limit_bytes: int) -> int:
    """Waves per workgroup the route prep uses for E experts under an LDS limit (0: none fits)."""
    return int(load(require_device=False).w4a8_route_prep_waves(E, lds_limit_bytes))


def route_prep(topk_ids: torch.Tensor, E: int, counts=None, offsets=None, row_of_slot=None):
    """topk_ids int32 [T, top_k] -> (counts [E], expert_offsets [E+1], row_of_slot [T*top_k])."""
    lib = load()
    if topk_ids.dim() != 2:
        raise ValueError("topk_ids must be [T, top_k]")
    T, k = topk_ids.shape
    _need(topk_ids, "topk_ids", torch.int32)
    dev = topk_ids.device
    if counts is None:
        counts = torch.empty(E, dtype=torch.int32, device=dev)
    if offsets is None:
        offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    if row_of_slot is None:
        row_of_slot = torch.empty(T * k, dtype=torch.int32, device=dev)
    _need(counts, "counts", torch.int32, E)
    _need(offsets, "expert_offsets", torch.int32, E + 1)
    _need(row_of_slot, "row_of_slot", torch.int32, T * k)
    _check("w4a8_route_prep", lib.w4a8_route_prep(_ptr(topk_ids), T, k, E, _ptr(counts),
                                                 _ptr(offsets), _ptr(row_of_slot), _stream()))
    return counts, offsets, row_of_slot


def plan(expert_offsets: torch.Tensor, E: int, N: int, K: int, max_total_rows: Optional[int] = None,
         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Device tile plan as an int32 tensor (8-word header + 4 words per m-tile)."""
    lib = load()
    _need(expert_offsets, "expert_offsets", torch.int32, E + 1)
    if out is None:
        if max_total_rows is None:
            raise ValueError("give max_total_rows (an upper bound on offsets[E]) or out")
        nbytes = lib.w4a8_plan_bytes(E, max_total_rows)
        if nbytes == 0:
            raise ValueError("invalid E or max_total_rows")
        out = torch.zeros(nbytes // 4, dtype=torch.int32, device=expert_offsets.device)
    _need(out, "plan", torch.int32)
    _check("w4a8_plan", lib.w4a8_plan(_ptr(expert_offsets), E, N, K, _ptr(out), out.numel() * 4,
                                      _stream()))
    return out


def grouped_gemm(A: torch.Tensor, SA: torch.Tensor, layout: int, B: torch.Tensor, SB: torch.Tensor,
                 expert_offsets: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C[R, N] (torch.bfloat16) of the grouped W4A8 GEMM.

    A uint8 [R, K] E4M3 codes; SA fp32 [R, K/128] (layout 0) or [K/128, R]
    (layout 1); B uint8 [E, N, K/2] packed E2M1; SB uint8 [E, N, K/32] E8M0;
    expert_offsets int32 [E+1] with offsets[E] == R.
    """
    lib = load()
    if A.dim() != 2 or B.dim() != 3 or SB.dim() != 3:
        raise ValueError("A must be [R, K], B [E, N, K/2], SB [E, N, K/32]")
    R, K = A.shape
    E, N, Kh = B.shape
    if Kh * 2 != K or SB.shape != (E, N, K // 32):
        raise ValueError("inconsistent K between A, B and SB")
    _need(A, "A", torch.uint8)
    _need(SA, "a_scales", torch.float32, R * (K // 128))
    _need(B, "B", torch.uint8)
    _need(SB, "b_scales", torch.uint8)
    _need(expert_offsets, "expert_offsets", torch.int32, E + 1)
    if out is None:
        out = torch.empty((R, N), dtype=torch.bfloat16, device=A.device)
    if out.dtype not in (torch.bfloat16, torch.uint16, torch.int16):
        raise TypeError("out must be bfloat16 (or 16-bit integer bits)")
    _need(out, "out", out.dtype, R * N)
    if R == 0:
        return out  # no rows: nothing to compute
    _check("w4a8_grouped_gemm", lib.w4a8_grouped_gemm(
        _ptr(A), _ptr(SA), int(layout), _ptr(B), _ptr(SB), _ptr(expert_offsets), E, N, K,
        _ptr(out), _stream()))
    return out


WSCALE_MX = 0  # MXFP4 weight scales: E8M0 per 32 K
WSCALE_NV = 1  # NVFP4 weight scales: E4M3 per 16 K


def grouped_gemm_a16(A: torch.Tensor, B: torch.Tensor, SB: torch.Tensor, fmt: int, expert_offsets: torch.Tensor,
                     expert_scales: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C[R, N] (bf16) of the grouped GEMM with bf16 activations and FP4
    weights.  A bf16 (or 16-bit integer bits) [R, K]; B uint8 [E, N, K/2]
    packed E2M1; SB uint8 [E, N, K/32] E8M0 (fmt WSCALE_MX) or [E, N, K/16]
    E4M3 (fmt WSCALE_NV); expert_scales fp32 [E] or None; expert_offsets
    int32 [E+1] with offsets[E] == R."""
    lib = load()
    if A.dim() != 2 or B.dim() != 3 or SB.dim() != 3:
        raise ValueError("A must be [R, K], B [E, N, K/2], SB [E, N, K/blk]")
    R, K = A.shape
    E, N, Kh = B.shape
    blk = 32 if fmt == WSCALE_MX else 16
    if Kh * 2 != K or SB.shape != (E, N, K // blk):
        raise ValueError("inconsistent K between A, B and SB")
    if A.dtype not in (torch.bfloat16, torch.uint16, torch.int16):
        raise TypeError("A must be bfloat16 (or 16-bit integer bits)")
    _need(A, "A", A.dtype)
    _need(B, "B", torch.uint8)
    _need(SB, "b_scales", torch.uint8)
    if expert_scales is not None:
        _need(expert_scales, "expert_scales", torch.float32, E)
    _need(expert_offsets, "expert_offsets", torch.int32, E + 1)
    if out is None:
        out = torch.empty((R, N), dtype=torch.bfloat16, device=A.device)
    if out.dtype not in (torch.bfloat16, torch.uint16, torch.int16):
        raise TypeError("out must be bfloat16 (or 16-bit integer bits)")
    _need(out, "out", out.dtype, R * N)
    if R == 0:
        return out
    _check("w4a8_grouped_gemm_a16", lib.w4a8_grouped_gemm_a16(
        _ptr(A), _ptr(B), _ptr(SB), int(fmt), _ptr(expert_scales), _ptr(expert_offsets), E, N, K,
        _ptr(out), _stream()))
    return out


def grouped_gemm_planned(A: torch.Tensor, SA: torch.Tensor, layout: int, B: torch.Tensor, SB: torch.Tensor,
                         expert_offsets: torch.Tensor, plan: torch.Tensor,
                         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C[R, N] (bf16) of the grouped W4A8 GEMM over a tile list `plan` (int32,
    w4a8_plan's format, e.g. the output of plan()); the rest as grouped_gemm."""
    lib = load()
    if A.dim() != 2 or B.dim() != 3 or SB.dim() != 3:
        raise ValueError("A must be [R, K], B [E, N, K/2], SB [E, N, K/32]")
    R, K = A.shape
    E, N, Kh = B.shape
    if Kh * 2 != K or SB.shape != (E, N, K // 32):
        raise ValueError("inconsistent K between A, B and SB")
    _need(A, "A", torch.uint8)
    _need(SA, "a_scales", torch.float32, R * (K // 128))
    _need(B, "B", torch.uint8)
    _need(SB, "b_scales", torch.uint8)
    _need(expert_offsets, "expert_offsets", torch.int32, E + 1)
    _need(plan, "plan", torch.int32)
    if out is None:
        out = torch.empty((R, N), dtype=torch.bfloat16, device=A.device)
    if out.dtype not in (torch.bfloat16, torch.uint16, torch.int16):
        raise TypeError("out must be bfloat16 (or 16-bit integer bits)")
    _need(out, "out", out.dtype, R * N)
    if R == 0:
        return out
    _check("w4a8_grouped_gemm_planned", lib.w4a8_grouped_gemm_planned(
        _ptr(A), _ptr(SA), int(layout), _ptr(B), _ptr(SB), _ptr(expert_offsets), E, N, K, _ptr(plan),
        plan.numel() * 4, _ptr(out), _stream()))
    return out


def grouped_gemm_planned_noalloc(A: torch.Tensor, SA: torch.Tensor, layout: int, B: torch.Tensor,
                                 SB: torch.Tensor, expert_offsets: torch.Tensor, out: torch.Tensor,
                                 max_total_rows: Optional[int] = None) -> torch.Tensor:
    """The planned GEMM with its plan in the library's device scratch: nothing
    is allocated, so `out` (bf16 [R, N]) must be given; max_total_rows
    defaults to R = A.shape[0]."""
    lib = load()
    if A.dim() != 2 or B.dim() != 3 or SB.dim() != 3:
        raise ValueError("A must be [R, K], B [E, N, K/2], SB [E, N, K/32]")
    R, K = A.shape
    E, N, Kh = B.shape
    if Kh * 2 != K or SB.shape != (E, N, K // 32):
        raise ValueError("inconsistent K between A, B and SB")
    _need(A, "A", torch.uint8)
    _need(SA, "a_scales", torch.float32, R * (K // 128))
    _need(B, "B", torch.uint8)
    _need(SB, "b_scales", torch.uint8)
    _need(expert_offsets, "expert_offsets", torch.int32, E + 1)
    if out.dtype not in (torch.bfloat16, torch.uint16, torch.int16):
        raise TypeError("out must be bfloat16 (or 16-bit integer bits)")
    _need(out, "out", out.dtype, R * N)
    if R == 0:
        return out
    _check("w4a8_grouped_gemm_planned_noalloc", lib.w4a8_grouped_gemm_planned_noalloc(
        _ptr(A), _ptr(SA), int(layout), _ptr(B), _ptr(SB), _ptr(expert_offsets), E, N, K,
        int(R if max_total_rows is None else max_total_rows), _ptr(out), _stream()))
    return out


def grouped_gemm_swiglu(A: torch.Tensor, SA: torch.Tensor, layout: int, B13: torch.Tensor, SB13: torch.Tensor,
                        expert_offsets: torch.Tensor, layout2: int, A2: Optional[torch.Tensor] = None,
                        SA2: Optional[torch.Tensor] = None):
    """The gate/up GEMM with SwiGLU and E4M3 requantization in its epilogue:
    (A2 uint8 [R, I] codes of silu(gate) * up, SA2 fp32 [R, I/128] for layout2
    0 or [I/128, R] for layout2 1).  B13 uint8 [E, 2I, K/2] (gate columns
    first), SB13 uint8 [E, 2I, K/32]; the rest as grouped_gemm."""
    lib = load()
    if A.dim() != 2 or B13.dim() != 3 or SB13.dim() != 3:
        raise ValueError("A must be [R, K], B13 [E, 2I, K/2], SB13 [E, 2I, K/32]")
    R, K = A.shape
    E, N2, Kh = B13.shape
    if Kh * 2 != K or N2 % 2 or SB13.shape != (E, N2, K // 32):
        raise ValueError("inconsistent shapes between A, B13 and SB13")
    I = N2 // 2
    _need(A, "A", torch.uint8)
    _need(SA, "a_scales", torch.float32, R * (K // 128))
    _need(B13, "B13", torch.uint8)
    _need(SB13, "b13_scales", torch.uint8)
    _need(expert_offsets, "expert_offsets", torch.int32, E + 1)
    if A2 is None:
        A2 = torch.empty((R, I), dtype=torch.uint8, device=A.device)
    if SA2 is None:
        SA2 = torch.empty((R, I // 128) if layout2 == 0 else (I // 128, R), dtype=torch.float32, device=A.device)
    _need(A2, "A2", torch.uint8, R * I)
    _need(SA2, "a2_scales", torch.float32, R * (I // 128))
    if R == 0:
        return A2, SA2
    _check("w4a8_grouped_gemm_swiglu", lib.w4a8_grouped_gemm_swiglu(
        _ptr(A), _ptr(SA), int(layout), _ptr(B13), _ptr(SB13), _ptr(expert_offsets), E, I, K, _ptr(A2),
        _ptr(SA2), int(layout2), _stream()))
    return A2, SA2


def quantize_gather(x: torch.Tensor, row_of_slot: torch.Tensor, top_k: int, R: int, layout: int,
                    A: Optional[torch.Tensor] = None, SA: Optional[torch.Tensor] = None):
    """bf16 tokens x [T, K] -> (A uint8 [R, K] E4M3 codes, SA fp32 scales) written
    to the grouped row of every slot (row_of_slot int32 [T * top_k]); SA is
    [R, K/128] for layout 0 and [K/128, R] for layout 1."""
    lib = load()
    if x.dim() != 2:
        raise ValueError("x must be [T, K]")
    T, K = x.shape
    if x.dtype not in (torch.bfloat16, torch.uint16, torch.int16):
        raise TypeError("x must be bfloat16 (or 16-bit integer bits)")
    _need(x, "x", x.dtype)
    _need(row_of_slot, "row_of_slot", torch.int32, T * top_k)
    if A is None:
        A = torch.zeros((R, K), dtype=torch.uint8, device=x.device)
    if SA is None:
        shape = (R, K // 128) if layout == 0 else (K // 128, R)
        SA = torch.zeros(shape, dtype=torch.float32, device=x.device)
    _need(A, "A", torch.uint8, R * K)
    _need(SA, "a_scales", torch.float32, R * (K // 128))
    _check("w4a8_quantize_gather", lib.w4a8_quantize_gather(
        _ptr(x), T, K, _ptr(row_of_slot), int(top_k), int(R), _ptr(A), _ptr(SA), int(layout), _stream()))
    return A, SA


def combine(C: torch.Tensor, row_of_slot: torch.Tensor, weights: torch.Tensor, top_k: int,
            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[t, :] (bf16) = sum_j weights[t*top_k + j] * C[row_of_slot[t*top_k + j], :],
    fp32 in slot order; C [R, N] bf16 grouped rows, row_of_slot int32 and
    weights fp32 of T*top_k slots."""
    lib = load()
    if C.dim() != 2:
        raise ValueError("C must be [R, N]")
    R, N = C.shape
    if C.dtype not in (torch.bfloat16, torch.uint16, torch.int16):
        raise TypeError("C must be bfloat16 (or 16-bit integer bits)")
    _need(C, "C", C.dtype)
    if row_of_slot.numel() % top_k:
        raise ValueError("row_of_slot must hold T * top_k entries")
    T = row_of_slot.numel() // top_k
    _need(row_of_slot, "row_of_slot", torch.int32, T * top_k)
    _need(weights, "weights", torch.float32, T * top_k)
    if out is None:
        out = torch.empty((T, N), dtype=torch.bfloat16, device=C.device)
    if out.dtype not in (torch.bfloat16, torch.uint16, torch.int16):
        raise TypeError("out must be bfloat16 (or 16-bit integer bits)")
    _need(out, "out", out.dtype, T * N)
    _check("w4a8_combine", lib.w4a8_combine(_ptr(C), R, N, _ptr(row_of_slot), _ptr(weights), T, int(top_k),
                                            _ptr(out), _stream()))
    return out


def swiglu_quant(C: torch.Tensor, layout: int, A: Optional[torch.Tensor] = None, SA: Optional[torch.Tensor] = None):
    """Gate/up output C [R, 2I] (bf16; gate columns first) -> (A uint8 [R, I]
    E4M3 codes of silu(gate) * up, SA fp32 scales [R, I/128] for layout 0 or
    [I/128, R] for layout 1)."""
    lib = load()
    if C.dim() != 2 or C.shape[1] % 2:
        raise ValueError("C must be [R, 2I]")
    R, I = C.shape[0], C.shape[1] // 2
    if C.dtype not in (torch.bfloat16, torch.uint16, torch.int16):
        raise TypeError("C must be bfloat16 (or 16-bit integer bits)")
    _need(C, "C", C.dtype)
    if A is None:
        A = torch.empty((R, I), dtype=torch.uint8, device=C.device)
    if SA is None:
        SA = torch.empty((R, I // 128) if layout == 0 else (I // 128, R), dtype=torch.float32, device=C.device)
    _need(A, "A", torch.uint8, R * I)
    _need(SA, "a_scales", torch.float32, R * (I // 128))
    _check("w4a8_swiglu_quant", lib.w4a8_swiglu_quant(_ptr(C), R, I, _ptr(A), _ptr(SA), int(layout), _stream()))
    return A, SA
