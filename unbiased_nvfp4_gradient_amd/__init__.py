"""MI355X-native NVFP4 quantizers of Quartet II (MS-EDEN, SR, RTN, 4/6) -- Python binding.

This module only marshals arguments to the C ABI of ``libnvfp4.so`` (declared in
``include/nvfp4.h``); every step of the quantizers runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream.  There is no CPU fallback: if the
library is missing, or a call fails, a RuntimeError is raised.

Layouts: ``"row"`` quantizes the rows of X (groups along the columns), ``"col"`` the
columns (groups along the rows, i.e. the row layout of X^T); each layout has its own tensor
scale and random stream.  Results are ``NVFP4`` triples of device tensors:
codes uint8 [vecs, n/2] (low nibble = even position), scales uint8 [vecs, n/16] (E4M3FN
bits; ``.view(torch.float8_e4m3fn)`` works), tensor_scale float32 [1] (with strip-local
scales, ``nvfp4_quantize_strips``: float32 [ceil(vecs / 128)], one per 128 vectors).
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple, Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnvfp4.so")

GROUP = 128
BLOCK = 16

# status codes (include/nvfp4.h)
OK, ERR_NULL, ERR_SHAPE, ERR_GROUP, ERR_ALIGN, ERR_WORKSPACE, ERR_HIP, ERR_ARG = (
    0, -1, -2, -3, -4, -5, -6, -7)

EXPORTED = ("nvfp4_workspace_bytes", "nvfp4_strerror", "eden_quantize",
            "eden_quantize_noalloc", "sr_quantize",
            "rtn_quantize", "fp46_quantize", "nvfp4_amax", "nvfp4_quantize_amax", "dequantize",
            "nvfp4_gemm_check", "nvfp4_strip_workspace_bytes", "nvfp4_quantize_strips",
            "dequantize_strips", "nvfp4_gemm_check_strips", "mxfp4_quantize", "mxfp4_gemm")

MODE_RTN, MODE_SR, MODE_EDEN, MODE_FP46 = 0, 1, 2, 3
MODES = {"rtn": MODE_RTN, "sr": MODE_SR, "eden": MODE_EDEN, "fp46": MODE_FP46}


class _CTensor(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("tensor_scale", ctypes.c_void_p)]


class _CMx(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("k_tiled", ctypes.c_int32)]


class MXFP4(NamedTuple):
    codes: torch.Tensor         # uint8 [vecs, n/2]; K-tiled: [n/128, vecs, 64]
    scales: torch.Tensor        # uint8 [vecs, n/32], E8M0 bits: 2^(byte - 127); K-tiled:
                                # [n/128, vecs, 4]
    k_tiled: bool = False       # the K-tiled layout (same values; the faster GEMM operand)


class MXQuantized(NamedTuple):
    row: Optional[MXFP4]
    col: Optional[MXFP4]


class NVFP4(NamedTuple):
    codes: torch.Tensor         # uint8 [vecs, n/2]
    scales: torch.Tensor        # uint8 [vecs, n/16], E4M3FN bits
    tensor_scale: torch.Tensor  # float32 [1]


class Quantized(NamedTuple):
    row: Optional[NVFP4]
    col: Optional[NVFP4]


class NVFP4Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed with status {status}: {strerror(status)}")
        self.status = status


_lib_handle = None


def lib() -> ctypes.CDLL:
    """The loaded libnvfp4.so (raises if it has not been built)."""
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m unbiased_nvfp4_gradient_amd.build`")
    h = ctypes.CDLL(LIB_PATH)
    P, i64, u64, i32, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_int,
                            ctypes.c_size_t)
    TP = ctypes.POINTER(_CTensor)
    h.nvfp4_workspace_bytes.argtypes = [i64, i64, i32]
    h.nvfp4_workspace_bytes.restype = sz
    h.nvfp4_strerror.argtypes = [i32]
    h.nvfp4_strerror.restype = ctypes.c_char_p
    h.eden_quantize.argtypes = [P, i64, i64, i32, i32, u64, u64, TP, TP, P, sz, P]
    h.eden_quantize_noalloc.argtypes = [P, i64, i64, i32, i32, u64, u64, TP, TP, P]
    h.sr_quantize.argtypes = [P, i64, i64, i32, i32, u64, i32, u64, TP, TP, P, sz, P]
    h.rtn_quantize.argtypes = [P, i64, i64, i32, i32, i32, u64, TP, TP, P, sz, P]
    h.fp46_quantize.argtypes = [P, i64, i64, i32, i32, i32, u64, TP, TP, P, sz, P]
    h.dequantize.argtypes = [TP, i64, i64, i32, i32, i32, u64, P, P]
    h.nvfp4_amax.argtypes = [P, i64, i64, i32, i32, i32, u64, i32, P, P]
    h.nvfp4_quantize_amax.argtypes = [i32, P, i64, i64, i32, i32, u64, i32, u64, P, TP, TP, P]
    h.nvfp4_gemm_check.argtypes = [TP, TP, i64, i64, i64, i32, P, P]
    h.nvfp4_strip_workspace_bytes.argtypes = [i64, i64, i32]
    h.nvfp4_strip_workspace_bytes.restype = sz
    h.nvfp4_quantize_strips.argtypes = [i32, P, i64, i64, i32, i32, u64, i32, u64, TP, TP, P, sz,
                                        P]
    h.dequantize_strips.argtypes = [TP, i64, i64, i32, i32, i32, u64, P, P]
    h.nvfp4_gemm_check_strips.argtypes = [TP, TP, i64, i64, i64, i32, P, P]
    MP = ctypes.POINTER(_CMx)
    h.mxfp4_quantize.argtypes = [P, i64, i64, i32, i32, u64, i32, u64, MP, MP, P]
    h.mxfp4_gemm.argtypes = [MP, MP, i64, i64, i64, i32, P, P]
    for name in ("eden_quantize", "eden_quantize_noalloc", "sr_quantize", "rtn_quantize", "fp46_quantize", "dequantize",
                 "nvfp4_amax", "nvfp4_quantize_amax", "nvfp4_gemm_check",
                 "nvfp4_quantize_strips", "dequantize_strips", "nvfp4_gemm_check_strips",
                 "mxfp4_quantize", "mxfp4_gemm"):
        getattr(h, name).restype = i32
    _lib_handle = h
    return h


def strerror(status: int) -> str:
    return lib().nvfp4_strerror(int(status)).decode()


def workspace_bytes(rows: int, cols: int, layouts_mask: int = 3) -> int:
    return int(lib().nvfp4_workspace_bytes(rows, cols, layouts_mask))


def _stream_ptr(stream, device) -> Optional[int]:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return s.cuda_stream


def _on(stream, device):
    """Context in which the binding allocates outputs and workspaces: the stream the call is
    enqueued on, so that the caching allocator hands a freed workspace only to later work on
    that same stream."""
    return torch.cuda.stream(stream if stream is not None else torch.cuda.current_stream(device))


def empty_layout(vecs: int, n: int, device) -> NVFP4:
    """Caller-side allocation of one layout's outputs."""
    return NVFP4(torch.empty((vecs, n // 2), dtype=torch.uint8, device=device),
                 torch.empty((vecs, n // BLOCK), dtype=torch.uint8, device=device),
                 torch.empty((1,), dtype=torch.float32, device=device))


def _ct(t: Optional[NVFP4]):
    if t is None:
        return None
    return ctypes.byref(_CTensor(t.codes.data_ptr(), t.scales.data_ptr(),
                                 t.tensor_scale.data_ptr()))


def _check_buffer(t, name: str, dtype, shape, device):
    """A caller-supplied buffer must be a contiguous tensor of the given dtype and shape on
    the input's device: the C ABI sees only its pointer, so a smaller or differently typed
    buffer would be overrun."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or t.device != device or \
            not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} "
                         f"on {device}; got {t.dtype} {tuple(t.shape)} on {t.device}"
                         f"{'' if t.is_contiguous() else ' (not contiguous)'}")


def _scale_count(vecs: int, strips: bool) -> int:
    return (vecs + GROUP - 1) // GROUP if strips else 1


def _check_layout(t: NVFP4, name: str, vecs: int, n: int, device, strips: bool = False):
    """One layout's outputs (or inputs, for the decoders and the GEMM): codes uint8
    [vecs, n/2], scales uint8 [vecs, n/16], tensor_scale float32 [1] (strip-local:
    [ceil(vecs/128)])."""
    if not isinstance(t, NVFP4):
        if not (isinstance(t, tuple) and len(t) == 3):
            raise ValueError(f"{name} must be an NVFP4 (codes, scales, tensor_scale) triple")
        t = NVFP4(*t)
    _check_buffer(t.codes, f"{name}.codes", torch.uint8, (vecs, n // 2), device)
    _check_buffer(t.scales, f"{name}.scales", torch.uint8, (vecs, n // BLOCK), device)
    _check_buffer(t.tensor_scale, f"{name}.tensor_scale", torch.float32,
                  (_scale_count(vecs, strips),), device)
    return t


def _check_outputs(x: torch.Tensor, out: Quantized, strips: bool = False) -> Quantized:
    rows, cols = x.shape
    row = None if out.row is None else _check_layout(out.row, "out.row", rows, cols, x.device,
                                                     strips)
    col = None if out.col is None else _check_layout(out.col, "out.col", cols, rows, x.device,
                                                     strips)
    return Quantized(row, col)


def _check_workspace(ws, need: int, device):
    if not isinstance(ws, torch.Tensor) or ws.dtype != torch.uint8 or ws.dim() != 1 or \
            ws.device != device or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous 1-D uint8 tensor on {device}")
    if ws.numel() < need:
        raise ValueError(f"workspace holds {ws.numel()} bytes; {need} are needed")


def _decoded_shape(t: NVFP4, name: str, strips: bool):
    """(vecs, n) of an encoded layout, after checking its three tensors agree."""
    if not isinstance(t.codes, torch.Tensor) or t.codes.dim() != 2:
        raise ValueError(f"{name}.codes must be a 2-D uint8 tensor")
    vecs, n = t.codes.shape[0], t.codes.shape[1] * 2
    _check_layout(t, name, vecs, n, t.codes.device, strips)
    return vecs, n


def _prepare(x: torch.Tensor, layouts: Sequence[str], out: Optional[Quantized], workspace,
             stream=None):
    if x.dtype != torch.bfloat16 or not x.is_cuda or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous 2-D bfloat16 device tensor")
    with _on(stream, x.device):
        return _allocate(x, layouts, out, workspace)


def _select(layouts, out: Quantized) -> Quantized:
    """The layouts of a caller's `out` that `layouts` asks for; the others are left alone
    (passed to the library as null, so it neither computes nor writes them)."""
    want_row, want_col = "row" in layouts, "col" in layouts
    for name, want, t in (("row", want_row, out.row), ("col", want_col, out.col)):
        if want and t is None:
            raise ValueError(f"`layouts` asks for the {name} layout but `out` has none")
    return Quantized(out.row if want_row else None, out.col if want_col else None)


def _allocate(x, layouts, out, workspace):
    rows, cols = x.shape
    want_row, want_col = "row" in layouts, "col" in layouts
    if out is None:
        out = Quantized(empty_layout(rows, cols, x.device) if want_row else None,
                        empty_layout(cols, rows, x.device) if want_col else None)
    else:
        out = _check_outputs(x, _select(layouts, out))
    need = workspace_bytes(rows, cols, (1 if want_row else 0) | (2 if want_col else 0))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    else:
        _check_workspace(workspace, need, x.device)
    return rows, cols, out, workspace


def _mode(mode: str) -> int:
    if mode not in MODES:
        raise ValueError(f"unknown quantizer mode {mode!r}; use one of {tuple(MODES)}")
    return MODES[mode]


def _check(fn: str, status: int):
    if status != OK:
        raise NVFP4Error(fn, status)


def eden_quantize(x: torch.Tensor, seed: int, rht_seed: Optional[int] = None,
                  layouts=("row", "col"), out: Optional[Quantized] = None,
                  workspace: Optional[torch.Tensor] = None, stream=None) -> Quantized:
    """MS-EDEN NVFP4 quantization (see include/nvfp4.h).  rht_seed defaults to seed; both
    operands of one GEMM must pass the same rht_seed."""
    rht_seed = seed if rht_seed is None else rht_seed
    rows, cols, out, ws = _prepare(x, layouts, out, workspace, stream)
    _check("eden_quantize", lib().eden_quantize(
        x.data_ptr(), rows, cols, GROUP, BLOCK, seed, rht_seed, _ct(out.row), _ct(out.col),
        ws.data_ptr(), ws.numel(), _stream_ptr(stream, x.device)))
    return out


def eden_quantize_noalloc(x: torch.Tensor, seed: int, rht_seed: Optional[int] = None,
                          layouts=("row", "col"), out: Optional[Quantized] = None,
                          stream=None) -> Quantized:
    """eden_quantize through the entry point that allocates nothing: the library keeps the
    call's workspace in its own device scratch (calls that overlap on one GPU race).  Pass
    `out` to allocate nothing here either."""
    rht_seed = seed if rht_seed is None else rht_seed
    if x.dtype != torch.bfloat16 or not x.is_cuda or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous 2-D bfloat16 device tensor")
    rows, cols = x.shape
    if out is None:
        with _on(stream, x.device):
            out = Quantized(empty_layout(rows, cols, x.device) if "row" in layouts else None,
                            empty_layout(cols, rows, x.device) if "col" in layouts else None)
    else:
        out = _check_outputs(x, _select(layouts, out))
    _check("eden_quantize_noalloc", lib().eden_quantize_noalloc(
        x.data_ptr(), rows, cols, GROUP, BLOCK, seed, rht_seed, _ct(out.row), _ct(out.col),
        _stream_ptr(stream, x.device)))
    return out


def sr_quantize(x: torch.Tensor, seed: int, rht: bool = False, rht_seed: int = 0,
                layouts=("row",), out: Optional[Quantized] = None,
                workspace: Optional[torch.Tensor] = None, stream=None) -> Quantized:
    """Plain stochastic-rounding NVFP4 quantization (optionally rotated first)."""
    rows, cols, out, ws = _prepare(x, layouts, out, workspace, stream)
    _check("sr_quantize", lib().sr_quantize(
        x.data_ptr(), rows, cols, GROUP, BLOCK, seed, int(bool(rht)), rht_seed, _ct(out.row),
        _ct(out.col), ws.data_ptr(), ws.numel(), _stream_ptr(stream, x.device)))
    return out


def rtn_quantize(x: torch.Tensor, rht: bool = False, rht_seed: int = 0, layouts=("row",),
                 out: Optional[Quantized] = None, workspace: Optional[torch.Tensor] = None,
                 stream=None) -> Quantized:
    """Round-to-nearest NVFP4 quantization (optionally rotated first)."""
    rows, cols, out, ws = _prepare(x, layouts, out, workspace, stream)
    _check("rtn_quantize", lib().rtn_quantize(
        x.data_ptr(), rows, cols, GROUP, BLOCK, int(bool(rht)), rht_seed, _ct(out.row),
        _ct(out.col), ws.data_ptr(), ws.numel(), _stream_ptr(stream, x.device)))
    return out


def fp46_quantize(x: torch.Tensor, rht: bool = False, rht_seed: int = 0,
                  layouts=("row", "col"), out: Optional[Quantized] = None,
                  workspace: Optional[torch.Tensor] = None, stream=None) -> Quantized:
    """Forward-pass 4/6 NVFP4 quantization (optionally rotated first)."""
    rows, cols, out, ws = _prepare(x, layouts, out, workspace, stream)
    _check("fp46_quantize", lib().fp46_quantize(
        x.data_ptr(), rows, cols, GROUP, BLOCK, int(bool(rht)), rht_seed, _ct(out.row),
        _ct(out.col), ws.data_ptr(), ws.numel(), _stream_ptr(stream, x.device)))
    return out


def nvfp4_amax(x: torch.Tensor, rht: bool, rht_seed: int = 0, layouts=("row", "col"),
               amax: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Phase 1: float32 [2] device tensor (row, column) of max |r| (rotated when rht)."""
    if x.dtype != torch.bfloat16 or not x.is_cuda or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous 2-D bfloat16 device tensor")
    if amax is None:
        with _on(stream, x.device):
            amax = torch.empty((2,), dtype=torch.float32, device=x.device)
    else:
        _check_buffer(amax, "amax", torch.float32, (2,), x.device)
    mask = (1 if "row" in layouts else 0) | (2 if "col" in layouts else 0)
    _check("nvfp4_amax", lib().nvfp4_amax(
        x.data_ptr(), x.shape[0], x.shape[1], GROUP, BLOCK, int(bool(rht)), rht_seed, mask,
        amax.data_ptr(), _stream_ptr(stream, x.device)))
    return amax


def nvfp4_quantize_amax(mode: str, x: torch.Tensor, amax: torch.Tensor, seed: int = 0,
                        rht: bool = False, rht_seed: int = 0, layouts=("row", "col"),
                        out: Optional[Quantized] = None, stream=None) -> Quantized:
    """Phase 2: quantizer `mode` ("rtn", "sr", "eden", "fp46") given phase-1 maxima."""
    if x.dtype != torch.bfloat16 or not x.is_cuda or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous 2-D bfloat16 device tensor")
    _check_buffer(amax, "amax", torch.float32, (2,), x.device)
    rows, cols = x.shape
    with _on(stream, x.device):
        if out is None:
            out = Quantized(empty_layout(rows, cols, x.device) if "row" in layouts else None,
                            empty_layout(cols, rows, x.device) if "col" in layouts else None)
        else:
            out = _check_outputs(x, _select(layouts, out))
    _check("nvfp4_quantize_amax", lib().nvfp4_quantize_amax(
        _mode(mode), x.data_ptr(), rows, cols, GROUP, BLOCK, seed, int(bool(rht)), rht_seed,
        amax.data_ptr(), _ct(out.row), _ct(out.col), _stream_ptr(stream, x.device)))
    return out


def dequantize(t: NVFP4, rht: bool = False, rht_seed: int = 0,
               out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Decode one layout to float32 [vecs, n]; undoes the rotation when rht is set."""
    vecs, n = _decoded_shape(t, "t", strips=False)
    if out is None:
        with _on(stream, t.codes.device):
            out = torch.empty((vecs, n), dtype=torch.float32, device=t.codes.device)
    else:
        _check_buffer(out, "out", torch.float32, (vecs, n), t.codes.device)
    _check("dequantize", lib().dequantize(
        _ct(t), vecs, n, GROUP, BLOCK, int(bool(rht)), rht_seed, out.data_ptr(),
        _stream_ptr(stream, t.codes.device)))
    return out


def strip_workspace_bytes(rows: int, cols: int, layouts_mask: int = 3) -> int:
    return int(lib().nvfp4_strip_workspace_bytes(rows, cols, layouts_mask))


def empty_strip_layout(vecs: int, n: int, device) -> NVFP4:
    """Caller-side allocation of one strip-local layout (one g per 128 vectors)."""
    return NVFP4(torch.empty((vecs, n // 2), dtype=torch.uint8, device=device),
                 torch.empty((vecs, n // BLOCK), dtype=torch.uint8, device=device),
                 torch.empty(((vecs + GROUP - 1) // GROUP,), dtype=torch.float32, device=device))


def nvfp4_quantize_strips(mode: str, x: torch.Tensor, seed: int = 0, rht: bool = False,
                          rht_seed: int = 0, layouts=("row", "col"),
                          out: Optional[Quantized] = None,
                          workspace: Optional[torch.Tensor] = None, stream=None) -> Quantized:
    """Quantizer `mode` ("rtn", "sr", "eden", "fp46") with strip-local scales: each run of
    128 vectors of a layout has its own tensor_scale entry (the CTA-local variant)."""
    if x.dtype != torch.bfloat16 or not x.is_cuda or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous 2-D bfloat16 device tensor")
    rows, cols = x.shape
    with _on(stream, x.device):
        if out is None:
            out = Quantized(
                empty_strip_layout(rows, cols, x.device) if "row" in layouts else None,
                empty_strip_layout(cols, rows, x.device) if "col" in layouts else None)
        else:
            out = _check_outputs(x, _select(layouts, out), strips=True)
        need = strip_workspace_bytes(rows, cols)
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
        else:
            _check_workspace(workspace, need, x.device)
    _check("nvfp4_quantize_strips", lib().nvfp4_quantize_strips(
        _mode(mode), x.data_ptr(), rows, cols, GROUP, BLOCK, seed, int(bool(rht)), rht_seed,
        _ct(out.row), _ct(out.col), workspace.data_ptr(), workspace.numel(),
        _stream_ptr(stream, x.device)))
    return out


def dequantize_strips(t: NVFP4, rht: bool = False, rht_seed: int = 0,
                      out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Decode one strip-local layout to float32 [vecs, n]."""
    vecs, n = _decoded_shape(t, "t", strips=True)
    if out is None:
        with _on(stream, t.codes.device):
            out = torch.empty((vecs, n), dtype=torch.float32, device=t.codes.device)
    else:
        _check_buffer(out, "out", torch.float32, (vecs, n), t.codes.device)
    _check("dequantize_strips", lib().dequantize_strips(
        _ct(t), vecs, n, GROUP, BLOCK, int(bool(rht)), rht_seed, out.data_ptr(),
        _stream_ptr(stream, t.codes.device)))
    return out


def nvfp4_gemm_check_strips(a: NVFP4, b: NVFP4, rotated_pair: bool = False,
                            out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """C = A B^T of two strip-local row-layout operands, FP32 [M, N]."""
    M, K = _decoded_shape(a, "a", strips=True)
    N, Kb = _decoded_shape(b, "b", strips=True)
    if Kb != K:
        raise ValueError("operands disagree on K")
    if b.codes.device != a.codes.device:
        raise ValueError("operands must be on one device")
    if out is None:
        with _on(stream, a.codes.device):
            out = torch.empty((M, N), dtype=torch.float32, device=a.codes.device)
    else:
        _check_buffer(out, "out", torch.float32, (M, N), a.codes.device)
    _check("nvfp4_gemm_check_strips", lib().nvfp4_gemm_check_strips(
        _ct(a), _ct(b), M, N, K, int(bool(rotated_pair)), out.data_ptr(),
        _stream_ptr(stream, a.codes.device)))
    return out


def nvfp4_gemm_check(a: NVFP4, b: NVFP4, rotated_pair: bool = False,
                     out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """C = A B^T of two row-layout NVFP4 operands ([M, K] and [N, K]), FP32 [M, N]."""
    M, K = _decoded_shape(a, "a", strips=False)
    N, Kb = _decoded_shape(b, "b", strips=False)
    if Kb != K:
        raise ValueError("operands disagree on K")
    if b.codes.device != a.codes.device:
        raise ValueError("operands must be on one device")
    if out is None:
        with _on(stream, a.codes.device):
            out = torch.empty((M, N), dtype=torch.float32, device=a.codes.device)
    else:
        _check_buffer(out, "out", torch.float32, (M, N), a.codes.device)
    _check("nvfp4_gemm_check", lib().nvfp4_gemm_check(
        _ct(a), _ct(b), M, N, K, int(bool(rotated_pair)), out.data_ptr(),
        _stream_ptr(stream, a.codes.device)))
    return out


def _mx_shapes(vecs: int, n: int, k_tiled: bool):
    if k_tiled:
        return (n // 128, vecs, 64), (n // 128, vecs, 4)
    return (vecs, n // 2), (vecs, n // 32)


def empty_mx_layout(vecs: int, n: int, device, k_tiled: bool = False) -> MXFP4:
    """Caller-side allocation of one MXFP4 layout's outputs (K-tiled: n a multiple of 128)."""
    cs, ss = _mx_shapes(vecs, n, k_tiled)
    return MXFP4(torch.empty(cs, dtype=torch.uint8, device=device),
                 torch.empty(ss, dtype=torch.uint8, device=device), bool(k_tiled))


def _cmx(t: Optional[MXFP4]):
    if t is None:
        return None
    return ctypes.byref(_CMx(t.codes.data_ptr(), t.scales.data_ptr(), int(bool(t.k_tiled))))


def _as_mx(t, name: str) -> MXFP4:
    if isinstance(t, MXFP4):
        return t
    if isinstance(t, tuple) and len(t) in (2, 3):
        return MXFP4(*t)
    raise ValueError(f"{name} must be an MXFP4 (codes, scales[, k_tiled]) tuple")


def _mx_dims(t: MXFP4, name: str):
    """(vecs, n) of an MXFP4 layout, from its codes tensor's shape."""
    want = 3 if t.k_tiled else 2
    if not isinstance(t.codes, torch.Tensor) or t.codes.dim() != want:
        raise ValueError(f"{name}.codes must be a {want}-D uint8 tensor")
    if t.k_tiled:
        return t.codes.shape[1], t.codes.shape[0] * 128
    return t.codes.shape[0], t.codes.shape[1] * 2


def _check_mx_layout(t, name: str, vecs: int, n: int, device) -> MXFP4:
    t = _as_mx(t, name)
    if t.k_tiled and n % 128:
        raise ValueError(f"{name}: a K-tiled layout needs n a multiple of 128, not {n}")
    cs, ss = _mx_shapes(vecs, n, t.k_tiled)
    _check_buffer(t.codes, f"{name}.codes", torch.uint8, cs, device)
    _check_buffer(t.scales, f"{name}.scales", torch.uint8, ss, device)
    return t


def mxfp4_quantize(x: torch.Tensor, sr: bool = False, seed: int = 0, rht: bool = False,
                   rht_seed: int = 0, layouts=("row",), out: Optional[MXQuantized] = None,
                   stream=None, k_tiled: bool = False) -> MXQuantized:
    """MXFP4 quantization (E2M1 codes, one E8M0 scale per 32), RTN or SR, optionally after the
    random-sign Hadamard rotation; the operand format of the native FP4 matrix cores.  With
    k_tiled the outputs it allocates take the K-tiled layout (a caller's `out` layouts carry
    their own flag)."""
    if x.dtype != torch.bfloat16 or not x.is_cuda or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous 2-D bfloat16 device tensor")
    rows, cols = x.shape
    want_row, want_col = "row" in layouts, "col" in layouts
    if out is None:
        for want, n in ((want_row, cols), (want_col, rows)):
            if want and k_tiled and n % 128:
                raise ValueError(f"a K-tiled layout needs n a multiple of 128, not {n}")
        with _on(stream, x.device):
            out = MXQuantized(
                empty_mx_layout(rows, cols, x.device, k_tiled) if want_row else None,
                empty_mx_layout(cols, rows, x.device, k_tiled) if want_col else None)
    else:
        for name, want, t in (("row", want_row, out.row), ("col", want_col, out.col)):
            if want and t is None:
                raise ValueError(f"`layouts` asks for the {name} layout but `out` has none")
        out = MXQuantized(
            _check_mx_layout(out.row, "out.row", rows, cols, x.device) if want_row else None,
            _check_mx_layout(out.col, "out.col", cols, rows, x.device) if want_col else None)
    _check("mxfp4_quantize", lib().mxfp4_quantize(
        x.data_ptr(), rows, cols, 32, int(bool(sr)), seed, int(bool(rht)), rht_seed,
        _cmx(out.row), _cmx(out.col), _stream_ptr(stream, x.device)))
    return out


def mxfp4_gemm(a: MXFP4, b: MXFP4, rotated_pair: bool = False,
               out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """C = A B^T of two MXFP4 row-layout operands ([M, K] and [N, K]) on the FP4 matrix
    cores, FP32 [M, N].  Both operands row-major or both K-tiled (the faster kernel); the
    result is the same bit for bit."""
    a, b = _as_mx(a, "a"), _as_mx(b, "b")
    if bool(a.k_tiled) != bool(b.k_tiled):
        raise ValueError("a and b must both be row-major or both K-tiled")
    M, K = _mx_dims(a, "a")
    N, _ = _mx_dims(b, "b")
    dev = a.codes.device
    a = _check_mx_layout(a, "a", M, K, dev)
    b = _check_mx_layout(b, "b", N, K, dev)
    if out is None:
        with _on(stream, dev):
            out = torch.empty((M, N), dtype=torch.float32, device=dev)
    else:
        _check_buffer(out, "out", torch.float32, (M, N), dev)
    _check("mxfp4_gemm", lib().mxfp4_gemm(_cmx(a), _cmx(b), M, N, K, int(bool(rotated_pair)),
                                          out.data_ptr(), _stream_ptr(stream, dev)))
    return out


__all__ = ["MXFP4", "MXQuantized", "mxfp4_quantize", "mxfp4_gemm", "empty_mx_layout",
           "NVFP4", "Quantized", "NVFP4Error", "eden_quantize", "eden_quantize_noalloc",
           "sr_quantize", "rtn_quantize",
           "fp46_quantize", "nvfp4_amax", "nvfp4_quantize_amax", "dequantize", "nvfp4_gemm_check",
           "nvfp4_quantize_strips", "dequantize_strips", "nvfp4_gemm_check_strips",
           "workspace_bytes", "strip_workspace_bytes", "strerror", "empty_layout",
           "empty_strip_layout", "lib", "LIB_PATH", "EXPORTED"]
