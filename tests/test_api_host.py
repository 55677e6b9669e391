"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every entry
point include/nvfp4.h declares, and rejects bad arguments with the documented status codes
before touching any device memory."""
import ctypes
import os
import re

import pytest

import unbiased_nvfp4_gradient_amd as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000000  # a well-aligned non-null address; validation never dereferences it


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(nv.LIB_PATH):
        from unbiased_nvfp4_gradient_amd import build

        build.build()
    return nv.lib()


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "nvfp4.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M))


def test_exports_every_declared_symbol(L):
    declared = _declared_functions()
    assert declared == set(nv.EXPORTED)
    for name in declared:
        assert hasattr(L, name), name


def test_strerror_and_workspace(L):
    for s in (0, -1, -2, -3, -4, -5, -6, -7):
        assert nv.strerror(s)
    assert nv.strerror(-99) == "unknown status"
    assert nv.workspace_bytes(16384, 8192, 3) == 16384 == nv.workspace_bytes(0, 0, 1)


def _layout(codes=FAKE, scales=FAKE + 4096, g=FAKE + 8192):
    return ctypes.byref(nv._CTensor(codes, scales, g))


def _eden(L, x=FAKE, rows=256, cols=256, group=128, block=16, row=True, col=True, ws=FAKE,
          wsb=16384, row_t=None, col_t=None):
    r = row_t if row_t is not None else (_layout() if row else None)
    c = col_t if col_t is not None else (_layout(FAKE + 65536, FAKE + 69632, FAKE + 73728)
                                         if col else None)
    return L.eden_quantize(x, rows, cols, group, block, 1, 1, r, c, ws, wsb, None)


def test_validation_errors(L):
    assert _eden(L, x=0) == nv.ERR_NULL
    assert _eden(L, x=0, rows=0) != nv.ERR_NULL          # an empty input may be NULL
    assert _eden(L, row=False, col=False) == nv.ERR_NULL
    assert _eden(L, row_t=_layout(codes=0)) == nv.ERR_NULL
    assert _eden(L, group=64) == nv.ERR_GROUP
    assert _eden(L, block=32) == nv.ERR_GROUP
    assert _eden(L, rows=-1) == nv.ERR_SHAPE
    assert _eden(L, cols=200) == nv.ERR_SHAPE           # row layout needs cols % 128
    assert _eden(L, rows=200, row=True, col=True) == nv.ERR_SHAPE
    assert _eden(L, cols=252) == nv.ERR_SHAPE           # cols % 8
    assert _eden(L, x=FAKE + 8) == nv.ERR_ALIGN
    assert _eden(L, row_t=_layout(codes=FAKE + 8)) == nv.ERR_ALIGN
    assert _eden(L, row_t=_layout(scales=FAKE + 4)) == nv.ERR_ALIGN
    assert _eden(L, ws=0) == nv.ERR_WORKSPACE
    assert _eden(L, wsb=8) == nv.ERR_WORKSPACE
    assert _eden(L, wsb=16384 - 1) == nv.ERR_WORKSPACE       # two floats x 2048 workgroups
    assert _eden(L, rows=1 << 32) == nv.ERR_ARG
    # the stated limits: each dimension below 2^31, their product below 2^40
    assert _eden(L, rows=1 << 31, col=False) == nv.ERR_ARG
    assert _eden(L, rows=(1 << 31) - 128, cols=1024, col=False) == nv.ERR_ARG  # > 2^40
    assert _eden(L, rows=1 << 21, cols=1 << 19, col=False) == nv.ERR_ARG      # = 2^40
    assert L.dequantize(_layout(), 1 << 31, 128, 128, 16, 0, 0, FAKE, None) == nv.ERR_ARG
    mx = ctypes.byref(nv._CMx(FAKE, FAKE + 4096))
    assert L.mxfp4_gemm(mx, mx, 1 << 21, 1 << 19, 128, 0, FAKE, None) == nv.ERR_ARG
    # sr / rtn / fp46 without rotation accept n % 16
    assert L.sr_quantize(FAKE, 256, 200, 128, 16, 1, 0, 1, _layout(), None, FAKE, 256,
                         None) in (nv.ERR_SHAPE,)           # cols % 8 ok, 200 % 16 != 0
    assert L.rtn_quantize(FAKE, 256, 256, 128, 16, 2, 1, _layout(), None, FAKE, 256,
                          None) == nv.ERR_ARG               # rht flag must be 0/1
    assert L.fp46_quantize(FAKE, 256, 144, 128, 16, 1, 1, _layout(), None, FAKE, 256,
                           None) == nv.ERR_SHAPE           # rotation needs n % 128
    t = _layout()
    assert L.dequantize(None, 4, 128, 128, 16, 0, 0, FAKE, None) == nv.ERR_NULL
    assert L.dequantize(t, 4, 100, 128, 16, 0, 0, FAKE, None) == nv.ERR_SHAPE
    assert L.dequantize(t, 4, 144, 128, 16, 1, 0, FAKE, None) == nv.ERR_SHAPE
    assert L.dequantize(t, 4, 128, 128, 16, 0, 0, FAKE + 4, None) == nv.ERR_ALIGN


def _has_gpu():
    try:
        import torch

        return torch.cuda.device_count() > 0
    except Exception:
        return False


@pytest.mark.skipif(_has_gpu(), reason="only meaningful on a host without a GPU")
def test_no_device_is_a_hip_error(L):
    assert _eden(L) == nv.ERR_HIP


def test_strip_entry_points_validate(L):
    # a 2 KiB table per row strip and per column strip, 32 bytes per tile, 256-byte multiple
    assert nv.strip_workspace_bytes(256, 256) == 2048 * 4 + 256        # 8320 rounded up
    assert nv.strip_workspace_bytes(16384, 8192) == 2048 * (128 + 64) + 32 * 128 * 64
    assert nv.strip_workspace_bytes(0, 0) == 256
    assert nv.strip_workspace_bytes(200, 8) == 2048 * 3 + 32 * 2 + 192   # rounded up
    r, c = _layout(), _layout(FAKE + 65536, FAKE + 69632, FAKE + 73728)

    def q(mode=2, rows=256, cols=256, rht=1, ws=FAKE, wsb=1 << 20):
        return L.nvfp4_quantize_strips(mode, FAKE, rows, cols, 128, 16, 1, rht, 1, r, c, ws, wsb,
                                       None)
    assert q(mode=4) == nv.ERR_ARG
    assert q(mode=-1) == nv.ERR_ARG
    assert q(rht=2) == nv.ERR_ARG
    assert q(cols=200) == nv.ERR_SHAPE
    assert q(ws=0) == nv.ERR_WORKSPACE
    assert q(wsb=2048 * 4) == nv.ERR_WORKSPACE                         # needs 8448 bytes
    assert q(ws=FAKE + 64) == nv.ERR_ALIGN
    assert L.nvfp4_quantize_strips(2, FAKE, 256, 256, 128, 16, 1, 1, 1, None, None, FAKE, 1 << 20,
                                   None) == nv.ERR_NULL
    assert L.dequantize_strips(None, 4, 128, 128, 16, 0, 0, FAKE, None) == nv.ERR_NULL
    assert L.dequantize_strips(r, 4, 100, 128, 16, 0, 0, FAKE, None) == nv.ERR_SHAPE
    assert L.nvfp4_gemm_check_strips(r, r, 48, 64, 128, 1, FAKE, None) == nv.ERR_SHAPE
    assert L.nvfp4_gemm_check_strips(r, r, 64, 64, 128, 3, FAKE, None) == nv.ERR_ARG


def test_gemm_alignment(L):
    ok, odd = _layout(), _layout(scales=FAKE + 4097)
    assert L.nvfp4_gemm_check(ok, odd, 64, 64, 128, 0, FAKE, None) == nv.ERR_ALIGN
    assert L.nvfp4_gemm_check(_layout(codes=FAKE + 8), ok, 64, 64, 128, 0, FAKE, None) == \
        nv.ERR_ALIGN
    assert L.nvfp4_gemm_check(ok, ok, 64, 64, 128, 0, FAKE + 2, None) == nv.ERR_ALIGN


def test_noalloc_validation(L):
    """eden_quantize_noalloc rejects bad arguments exactly as eden_quantize does, before it
    looks up its device scratch (so with no device at all, argument errors still come first)."""
    r, c = _layout(), _layout(FAKE + 65536, FAKE + 69632, FAKE + 73728)

    def q(x=FAKE, rows=256, cols=256, group=128, block=16, row=r, col=c):
        return L.eden_quantize_noalloc(x, rows, cols, group, block, 1, 1, row, col, None)
    assert q(x=0) == nv.ERR_NULL
    assert q(row=None, col=None) == nv.ERR_NULL
    assert q(group=64) == nv.ERR_GROUP
    assert q(cols=200) == nv.ERR_SHAPE
    assert q(x=FAKE + 8) == nv.ERR_ALIGN
    assert q(rows=1 << 32) == nv.ERR_ARG
    if not _has_gpu():
        assert q() == nv.ERR_HIP


def test_mxfp4_validation(L):
    r = ctypes.byref(nv._CMx(FAKE, FAKE + 4096))
    c = ctypes.byref(nv._CMx(FAKE + 65536, FAKE + 69632))

    def q(x=FAKE, rows=256, cols=256, block=32, sr=0, rht=0, row=r, col=c):
        return L.mxfp4_quantize(x, rows, cols, block, sr, 1, rht, 1, row, col, None)
    assert q(row=None, col=None) == nv.ERR_NULL
    assert q(x=0) == nv.ERR_NULL
    assert q(block=16) == nv.ERR_GROUP
    assert q(sr=2) == nv.ERR_ARG
    assert q(cols=200) == nv.ERR_SHAPE                    # row layout needs cols % 32
    assert q(rows=160, cols=256, rht=1) == nv.ERR_SHAPE   # rotation needs rows % 128 (col)
    assert q(row=ctypes.byref(nv._CMx(FAKE + 8, FAKE))) == nv.ERR_ALIGN
    assert q(row=ctypes.byref(nv._CMx(FAKE, FAKE + 2))) == nv.ERR_ALIGN
    assert L.mxfp4_gemm(r, r, 64, 64, 64, 0, FAKE, None) == nv.ERR_SHAPE      # K % 128
    assert L.mxfp4_gemm(r, r, 48, 64, 128, 0, FAKE, None) == nv.ERR_SHAPE     # M % 32
    assert L.mxfp4_gemm(r, r, 64, 64, 128, 2, FAKE, None) == nv.ERR_ARG
    assert L.mxfp4_gemm(None, r, 64, 64, 128, 0, FAKE, None) == nv.ERR_NULL
    assert L.mxfp4_gemm(r, r, 64, 64, 128, 0, FAKE + 2, None) == nv.ERR_ALIGN


def test_mxfp4_k_tiled_validation(L):
    """The K-tiled flag: 0 or 1; a K-tiled layout needs n % 128 == 0 even without the
    rotation; the GEMM's operands must agree on it."""
    r = ctypes.byref(nv._CMx(FAKE, FAKE + 4096, 0))
    t = ctypes.byref(nv._CMx(FAKE, FAKE + 4096, 1))
    bad = ctypes.byref(nv._CMx(FAKE, FAKE + 4096, 2))

    def q(rows=256, cols=256, row=t, col=None):
        return L.mxfp4_quantize(FAKE, rows, cols, 32, 0, 1, 0, 1, row, col, None)
    assert q(row=bad) == nv.ERR_ARG
    assert q(cols=160) == nv.ERR_SHAPE                   # K-tiled row layout: cols % 128
    assert q(rows=96, row=None, col=t) == nv.ERR_SHAPE   # K-tiled column layout: rows % 128
    if not _has_gpu():                                   # never launch on fake pointers
        assert q(cols=160, row=r) == nv.ERR_HIP          # row-major only needs cols % 32
    assert L.mxfp4_gemm(r, t, 64, 64, 128, 0, FAKE, None) == nv.ERR_ARG
    assert L.mxfp4_gemm(t, r, 64, 64, 128, 0, FAKE, None) == nv.ERR_ARG
    assert L.mxfp4_gemm(bad, bad, 64, 64, 128, 0, FAKE, None) == nv.ERR_ARG
    assert L.mxfp4_gemm(t, t, 64, 64, 64, 0, FAKE, None) == nv.ERR_SHAPE     # K % 128
