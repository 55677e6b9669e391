"""eden_quantize_noalloc, the entry point that allocates nothing, against eden_quantize (the
same quantizer with a caller workspace), called through the C ABI: two calls in a row, the
second on a smaller input, each compared bit for bit (codes, scales, tensor scales of both
layouts).  The library's device scratch keeps the first call's contents when the second one
starts, so the second comparison also checks that nothing stale is read."""
import ctypes

import numpy as np
import pytest
import torch

import unbiased_nvfp4_gradient_amd as nv
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _noalloc_c_abi(x, seed, rht_seed, out):
    """Call the C entry point directly with ctypes: device pointers, sizes, the stream."""
    L = nv.lib()
    rows, cols = x.shape
    row = nv._CTensor(out.row.codes.data_ptr(), out.row.scales.data_ptr(),
                      out.row.tensor_scale.data_ptr())
    col = nv._CTensor(out.col.codes.data_ptr(), out.col.scales.data_ptr(),
                      out.col.tensor_scale.data_ptr())
    return L.eden_quantize_noalloc(x.data_ptr(), rows, cols, 128, 16, seed, rht_seed,
                                   ctypes.byref(row), ctypes.byref(col),
                                   torch.cuda.current_stream(DEV).cuda_stream)


@pytest.mark.parametrize("first,second", [((2048, 4096), (384, 640)),
                                          ((16384, 8192), (256, 1024))])
def test_noalloc_matches_eden_quantize(first, second):
    for k, shape in enumerate((first, second)):
        print(f"case: eden_quantize_noalloc call {k + 1}, {shape}", flush=True)
        x = workloads.c4(seed=k + 3, shape=shape).to(DEV)
        rows, cols = shape
        out = nv.Quantized(nv.empty_layout(rows, cols, DEV), nv.empty_layout(cols, rows, DEV))
        for t in out:
            t.codes.fill_(0xEE)
            t.scales.fill_(0xEE)
            t.tensor_scale.fill_(-1.0)
        assert _noalloc_c_abi(x, 11 + k, 5 + k, out) == 0
        ref = nv.eden_quantize(x, 11 + k, 5 + k, layouts=("row", "col"))
        torch.cuda.synchronize()
        for lay in ("row", "col"):
            a, b = getattr(out, lay), getattr(ref, lay)
            assert torch.equal(a.tensor_scale, b.tensor_scale), (shape, lay)
            for f in ("codes", "scales"):
                ga, gb = getattr(a, f).cpu().numpy(), getattr(b, f).cpu().numpy()
                assert np.array_equal(ga, gb), (shape, lay, f, int((ga != gb).sum()))


def test_noalloc_one_layout_and_errors():
    print("case: eden_quantize_noalloc one layout, rejected shapes", flush=True)
    x = workloads.normal((256, 384), seed=9).to(DEV)
    got = nv.eden_quantize_noalloc(x, 3, 4, layouts=("col",))
    ref = nv.eden_quantize(x, 3, 4, layouts=("col",))
    torch.cuda.synchronize()
    assert got.row is None
    for f in ("codes", "scales", "tensor_scale"):
        assert torch.equal(getattr(got.col, f), getattr(ref.col, f)), f
    bad = workloads.normal((256, 200), seed=9).to(DEV)          # n % 128 != 0
    with pytest.raises(nv.NVFP4Error) as e:
        nv.eden_quantize_noalloc(bad, 1, 1, layouts=("row",))
    assert e.value.status == nv.ERR_SHAPE
