"""The binding's host logic (nothing here reaches a GPU): the choice of layouts when the
caller brings its own outputs, and the checks of every caller-supplied buffer (dtype, shape,
device, contiguity, size), which must raise before anything is launched."""
import pytest
import torch

import unbiased_nvfp4_gradient_amd as nv


def layout(vecs, n):
    return nv.NVFP4(torch.empty((vecs, n // 2), dtype=torch.uint8),
                    torch.empty((vecs, n // 16), dtype=torch.uint8),
                    torch.empty((1,), dtype=torch.float32))


def test_only_requested_layouts_are_passed():
    out = nv.Quantized(layout(32, 64), layout(64, 32))
    x = torch.empty((32, 64), dtype=torch.bfloat16)
    ws = torch.empty(nv.workspace_bytes(32, 64), dtype=torch.uint8)
    for layouts, row, col in ((("row",), True, False), (("col",), False, True),
                              (("row", "col"), True, True)):
        _, _, sel, w = nv._allocate(x, layouts, out, ws)
        assert (sel.row is out.row) == row and (sel.row is None) == (not row)
        assert (sel.col is out.col) == col and (sel.col is None) == (not col)
        assert w is ws


def test_missing_requested_layout_raises():
    out = nv.Quantized(layout(32, 64), None)
    x = torch.empty((32, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        nv._allocate(x, ("row", "col"), out,
                     torch.empty(nv.workspace_bytes(32, 64), dtype=torch.uint8))


def _ws(rows=32, cols=64):
    return torch.empty(nv.workspace_bytes(rows, cols), dtype=torch.uint8)


@pytest.mark.parametrize("bad", [
    lambda: nv.NVFP4(torch.empty((32, 31), dtype=torch.uint8),      # codes one byte short
                     torch.empty((32, 4), dtype=torch.uint8), torch.empty(1)),
    lambda: nv.NVFP4(torch.empty((32, 32), dtype=torch.uint8),
                     torch.empty((32, 3), dtype=torch.uint8), torch.empty(1)),   # scales short
    lambda: nv.NVFP4(torch.empty((32, 32), dtype=torch.int16),      # wrong dtype
                     torch.empty((32, 4), dtype=torch.uint8), torch.empty(1)),
    lambda: nv.NVFP4(torch.empty((32, 32), dtype=torch.uint8),
                     torch.empty((32, 4), dtype=torch.uint8),
                     torch.empty(1, dtype=torch.bfloat16)),          # tensor scale dtype
    lambda: nv.NVFP4(torch.empty((32, 32), dtype=torch.uint8),
                     torch.empty((32, 4), dtype=torch.uint8), torch.empty(2)),   # two scales
    lambda: nv.NVFP4(torch.empty((32, 64), dtype=torch.uint8)[:, ::2],          # strided
                     torch.empty((32, 4), dtype=torch.uint8), torch.empty(1)),
    lambda: (torch.empty((32, 32), dtype=torch.uint8), torch.empty((32, 4), dtype=torch.uint8)),
])
def test_bad_output_buffers_raise(bad):
    x = torch.empty((32, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        nv._allocate(x, ("row",), nv.Quantized(bad(), None), _ws())


def test_good_output_buffers_pass():
    x = torch.empty((32, 64), dtype=torch.bfloat16)
    out = nv.Quantized(layout(32, 64), layout(64, 32))
    _, _, sel, _ = nv._allocate(x, ("row", "col"), out, _ws())
    assert sel.row.codes is out.row.codes and sel.col.scales is out.col.scales


def test_bad_workspace_raises():
    x = torch.empty((32, 64), dtype=torch.bfloat16)
    out = nv.Quantized(layout(32, 64), None)
    need = nv.workspace_bytes(32, 64)
    for ws in (torch.empty(need - 1, dtype=torch.uint8),            # too small
               torch.empty(need // 4, dtype=torch.float32),         # right bytes, wrong type
               torch.empty((2, need), dtype=torch.uint8)):          # not 1-D
        with pytest.raises(ValueError):
            nv._allocate(x, ("row",), out, ws)


def test_strip_outputs_need_one_scale_per_strip():
    x = torch.empty((300, 256), dtype=torch.bfloat16)
    good = nv.empty_strip_layout(300, 256, "cpu")
    assert good.tensor_scale.shape == (3,)
    assert nv._check_outputs(x, nv.Quantized(good, None), strips=True).row is not None
    with pytest.raises(ValueError):            # a per-tensor layout has one scale, not three
        nv._check_outputs(x, nv.Quantized(layout(300, 256), None), strips=True)


def test_decoders_check_their_inputs_and_outputs():
    t = layout(32, 64)
    with pytest.raises(ValueError):            # output one row short
        nv.dequantize(t, out=torch.empty((31, 64)))
    with pytest.raises(ValueError):            # output of the wrong type
        nv.dequantize(t, out=torch.empty((32, 64), dtype=torch.float64))
    with pytest.raises(ValueError):            # per-tensor scale given to the strip decoder
        nv.dequantize_strips(layout(300, 64))
    bad = nv.NVFP4(t.codes, torch.empty((32, 5), dtype=torch.uint8), t.tensor_scale)
    with pytest.raises(ValueError):            # scales disagree with the codes
        nv.dequantize(bad)


def test_gemm_checks_operands_and_output():
    a, b = layout(64, 128), layout(32, 128)
    with pytest.raises(ValueError):
        nv.nvfp4_gemm_check(a, layout(32, 256))            # K differs
    with pytest.raises(ValueError):
        nv.nvfp4_gemm_check(a, b, out=torch.empty((64, 31)))
    with pytest.raises(ValueError):                        # per-tensor scales, 3 strips
        nv.nvfp4_gemm_check_strips(layout(320, 128), b)


def test_phase_buffers_checked():
    x = torch.empty((32, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        nv._check_buffer(torch.empty(1), "amax", torch.float32, (2,), x.device)
    nv._check_buffer(torch.empty(2), "amax", torch.float32, (2,), x.device)
