"""The binding's choice of layouts when the caller brings its own outputs (host logic only:
nothing here reaches the library)."""
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
    ws = torch.empty(1, dtype=torch.uint8)
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
        nv._allocate(x, ("row", "col"), out, torch.empty(1, dtype=torch.uint8))
