"""Guard bytes around GPU output buffers: each output tensor is a view into the middle of a
larger allocation whose margins hold a sentinel, so a write past either end of any output
(codes, scales or tensor scale) shows up as a changed margin."""
import torch

import unbiased_nvfp4_gradient_amd as nv

MARGIN = 4096           # bytes before and after each output; keeps every view 256-byte aligned
SENTINEL = 0xA7


class Guarded:
    def __init__(self, vecs: int, n: int, device, scales_per_layout: int = 1):
        self._bufs = []
        codes = self._alloc(vecs * (n // 2), device).view(vecs, n // 2)
        scales = self._alloc(vecs * (n // 16), device).view(vecs, n // 16)
        g = self._alloc(4 * scales_per_layout, device).view(torch.float32)
        self.layout = nv.NVFP4(codes, scales, g)

    def _alloc(self, nbytes, device):
        buf = torch.full((MARGIN + nbytes + MARGIN,), SENTINEL, dtype=torch.uint8,
                         device=device)
        self._bufs.append((buf, nbytes))
        return buf[MARGIN:MARGIN + nbytes]

    def intact(self) -> bool:
        for buf, nbytes in self._bufs:
            if not bool((buf[:MARGIN] == SENTINEL).all()):
                return False
            if not bool((buf[MARGIN + nbytes:] == SENTINEL).all()):
                return False
        return True


def guarded_outputs(rows, cols, layouts, device, strips=False):
    """nv.Quantized outputs wrapped in guard margins, and the guards to check."""
    per = (lambda v: (v + 127) // 128) if strips else (lambda v: 1)
    row = Guarded(rows, cols, device, per(rows)) if "row" in layouts else None
    col = Guarded(cols, rows, device, per(cols)) if "col" in layouts else None
    out = nv.Quantized(row.layout if row else None, col.layout if col else None)
    return out, [g for g in (row, col) if g is not None]
