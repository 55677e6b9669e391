"""Quartet II linear layer: every product of a linear layer's forward and backward pass on
NVFP4 operands, built from this package's quantizers and its MFMA GEMM consumer.

The Quartet II summaries (itsolotime.com, abstract; Telegram digest quant_prune_distill
post 640, "Method") describe a fully NVFP4 linear layer whose products give better, unbiased
gradient estimates in the forward and the backward pass: the forward quantizes with the 4/6
choice, the backward with MS-EDEN, and Fig. 9 of the itsolotime summary checks that the mean
of many quantized backward passes converges to the unquantized one as 1/B.

With X [T, in], W [out, in] and Y = X W^T:
  forward   Y  = Q46(X) Q46(W)^T          contraction over in:  X rows, W rows
  backward  dX = Qb(dY) Qb(W)             contraction over out: dY rows, W columns
            dW = Qb(dY)^T Qb(X)           contraction over T:   dY columns, X columns
Each product's two operands share a random-sign Hadamard rotation along the contraction
dimension (the product of the rotated operands is 128 times the unrotated one, which the
GEMM undoes), and every operand draws its own stochastic rounding.  Qb is MS-EDEN; plain SR,
RTN and 4/6 are available as backward schemes for comparison.  Three NVFP4 GEMMs and five
quantizer calls per step run in this package's HIP kernels; this module only orders them.

Seeds: a call with seed s uses rotation seed 2s in the forward and 2s + 1 in the backward,
and stochastic-rounding seeds 3s, 3s + 1, 3s + 2 for dY, W and X.  All three dimensions
must be multiples of 128 (rotation groups); the GEMM needs M, N % 32 and K % 64, implied.

scales="strip" switches every operand to strip-local scales (the CTA-local variant of the
rit.work note on "Format-Aware Fusion for Fast FP4 Pretraining"): one FP32 scale per 128
vectors of each operand, i.e. per block of 128 rows of the product's first operand and 128
columns of its second, which the GEMM applies after its sum over K.  Every operand's strips
run along a dimension that is not contracted, so each product keeps one correction per
output row block and one per output column block.

scales="mx" runs the layer on the native FP4 recipe instead (the same note's "fast route":
MXFP4, one power-of-two scale per 32 elements, a Hadamard transform and stochastic rounding):
every operand is MXFP4 in the K-tiled layout, the forward rounds to nearest, the backward
uses the scheme "sr" (unbiased) or "rtn", and the three products run on the FP4 matrix
cores (mxfp4_gemm).  Rotation and rounding seeds are those above.
"""
from __future__ import annotations

import torch

from . import (eden_quantize, fp46_quantize, mxfp4_gemm, mxfp4_quantize, nvfp4_gemm_check,
               nvfp4_gemm_check_strips, nvfp4_quantize_strips, rtn_quantize, sr_quantize)

BACKWARD_SCHEMES = ("eden", "sr", "rtn", "fp46")
MX_BACKWARD_SCHEMES = ("sr", "rtn")
SCALES = ("tensor", "strip", "mx")


def _gemm(scales: str):
    if scales not in SCALES:
        raise ValueError(f"unknown scales {scales!r}; use one of {SCALES}")
    if scales == "mx":
        return mxfp4_gemm
    return nvfp4_gemm_check_strips if scales == "strip" else nvfp4_gemm_check


def _quantize(scheme: str, x: torch.Tensor, seed: int, rht_seed: int, layouts,
              scales: str = "tensor"):
    if scales == "mx":
        if scheme not in MX_BACKWARD_SCHEMES:
            raise ValueError(f"scheme {scheme!r} has no MXFP4 form; use one of "
                             f"{MX_BACKWARD_SCHEMES}")
        return mxfp4_quantize(x, sr=scheme == "sr", seed=seed, rht=True, rht_seed=rht_seed,
                              layouts=layouts, k_tiled=True)
    if scales == "strip":
        if scheme not in BACKWARD_SCHEMES:
            raise ValueError(f"unknown scheme {scheme!r}; use one of {BACKWARD_SCHEMES}")
        return nvfp4_quantize_strips(scheme, x, seed=seed, rht=True, rht_seed=rht_seed,
                                     layouts=layouts)
    if scheme == "eden":
        return eden_quantize(x, seed, rht_seed, layouts=layouts)
    if scheme == "sr":
        return sr_quantize(x, seed, rht=True, rht_seed=rht_seed, layouts=layouts)
    if scheme == "rtn":
        return rtn_quantize(x, rht=True, rht_seed=rht_seed, layouts=layouts)
    if scheme == "fp46":
        return fp46_quantize(x, rht=True, rht_seed=rht_seed, layouts=layouts)
    raise ValueError(f"unknown backward scheme {scheme!r}; use one of {BACKWARD_SCHEMES}")


def _check_shapes(x: torch.Tensor, w: torch.Tensor):
    if x.dim() != 2 or w.dim() != 2 or x.shape[1] != w.shape[1]:
        raise ValueError(f"need x [T, in] and w [out, in], got {tuple(x.shape)} and "
                         f"{tuple(w.shape)}")
    for name, n in (("T", x.shape[0]), ("in", x.shape[1]), ("out", w.shape[0])):
        if n % 128:
            raise ValueError(f"{name} = {n} must be a multiple of 128")
    if x.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
        raise ValueError("x and w must be bfloat16")


def forward_product(x: torch.Tensor, w: torch.Tensor, seed: int, operands: bool = False,
                    scales: str = "tensor"):
    """Y = Q46(X) Q46(W)^T in FP32 (round-to-nearest MXFP4 with scales="mx"), X and W rotated
    along in with rotation seed 2s.  With operands=True also returns the two quantized
    operands (X rows, W rows)."""
    gemm = _gemm(scales)
    rs = 2 * seed
    fwd = "rtn" if scales == "mx" else "fp46"
    qx = _quantize(fwd, x, 0, rs, ("row",), scales).row
    qw = _quantize(fwd, w, 0, rs, ("row",), scales).row
    y = gemm(qx, qw, rotated_pair=True)
    return (y, (qx, qw)) if operands else y


def backward_products(dy: torch.Tensor, x: torch.Tensor, w: torch.Tensor, seed: int,
                      scheme: str = "eden", operands: bool = False, scales: str = "tensor"):
    """(dX, dW) in FP32 from bfloat16 dY [T, out], X [T, in], W [out, in].  With
    operands=True also returns the quantized operands (dY rows, W columns, dY columns,
    X columns)."""
    gemm = _gemm(scales)
    rs = 2 * seed + 1
    qdy = _quantize(scheme, dy, 3 * seed, rs, ("row", "col"), scales)
    qw = _quantize(scheme, w, 3 * seed + 1, rs, ("col",), scales).col
    qx = _quantize(scheme, x, 3 * seed + 2, rs, ("col",), scales).col
    dx = gemm(qdy.row, qw, rotated_pair=True)
    dw = gemm(qdy.col, qx, rotated_pair=True)
    return ((dx, dw), (qdy.row, qw, qdy.col, qx)) if operands else (dx, dw)


class QuartetLinearFunction(torch.autograd.Function):
    """Y = X W^T with NVFP4 products (no bias), Y in FP32.  dY is rounded to bfloat16, the
    quantizers' input format; the gradients are returned in the dtypes of X and W."""

    @staticmethod
    def forward(ctx, x, w, seed: int, scheme: str = "eden", scales: str = "tensor"):
        if scales == "mx" and scheme not in MX_BACKWARD_SCHEMES:
            raise ValueError(f"scheme {scheme!r} has no MXFP4 form")
        _check_shapes(x, w)
        x, w = x.contiguous(), w.contiguous()
        ctx.save_for_backward(x, w)
        ctx.seed, ctx.scheme, ctx.scales = int(seed), scheme, scales
        return forward_product(x, w, int(seed), scales=scales)

    @staticmethod
    def backward(ctx, dy):
        x, w = ctx.saved_tensors
        dyb = dy.to(torch.bfloat16).contiguous()
        dx, dw = backward_products(dyb, x, w, ctx.seed, ctx.scheme, scales=ctx.scales)
        return dx.to(x.dtype), dw.to(w.dtype), None, None, None


class QuartetLinear(torch.nn.Module):
    """A bias-free linear layer whose products run on NVFP4 operands.  Each call draws a new
    seed (a counter started at `seed`), so repeated steps use fresh rotations and roundings."""

    def __init__(self, in_features: int, out_features: int, seed: int = 0,
                 scheme: str = "eden", device=None, scales: str = "tensor"):
        super().__init__()
        if scheme not in BACKWARD_SCHEMES:
            raise ValueError(f"unknown backward scheme {scheme!r}")
        if scales not in SCALES:
            raise ValueError(f"unknown scales {scales!r}")
        if scales == "mx" and scheme not in MX_BACKWARD_SCHEMES:
            raise ValueError(f"scheme {scheme!r} has no MXFP4 form; use one of "
                             f"{MX_BACKWARD_SCHEMES}")
        self.scales = scales
        self.weight = torch.nn.Parameter(torch.empty(
            (out_features, in_features), dtype=torch.bfloat16, device=device))
        torch.nn.init.normal_(self.weight, std=0.02)
        self.scheme = scheme
        self._seed = int(seed)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        s = self._seed
        self._seed += 1
        return QuartetLinearFunction.apply(x, self.weight, s, self.scheme, self.scales)
