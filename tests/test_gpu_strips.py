"""Strip-local ("CTA-local") scaling on the GPU against the oracle: each run of 128 vectors of a
layout has its own FP32 scale (rit.work note on "Format-Aware Fusion for Fast FP4
Pretraining", section "speedup is lost between matmuls": maxima inside a block of work, row
and column corrections applied after the GEMM's sum).  Codes, scales and every strip's g
bit-exact; the dequantizer bit-exact; the GEMM consumer within the FP32 accumulation bound of
the exact product, with the per-strip corrections."""
import numpy as np
import pytest
import torch

import oracle
import unbiased_nvfp4_gradient_amd as nv
import workloads
from gemm_ref import check_entries
from parity import assert_same_floats, compare

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_strips(mode, x, layouts, seed=1, rht=False, rht_seed=1):
    q = nv.nvfp4_quantize_strips(mode, x.to(DEV), seed=seed, rht=rht, rht_seed=rht_seed,
                                 layouts=layouts)
    torch.cuda.synchronize()
    return {axis: t for axis, t in ((0, q.row), (1, q.col)) if t is not None}


def check_strips(mode, x, layouts, seed=1, rht=False, rht_seed=1, margins=True, what=""):
    got = run_strips(mode, x, layouts, seed, rht, rht_seed)
    xb = workloads.bf16_bits(x)
    for axis, t in got.items():
        ref = oracle.quantize_strips(mode, xb, axis=axis, seed=seed, rht=rht, rht_seed=rht_seed,
                                     margins=margins)
        g = t.tensor_scale.cpu().numpy()
        assert g.shape == ref.g.shape, (what, axis)
        assert np.array_equal(g, ref.g), f"{what} axis={axis}: strip scales differ"
        codes, scales = t.codes.cpu().numpy(), t.scales.cpu().numpy()
        if margins:
            rep = compare(mode, codes, scales, ref)
            assert rep.ok(), f"{what} axis={axis}: {rep}"
        else:
            assert np.array_equal(codes, ref.codes), f"{what} axis={axis}: codes differ"
            assert np.array_equal(scales, ref.scales), f"{what} axis={axis}: scales differ"
    return got


MODES = [("rtn", False), ("sr", False), ("eden", True), ("fp46", False), ("rtn", True),
         ("sr", True), ("fp46", True)]


@pytest.mark.parametrize("mode,rht", MODES)
@pytest.mark.parametrize("layouts", [("row",), ("col",), ("row", "col")])
def test_config1_strips_all_modes(mode, rht, layouts):
    """c1 (256 x 1024): two row strips, eight column strips."""
    print(f"case: strips c1 mode={mode} rht={rht} layouts={layouts}", flush=True)
    check_strips(mode, workloads.c1(), layouts, seed=2, rht=rht, rht_seed=5,
                 what=f"c1 {mode} rht={rht}")


@pytest.mark.parametrize("shape,mode,rht,layouts", [
    ((300, 384), "eden", True, ("row",)),          # ragged last row strip (44 rows)
    ((256, 328), "eden", True, ("col",)),          # ragged last column strip (72 columns)
    ((304, 400), "rtn", False, ("row", "col")),    # ragged strips both ways, no rotation
    ((304, 400), "sr", False, ("row", "col")),
    ((144, 48), "fp46", False, ("row", "col")),    # tiny
    ((640, 384), "fp46", True, ("row", "col")),    # several strips both ways
    ((128, 128), "sr", True, ("row", "col")),      # one strip each way: the global method
])
def test_ragged_and_multi_strip(shape, mode, rht, layouts):
    print(f"case: strips shape={shape} mode={mode} rht={rht} layouts={layouts}", flush=True)
    x = workloads.c4(seed=sum(shape), shape=shape)   # column magnitudes vary: strips differ
    check_strips(mode, x, layouts, seed=9, rht=rht, rht_seed=4, what=f"{shape} {mode}")


def test_one_strip_equals_global_quantizer():
    print("case: strips vs global on one 128 x 128 tile", flush=True)
    x = workloads.normal((128, 128), seed=3).to(DEV)
    a = nv.nvfp4_quantize_strips("eden", x, seed=4, rht_seed=6)
    b = nv.eden_quantize(x, seed=4, rht_seed=6)
    torch.cuda.synchronize()
    for ta, tb in ((a.row, b.row), (a.col, b.col)):
        assert torch.equal(ta.codes, tb.codes) and torch.equal(ta.scales, tb.scales)
        assert torch.equal(ta.tensor_scale, tb.tensor_scale)


def test_strip_scale_isolation():
    """A strip 2^-24 below the rest keeps its resolution (the global scale loses it)."""
    print("case: strips, one strip scaled by 2^-24", flush=True)
    x = workloads.normal((384, 256), seed=8).float()
    x[128:256] *= 2.0 ** -24
    x = x.to(torch.bfloat16)
    got = check_strips("eden", x, ("row",), seed=3, rht_seed=2, what="isolation")
    back = nv.dequantize_strips(got[0], rht=True, rht_seed=2).cpu().double().numpy()
    xf = x.double().numpy()
    for s in range(3):
        sl = slice(128 * s, 128 * s + 128)
        rel = ((back[sl] - xf[sl]) ** 2).sum() / (xf[sl] ** 2).sum()
        assert rel < 0.02, (s, rel)


def test_zero_and_empty_strips():
    print("case: strips zeros 256x384 and empty 0x256 / 256x0", flush=True)
    check_strips("eden", torch.zeros((256, 384), dtype=torch.bfloat16), ("row", "col"),
                 what="zeros")
    for shape, layouts in (((0, 256), ("col",)), ((256, 0), ("row",))):
        x = torch.zeros(shape, dtype=torch.bfloat16, device=DEV)
        q = nv.nvfp4_quantize_strips("eden", x, seed=1, rht_seed=1, layouts=layouts)
        torch.cuda.synchronize()
        t = q.row if q.row is not None else q.col
        assert t.tensor_scale.shape == (2,) and not t.tensor_scale.any()
        assert t.codes.numel() == 0


def test_config3_strips_both_layouts():
    """c3 (16384 x 2048, rows whose magnitudes span 10^-6..10), all outputs compared."""
    print("case: strips c3 eden both layouts (full compare)", flush=True)
    check_strips("eden", workloads.c3(), ("row", "col"), seed=1, rht_seed=1, margins=False,
                 what="c3")


def test_config4_strips_both_layouts():
    """c4 (16384 x 8192): 128 row strips and 64 column strips, all outputs compared."""
    print("case: strips c4 eden both layouts (full compare)", flush=True)
    check_strips("eden", workloads.c4(), ("row", "col"), seed=1, rht_seed=1, margins=False,
                 what="c4")


@pytest.mark.parametrize("mode,rht", [("eden", True), ("rtn", False), ("fp46", True)])
def test_dequantize_strips_parity(mode, rht):
    print(f"case: dequantize_strips {mode} rht={rht}", flush=True)
    x = workloads.c4(seed=5, shape=(384, 256))
    got = check_strips(mode, x, ("row", "col"), seed=2, rht=rht, rht_seed=3, what="dequant")
    rot = rht or mode == "eden"
    for axis, t in got.items():
        out = nv.dequantize_strips(t, rht=rot, rht_seed=3)
        torch.cuda.synchronize()
        ref = oracle.dequantize_strips(t.codes.cpu().numpy(), t.scales.cpu().numpy(),
                                       t.tensor_scale.cpu().numpy(), rht=rot, rht_seed=3)
        assert_same_floats(out.cpu().numpy(), ref, f"{mode} axis={axis}", zero_sign_free=rot)


@pytest.mark.parametrize("M,N,K", [(384, 256, 512), (96, 160, 256), (256, 640, 128)])
def test_gemm_strips(M, N, K):
    """C = f gA[m/128] gB[n/128] sum_k a b: per-strip corrections after the sum over K."""
    print(f"case: gemm strips M={M} N={N} K={K}", flush=True)
    x = workloads.c4(seed=M, shape=(M, K))
    w = workloads.normal((N, K), seed=N + K, scale=0.02).float()
    w[: min(N, 128)] *= 64.0                       # strips of very different magnitude
    w = w.to(torch.bfloat16)
    a = nv.nvfp4_quantize_strips("eden", x.to(DEV), seed=3, rht_seed=9, layouts=("row",)).row
    b = nv.nvfp4_quantize_strips("fp46", w.to(DEV), rht=True, rht_seed=9, layouts=("row",)).row
    c = nv.nvfp4_gemm_check_strips(a, b, rotated_pair=True)
    torch.cuda.synchronize()
    assert a.tensor_scale.shape == (-(-M // 128),) and b.tensor_scale.shape == (-(-N // 128),)
    got, _ = check_entries(c, a, b, np.arange(M), np.arange(N), 2.0 ** -7, strips=True)
    xw = (x.double() @ w.double().T).numpy()
    rel = np.linalg.norm(got - xw) / np.linalg.norm(xw)
    assert rel < 0.2, rel
