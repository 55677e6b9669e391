"""Quartet II linear layer (forward 4/6, backward MS-EDEN, the products on the MFMA GEMM
consumer): every quantized operand against the oracle, bit for bit; every product against
the exact product of its operands within the FP32 accumulation bound; and the Fig. 9 method
of the itsolotime summary (Q1): the mean of B quantized backward passes converges to the
unquantized gradient as 1/B when the backward scheme is unbiased (MS-EDEN, SR) and plateaus
when it is deterministic (RTN, 4/6 with the rotation).

Inputs stand in for one linear layer's tensors in a training step: X ~ N(0,1),
W ~ N(0, 0.02), dY ~ N(0,1), BF16, numpy seeds."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gemm_ref import check_entries, check_mx_entries
from parity import assert_parity
from unbiased_nvfp4_gradient_amd import linear

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def layer_inputs(t, n_in, n_out, seed):
    x = workloads.normal((t, n_in), seed=seed)
    w = workloads.normal((n_out, n_in), seed=seed + 1, scale=0.02)
    dy = workloads.normal((t, n_out), seed=seed + 2)
    return x, w, dy


def _operand_parity(mode, q, x_cpu, axis, seed, rht_seed, what):
    ref = oracle.quantize(mode, workloads.bf16_bits(x_cpu), axis=axis, seed=seed, rht=True,
                          rht_seed=rht_seed)
    assert_parity(mode, q.codes.cpu().numpy(), q.scales.cpu().numpy(),
                  float(q.tensor_scale.cpu()[0]), ref, what)


@pytest.mark.parametrize("t,n_in,n_out", [(256, 256, 384), (384, 512, 128)])
def test_layer_operands_and_products(t, n_in, n_out):
    print(f"case: linear layer T={t} in={n_in} out={n_out}", flush=True)
    x, w, dy = layer_inputs(t, n_in, n_out, seed=t + n_in)
    xd, wd, dyd = x.to(DEV), w.to(DEV), dy.to(DEV)
    s = 7
    y, (qx, qw) = linear.forward_product(xd, wd, s, operands=True)
    (dx, dw), (qdy_r, qw_c, qdy_c, qx_c) = linear.backward_products(dyd, xd, wd, s, "eden",
                                                                    operands=True)
    torch.cuda.synchronize()
    _operand_parity("fp46", qx, x, 0, 0, 2 * s, "X rows")
    _operand_parity("fp46", qw, w, 0, 0, 2 * s, "W rows")
    _operand_parity("eden", qdy_r, dy, 0, 3 * s, 2 * s + 1, "dY rows")
    _operand_parity("eden", qdy_c, dy, 1, 3 * s, 2 * s + 1, "dY columns")
    _operand_parity("eden", qw_c, w, 1, 3 * s + 1, 2 * s + 1, "W columns")
    _operand_parity("eden", qx_c, x, 1, 3 * s + 2, 2 * s + 1, "X columns")
    f = 2.0 ** -7                    # both operands of every product carry the rotation
    check_entries(y, qx, qw, np.arange(t), np.arange(n_out), f)
    check_entries(dx, qdy_r, qw_c, np.arange(t), np.arange(n_in), f)
    check_entries(dw, qdy_c, qx_c, np.arange(n_out), np.arange(n_in), f)
    xf, wf, dyf = x.double().numpy(), w.double().numpy(), dy.double().numpy()
    for name, got, ex in (("Y", y, xf @ wf.T), ("dX", dx, dyf @ wf), ("dW", dw, dyf.T @ xf)):
        rel = np.linalg.norm(got.cpu().double().numpy() - ex) / np.linalg.norm(ex)
        print(f"{name}: relative error {rel:.4f}", flush=True)
        assert rel < 0.25, (name, rel)


@pytest.mark.parametrize("scheme,scales", [("eden", "tensor"), ("sr", "mx")])
def test_autograd_module(scheme, scales):
    print(f"case: QuartetLinear forward + backward through autograd, {scheme}/{scales}",
          flush=True)
    t, n_in, n_out = 256, 384, 256
    x, _, dy = layer_inputs(t, n_in, n_out, seed=40)
    layer = linear.QuartetLinear(n_in, n_out, seed=11, device=DEV, scheme=scheme, scales=scales)
    with torch.no_grad():
        layer.weight.copy_(workloads.normal((n_out, n_in), seed=41, scale=0.02).to(DEV))
    xd = x.to(DEV).requires_grad_(True)
    y = layer(xd)
    assert y.shape == (t, n_out) and y.dtype == torch.float32
    y.backward(dy.to(DEV).float())
    assert xd.grad.dtype == torch.bfloat16 and layer.weight.grad.dtype == torch.bfloat16
    wf = layer.weight.detach().double().cpu().numpy()
    dyf, xf = dy.double().numpy(), x.double().numpy()
    for name, got, ex in (("dX", xd.grad, dyf @ wf), ("dW", layer.weight.grad, dyf.T @ xf)):
        g = got.double().cpu().numpy()
        assert np.isfinite(g).all()
        rel = np.linalg.norm(g - ex) / np.linalg.norm(ex)
        assert rel < 0.3, (name, rel)
    with pytest.raises(ValueError):
        layer(torch.zeros((100, n_in), dtype=torch.bfloat16, device=DEV))
    if scales == "mx":
        with pytest.raises(ValueError):
            linear.QuartetLinear(n_in, n_out, scheme="eden", scales="mx")


def _gradient_curve(scheme, xd, wd, dyd, exact, b_max):
    """Relative squared error of the mean of b backward passes (seeds 1..b) for b a power
    of two, and the mean single-pass error divided by b."""
    acc = [torch.zeros_like(e) for e in exact]
    norms = [float((e * e).sum()) for e in exact]
    single = [0.0, 0.0]
    pts = {}
    for b in range(1, b_max + 1):
        grads = linear.backward_products(dyd, xd, wd, b, scheme)
        for i, g in enumerate(grads):
            g = g.double()
            acc[i] += g
            single[i] += float(((g - exact[i]) ** 2).sum()) / norms[i]
        if b & (b - 1) == 0:
            pts[b] = [(float(((acc[i] / b - exact[i]) ** 2).sum()) / norms[i], single[i] / b / b)
                      for i in range(2)]
    return pts


def test_fig9_gradient_mean_converges_as_1_over_b():
    print("case: Fig. 9 method on a 512 x 256 -> 256 layer, B = 1..1024", flush=True)
    t, n_in, n_out = 512, 256, 256
    x, w, dy = layer_inputs(t, n_in, n_out, seed=50)
    xd, wd, dyd = x.to(DEV), w.to(DEV), dy.to(DEV)
    exact = [dyd.double() @ wd.double(), dyd.double().t() @ xd.double()]   # dX, dW
    b_max = 1024
    for scheme in ("eden", "sr"):
        pts = _gradient_curve(scheme, xd, wd, dyd, exact, b_max)
        for i, name in enumerate(("dX", "dW")):
            print(scheme, name, {b: f"{v[i][0]:.2e}/{v[i][1]:.2e}" for b, v in pts.items()},
                  flush=True)
            for b, v in pts.items():
                bias, expect = v[i]
                assert 0.7 * expect < bias < 1.4 * expect, (scheme, name, b, bias, expect)
            slope = np.log(pts[b_max][i][0] / pts[1][i][0]) / np.log(b_max)
            assert -1.1 < slope < -0.9, (scheme, name, slope)
    for scheme in ("rtn", "fp46"):                # deterministic given the rotation
        pts = _gradient_curve(scheme, xd, wd, dyd, exact, b_max)
        for i, name in enumerate(("dX", "dW")):
            print(scheme, name, {b: f"{v[i][0]:.2e}/{v[i][1]:.2e}" for b, v in pts.items()},
                  flush=True)
            bias, expect = pts[b_max][i]
            assert bias > 2.0 * expect, (scheme, name, bias, expect)


# ----------------------------------------------------------------------------- strip-local scales

def _strip_parity(mode, q, x_cpu, axis, seed, rht_seed, what):
    ref = oracle.quantize_strips(mode, workloads.bf16_bits(x_cpu), axis=axis, seed=seed,
                                 rht=True, rht_seed=rht_seed, margins=False)
    assert np.array_equal(q.tensor_scale.cpu().numpy(), ref.g), what
    assert np.array_equal(q.codes.cpu().numpy(), ref.codes), what
    assert np.array_equal(q.scales.cpu().numpy(), ref.scales), what


def test_layer_with_strip_scales():
    """The layer with strip-local scales on every operand: operands bit-exact against the
    oracle's strip quantizer, products within the FP32 bound with per-strip corrections."""
    t, n_in, n_out = 384, 256, 512
    print(f"case: linear layer, strip scales, T={t} in={n_in} out={n_out}", flush=True)
    x, w, dy = layer_inputs(t, n_in, n_out, seed=60)
    xd, wd, dyd = x.to(DEV), w.to(DEV), dy.to(DEV)
    s = 5
    y, (qx, qw) = linear.forward_product(xd, wd, s, operands=True, scales="strip")
    (dx, dw), (qdy_r, qw_c, qdy_c, qx_c) = linear.backward_products(
        dyd, xd, wd, s, "eden", operands=True, scales="strip")
    torch.cuda.synchronize()
    _strip_parity("fp46", qx, x, 0, 0, 2 * s, "X rows")
    _strip_parity("fp46", qw, w, 0, 0, 2 * s, "W rows")
    _strip_parity("eden", qdy_r, dy, 0, 3 * s, 2 * s + 1, "dY rows")
    _strip_parity("eden", qdy_c, dy, 1, 3 * s, 2 * s + 1, "dY columns")
    _strip_parity("eden", qw_c, w, 1, 3 * s + 1, 2 * s + 1, "W columns")
    _strip_parity("eden", qx_c, x, 1, 3 * s + 2, 2 * s + 1, "X columns")
    f = 2.0 ** -7
    check_entries(y, qx, qw, np.arange(t), np.arange(n_out), f, strips=True)
    check_entries(dx, qdy_r, qw_c, np.arange(t), np.arange(n_in), f, strips=True)
    check_entries(dw, qdy_c, qx_c, np.arange(n_out), np.arange(n_in), f, strips=True)


def test_fig9_with_strip_scales():
    """Strip-local MS-EDEN stays unbiased in the layer: the mean of B backward passes tracks
    mse/B out to B = 256."""
    print("case: Fig. 9 method with strip scales, 512 x 256 -> 256, B = 1..256", flush=True)
    t, n_in, n_out = 512, 256, 256
    x, w, dy = layer_inputs(t, n_in, n_out, seed=70)
    xd, wd, dyd = x.to(DEV), w.to(DEV), dy.to(DEV)
    exact = [dyd.double() @ wd.double(), dyd.double().t() @ xd.double()]
    acc = [torch.zeros_like(e) for e in exact]
    norms = [float((e * e).sum()) for e in exact]
    single = [0.0, 0.0]
    for b in range(1, 257):
        grads = linear.backward_products(dyd, xd, wd, b, "eden", scales="strip")
        for i, g in enumerate(grads):
            g = g.double()
            acc[i] += g
            single[i] += float(((g - exact[i]) ** 2).sum()) / norms[i]
        if b in (1, 16, 256):
            for i, name in enumerate(("dX", "dW")):
                bias = float(((acc[i] / b - exact[i]) ** 2).sum()) / norms[i]
                expect = single[i] / b / b
                print(name, b, f"{bias:.3e}/{expect:.3e}", flush=True)
                assert 0.7 * expect < bias < 1.4 * expect, (name, b, bias, expect)


# ----------------------------------------------------------------------------- the MXFP4 recipe

def _mx_operand(q, x_cpu, axis, sr, seed, rht_seed, what):
    """A K-tiled MXFP4 operand against the oracle's quantization, rearranged by the layout's
    definition; returns the oracle's row-major codes and scales."""
    ref = oracle.mx_quantize(workloads.bf16_bits(x_cpu), axis=axis, sr=sr, seed=seed, rht=True,
                             rht_seed=rht_seed)
    tc, ts = oracle.mx_k_tile(ref.codes, ref.scales)
    assert q.k_tiled, what
    assert np.array_equal(q.codes.cpu().numpy(), tc), what
    assert np.array_equal(q.scales.cpu().numpy(), ts), what
    return ref.codes, ref.scales


def test_layer_mxfp4_recipe():
    """scales="mx": every operand K-tiled MXFP4, bit-exact against the oracle (forward RTN,
    backward SR, the layer's seeds), and every entry of the three products on the FP4 matrix
    cores against the exact product of its operands within the FP32 bound."""
    t, n_in, n_out = 256, 384, 128
    print(f"case: linear layer, MXFP4 recipe, T={t} in={n_in} out={n_out}", flush=True)
    x, w, dy = layer_inputs(t, n_in, n_out, seed=80)
    xd, wd, dyd = x.to(DEV), w.to(DEV), dy.to(DEV)
    s = 3
    y, (qx, qw) = linear.forward_product(xd, wd, s, operands=True, scales="mx")
    (dx, dw), (qdy_r, qw_c, qdy_c, qx_c) = linear.backward_products(
        dyd, xd, wd, s, "sr", operands=True, scales="mx")
    torch.cuda.synchronize()
    ax = _mx_operand(qx, x, 0, False, 0, 2 * s, "X rows")
    aw = _mx_operand(qw, w, 0, False, 0, 2 * s, "W rows")
    ady_r = _mx_operand(qdy_r, dy, 0, True, 3 * s, 2 * s + 1, "dY rows")
    ady_c = _mx_operand(qdy_c, dy, 1, True, 3 * s, 2 * s + 1, "dY columns")
    aw_c = _mx_operand(qw_c, w, 1, True, 3 * s + 1, 2 * s + 1, "W columns")
    ax_c = _mx_operand(qx_c, x, 1, True, 3 * s + 2, 2 * s + 1, "X columns")
    f = 2.0 ** -7
    check_mx_entries(y, *ax, *aw, f)
    check_mx_entries(dx, *ady_r, *aw_c, f)
    check_mx_entries(dw, *ady_c, *ax_c, f)
    xf, wf, dyf = x.double().numpy(), w.double().numpy(), dy.double().numpy()
    for name, got, ex in (("Y", y, xf @ wf.T), ("dX", dx, dyf @ wf), ("dW", dw, dyf.T @ xf)):
        rel = np.linalg.norm(got.cpu().double().numpy() - ex) / np.linalg.norm(ex)
        print(f"{name}: relative error {rel:.4f}", flush=True)
        assert rel < 0.3, (name, rel)
    with pytest.raises(ValueError):
        linear.backward_products(dyd, xd, wd, s, "eden", scales="mx")


def test_fig9_mxfp4_recipe():
    """The MXFP4 recipe's SR backward is unbiased in the layer: the mean of B backward passes
    tracks mse/B out to B = 256; the mean of round-to-nearest passes (whose rotations change
    with the seed, but whose rounding is deterministic) has left mse/B by B = 256."""
    print("case: Fig. 9 method, MXFP4 recipe, 512 x 256 -> 256, B = 1..256", flush=True)
    t, n_in, n_out = 512, 256, 256
    x, w, dy = layer_inputs(t, n_in, n_out, seed=90)
    xd, wd, dyd = x.to(DEV), w.to(DEV), dy.to(DEV)
    exact = [dyd.double() @ wd.double(), dyd.double().t() @ xd.double()]
    norms = [float((e * e).sum()) for e in exact]
    for scheme in ("sr", "rtn"):
        acc = [torch.zeros_like(e) for e in exact]
        single = [0.0, 0.0]
        for b in range(1, 257):
            grads = linear.backward_products(dyd, xd, wd, b, scheme, scales="mx")
            for i, g in enumerate(grads):
                g = g.double()
                acc[i] += g
                single[i] += float(((g - exact[i]) ** 2).sum()) / norms[i]
            if b in (1, 16, 256):
                for i, name in enumerate(("dX", "dW")):
                    bias = float(((acc[i] / b - exact[i]) ** 2).sum()) / norms[i]
                    expect = single[i] / b / b
                    print(scheme, name, b, f"{bias:.3e}/{expect:.3e}", flush=True)
                    if scheme == "sr":
                        assert 0.7 * expect < bias < 1.4 * expect, (name, b, bias, expect)
                    elif b == 256:
                        assert bias > 2.0 * expect, (name, b, bias, expect)
