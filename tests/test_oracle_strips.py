"""Pins of the oracle's strip-local scaling (the CTA-local variant of the rit.work note on
"Format-Aware Fusion for Fast FP4 Pretraining": the maximum behind the FP32 scale is taken
inside one block of work, and the GEMM applies separate row and column corrections after its
sum over K).  Reading: strips of 128 consecutive vectors, each with the scale of its own
maximum, every vector otherwise quantized as by the global method.

What fixes it apart from its own code: with one strip it is the global method (already pinned
elsewhere); each strip is the global method applied to that strip's vectors alone; scaling one
strip by a power of two scales only that strip's g and changes no code or scale anywhere (the
global method fails this: its shared g moves every strip's scales); a strip 2^-24 below the
rest keeps its resolution; and the unbiased schemes stay unbiased."""
import numpy as np
import pytest
import torch

import workloads

MODES = [("rtn", False), ("rtn", True), ("sr", False), ("sr", True), ("eden", True),
         ("fp46", False), ("fp46", True)]


def _bits(t):
    return workloads.bf16_bits(t)


def _scale_strip(x, axis, s, k, strip=128):
    """x with strip s of layout `axis` multiplied by 2^k (exact in bf16 away from the ends)."""
    y = x.float().clone()
    if axis == 0:
        y[s * strip:(s + 1) * strip, :] *= 2.0 ** k
    else:
        y[:, s * strip:(s + 1) * strip] *= 2.0 ** k
    out = y.to(torch.bfloat16)
    assert torch.equal(out.float(), y), "scaling must be exact"
    return out


@pytest.mark.parametrize("mode,rht", MODES)
@pytest.mark.parametrize("axis", [0, 1])
def test_one_strip_is_the_global_method(oracle_mod, mode, rht, axis):
    x = workloads.normal((128, 256), seed=11)
    xb = _bits(x)
    ref = oracle_mod.quantize(mode, xb, axis=axis, seed=4, rht=rht, rht_seed=6)
    vecs = 128 if axis == 0 else 256
    q = oracle_mod.quantize_strips(mode, xb, axis=axis, seed=4, rht=rht, rht_seed=6,
                                   strip=vecs)
    assert q.g.shape == (1,) and q.g[0] == np.float32(ref.g)
    for name in ("codes", "scales", "elem_margin", "scale_margin"):
        np.testing.assert_array_equal(getattr(q, name), getattr(ref, name), err_msg=name)


@pytest.mark.parametrize("mode,rht", MODES)
@pytest.mark.parametrize("axis", [0, 1])
def test_each_strip_is_the_global_method_on_its_vectors(oracle_mod, mode, rht, axis):
    """Strip s equals: the global tensor scale of the sub-matrix of strip s's vectors, then
    those vectors quantized with it (random streams by index in the whole layout).  The
    shape has a ragged last strip."""
    shape = (300, 256) if axis == 0 else (256, 320)
    x = workloads.c4(seed=2, shape=shape)
    xb = _bits(x)
    q = oracle_mod.quantize_strips(mode, xb, axis=axis, seed=8, rht=rht, rht_seed=5)
    vecs = shape[0] if axis == 0 else shape[1]
    assert q.g.shape == (-(-vecs // 128),)
    for s, v0 in enumerate(range(0, vecs, 128)):
        v1 = min(vecs, v0 + 128)
        sub = xb[v0:v1, :] if axis == 0 else xb[:, v0:v1]
        amax = oracle_mod.amax(np.ascontiguousarray(sub), axis, rht or mode == "eden", 5)
        g = oracle_mod.tensor_scale(mode, amax)
        assert q.g[s] == np.float32(g), s
        ref = oracle_mod.quantize_vectors(mode, xb, axis, np.arange(v0, v1), g, seed=8, rht=rht,
                                          rht_seed=5)
        np.testing.assert_array_equal(q.codes[v0:v1], ref.codes)
        np.testing.assert_array_equal(q.scales[v0:v1], ref.scales)


@pytest.mark.parametrize("mode,rht", MODES)
@pytest.mark.parametrize("axis", [0, 1])
def test_power_of_two_equivariance_per_strip(oracle_mod, mode, rht, axis):
    x = workloads.normal((384, 256) if axis == 0 else (256, 384), seed=21)
    q0 = oracle_mod.quantize_strips(mode, _bits(x), axis=axis, seed=3, rht=rht, rht_seed=2)
    for k in (-7, 4):
        xs = _scale_strip(x, axis, 1, k)
        q1 = oracle_mod.quantize_strips(mode, _bits(xs), axis=axis, seed=3, rht=rht, rht_seed=2)
        np.testing.assert_array_equal(q1.codes, q0.codes)
        np.testing.assert_array_equal(q1.scales, q0.scales)
        assert q1.g[0] == q0.g[0] and q1.g[2] == q0.g[2]
        assert q1.g[1] == np.float32(q0.g[1] * 2.0 ** k)
    # the global method is not strip-local: shrinking one strip moves that strip's scales
    g0 = oracle_mod.quantize(mode, _bits(x), axis=axis, seed=3, rht=rht, rht_seed=2)
    g1 = oracle_mod.quantize(mode, _bits(_scale_strip(x, axis, 1, -7)), axis=axis, seed=3,
                             rht=rht, rht_seed=2)
    assert not np.array_equal(g1.scales[128:256], g0.scales[128:256])


@pytest.mark.parametrize("axis", [0, 1])
def test_small_strip_keeps_its_resolution(oracle_mod, axis):
    """A strip 2^-24 below the others: under one tensor scale its block scales fall below
    E4M3's smallest value and the strip decodes to zero; with its own scale it keeps the
    same relative error as the other strips."""
    x = _scale_strip(workloads.normal((256, 256), seed=5), axis, 1, -24)
    xf = x.float().numpy().astype(np.float64)
    xf = xf if axis == 0 else xf.T
    rel = {}
    for name, q in (("global", oracle_mod.quantize("eden", _bits(x), axis=axis, seed=1,
                                                   rht_seed=1)),
                    ("strip", oracle_mod.quantize_strips("eden", _bits(x), axis=axis, seed=1,
                                                         rht_seed=1))):
        g = np.full(2, q.g, dtype=np.float32) if name == "global" else q.g
        back = oracle_mod.dequantize_strips(q.codes, q.scales, g, rht=True, rht_seed=1)
        rel[name] = [((back[s] - xf[s]) ** 2).sum() / (xf[s] ** 2).sum()
                     for s in (slice(0, 128), slice(128, 256))]
    assert rel["global"][1] > 0.99                       # the strip is lost
    assert rel["strip"][1] < 0.02 and rel["strip"][0] < 0.02
    assert abs(rel["strip"][1] - rel["strip"][0]) < 0.005


@pytest.mark.parametrize("mode,rht", [("eden", True), ("sr", False)])
def test_strip_scales_stay_unbiased(oracle_mod, mode, rht):
    """The mean of B strip-local passes (fresh seeds) converges as mse/B, as for one tensor
    scale: strips of very different magnitude (c3's rows span 10^-6 .. 10)."""
    x = workloads.c3(seed=1, shape=(256, 256))
    xb = _bits(x)
    xf = x.float().numpy().astype(np.float64)
    acc = np.zeros_like(xf)
    mse = 0.0
    norm = (xf ** 2).sum()
    for b in range(1, 257):
        q = oracle_mod.quantize_strips(mode, xb, axis=0, seed=b, rht=rht, rht_seed=b)
        back = oracle_mod.dequantize_strips(q.codes, q.scales, q.g, rht=rht, rht_seed=b)
        acc += back
        mse += ((back - xf) ** 2).sum() / norm
        if b in (1, 16, 256):
            bias = ((acc / b - xf) ** 2).sum() / norm
            expect = mse / b / b
            assert 0.7 * expect < bias < 1.4 * expect, (b, bias, expect)


def test_empty_and_degenerate(oracle_mod):
    z = np.zeros((0, 256), dtype=np.uint16)
    q = oracle_mod.quantize_strips("eden", z, axis=1, seed=1, rht_seed=1)
    assert q.g.shape == (2,) and not q.g.any() and q.codes.shape == (256, 0)
    q = oracle_mod.quantize_strips("eden", z, axis=0, seed=1, rht_seed=1)
    assert q.g.shape == (0,)
    zeros = np.zeros((200, 128), dtype=np.uint16)
    q = oracle_mod.quantize_strips("sr", zeros, axis=0, seed=1)
    assert q.g.shape == (2,) and not q.g.any() and not q.codes.any() and not q.scales.any()
