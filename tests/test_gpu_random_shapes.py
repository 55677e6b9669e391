"""Parity on a seeded sweep of shapes: every quantizer, with and without strip-local scales,
on row counts and column counts drawn at random within the rules of the C ABI (a layout's n
a multiple of 128 with the rotation, of 16 without; cols a multiple of 8).  Each case is
compared in full against the oracle: codes, scales and every tensor scale bit for bit."""
import numpy as np
import pytest

import oracle
import workloads
from parity import assert_parity, compare
from test_gpu_parity import run_gpu
from test_gpu_strips import run_strips

pytestmark = pytest.mark.gpu

MODES = [("rtn", False), ("sr", False), ("eden", True), ("fp46", False), ("rtn", True),
         ("sr", True), ("fp46", True)]


def _cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for k in range(n):
        mode, rht = MODES[k % len(MODES)]
        rot = rht or mode == "eden"
        layouts = [("row",), ("col",), ("row", "col")][rng.integers(3)]
        unit = 128 if rot else 16
        # a dimension that is some layout's n follows that layout's rule; the other is free
        rows = int(rng.integers(1, 6)) * unit if "col" in layouts else int(rng.integers(1, 700))
        cols = int(rng.integers(1, 6)) * unit if "row" in layouts else 8 * int(rng.integers(1, 90))
        out.append((mode, rht, layouts, rows, cols, int(rng.integers(1 << 30))))
    return out


@pytest.mark.parametrize("mode,rht,layouts,rows,cols,seed", _cases(21, 2024))
def test_random_shape_tensor_scale(mode, rht, layouts, rows, cols, seed):
    print(f"case: {mode} rht={rht} {layouts} {rows}x{cols} seed={seed}", flush=True)
    x = workloads.c4(seed=seed % 1000, shape=(rows, cols))
    got = run_gpu(mode, x, layouts, seed=seed, rht=rht, rht_seed=seed + 1, guard=True)
    xb = workloads.bf16_bits(x)
    for axis, (codes, scales, g, _) in got.items():
        ref = oracle.quantize(mode, xb, axis=axis, seed=seed, rht=rht, rht_seed=seed + 1)
        assert_parity(mode, codes, scales, g, ref, f"axis={axis}")


@pytest.mark.parametrize("mode,rht,layouts,rows,cols,seed", _cases(14, 77))
def test_random_shape_strip_scales(mode, rht, layouts, rows, cols, seed):
    print(f"case: strips {mode} rht={rht} {layouts} {rows}x{cols} seed={seed}", flush=True)
    x = workloads.c4(seed=seed % 997, shape=(rows, cols))
    got = run_strips(mode, x, layouts, seed=seed, rht=rht, rht_seed=seed + 2)
    xb = workloads.bf16_bits(x)
    for axis, t in got.items():
        ref = oracle.quantize_strips(mode, xb, axis=axis, seed=seed, rht=rht, rht_seed=seed + 2)
        assert np.array_equal(t.tensor_scale.cpu().numpy(), ref.g), f"axis={axis}: strip g"
        rep = compare(mode, t.codes.cpu().numpy(), t.scales.cpu().numpy(), ref)
        assert rep.ok(), f"axis={axis}: {rep}"
