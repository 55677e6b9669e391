"""Pins of the oracle's MXFP4 block contract (CPU only): E2M1 elements with one power-of-two
(E8M0) scale per 32, the scale the smallest power of two that lets the grid's top (6) cover the
block.  Checked against brute force in fp64, closed-form round trips of on-grid inputs (with
and without the rotation), the layout and scaling invariants, and the unbiasedness of the SR
variant by the Fig. 9 method of the Quartet II summary."""
import numpy as np
import pytest
import torch

import oracle
import workloads

MAGS = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)


def _bits(t):
    return workloads.bf16_bits(t)


def test_scale_exponent_brute_force():
    rng = np.random.default_rng(0)
    m = np.concatenate([
        np.exp2(rng.uniform(-149, 127, 20000)),
        [6.0 * 2.0 ** k for k in range(-40, 40)],                     # exactly 6 * 2^k
        [np.nextafter(np.float32(6.0 * 2.0 ** k), np.float32(np.inf)) for k in range(-40, 40)],
        [1.5 * 2.0 ** k for k in range(-40, 40)], [2.0 ** k for k in range(-149, 128)],
        [np.finfo(np.float32).max, np.finfo(np.float32).tiny, 1e-45],
    ]).astype(np.float32)
    m = m[np.isfinite(m) & (m > 0)]
    for v in m:
        e = oracle.mx_scale_exp(float(v))
        assert -127 <= e <= 127
        assert 6.0 * 2.0 ** e >= float(v), (v, e)                       # covers the block
        assert e == -127 or 6.0 * 2.0 ** (e - 1) < float(v), (v, e)     # and is the smallest
    assert oracle.mx_scale_exp(0.0) == -127


def test_rtn_codes_are_nearest_and_never_clip():
    x = workloads.c4(seed=2, shape=(256, 1024))
    q = oracle.mx_quantize(_bits(x), axis=0)
    r = x.float().numpy().astype(np.float64)
    e = q.scales.astype(np.int64) - 127
    blockmax = np.abs(r).reshape(256, -1, 32).max(-1)
    assert np.all(6.0 * np.exp2(e) >= blockmax) and np.all(6.0 * np.exp2(e - 1) < blockmax)
    y = np.abs(r) / np.repeat(np.exp2(e), 32, axis=1)
    assert y.max() <= 6.0
    codes = oracle.unpack_codes(q.codes)
    d_all = np.abs(y[..., None] - MAGS)
    d_pick = np.take_along_axis(d_all, (codes & 7)[..., None].astype(np.int64), -1)[..., 0]
    assert np.all(d_pick <= d_all.min(-1) + 1e-12)
    assert np.all(((codes & 8) != 0) == (r < 0))


def test_sr_codes_are_grid_neighbours():
    x = workloads.c1()
    q = oracle.mx_quantize(_bits(x), axis=0, sr=True, seed=3)
    r = x.float().numpy().astype(np.float64)
    e = q.scales.astype(np.int64) - 127
    y = np.abs(r) / np.repeat(np.exp2(e), 32, axis=1)
    lo = np.searchsorted(MAGS, y, side="right") - 1
    codes = oracle.unpack_codes(q.codes) & 7
    assert np.all((codes == lo) | (codes == np.minimum(lo + 1, 7)))
    # the draws differ per seed and per element
    q2 = oracle.mx_quantize(_bits(x), axis=0, sr=True, seed=4)
    assert np.mean(q2.codes != q.codes) > 0.05


def _on_grid(rng, rows, cols, k):
    """x = sign * V * 2^e per 32-block, every block holding a +-6 (so its scale is 2^e)."""
    x = np.zeros((rows, cols))
    for r in range(rows):
        for b in range(cols // 32):
            if rng.random() < 0.1:
                continue
            e = int(rng.integers(-20, 20)) + k
            v = rng.choice(MAGS, 32) * rng.choice([-1.0, 1.0], 32)
            v[rng.integers(32)] = 6.0 * rng.choice([-1.0, 1.0])
            x[r, 32 * b:32 * b + 32] = v * 2.0 ** e
    return x


def test_round_trip_on_grid_inputs():
    rng = np.random.default_rng(5)
    x = _on_grid(rng, 64, 256, 0)
    xt = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(xt.double().numpy(), x)
    q = oracle.mx_quantize(_bits(xt), axis=0)
    np.testing.assert_array_equal(oracle.mx_dequantize(q.codes, q.scales).astype(np.float64), x)
    q = oracle.mx_quantize(_bits(xt), axis=0, sr=True, seed=9)       # on the grid: exact too
    np.testing.assert_array_equal(oracle.mx_dequantize(q.codes, q.scales).astype(np.float64), x)


def test_rotated_round_trip():
    """x = sigma * H (c v) / 128 with v on the grid: the rotation gives back c v exactly, RTN
    keeps it, and decoding with the rotation returns x."""
    rng = np.random.default_rng(6)
    h = np.array([[1]], dtype=np.int64)
    while h.shape[0] < 128:
        h = np.kron(np.array([[1, 1], [1, -1]]), h)
    rht_seed = 13
    sig = oracle.signs(rht_seed).astype(np.float64)
    v = np.zeros((8, 128))
    for i in range(8):
        for b in range(4):
            k = rng.choice(32, 2, replace=False)
            v[i, 32 * b + k[0]] = 6.0 * rng.choice([-1, 1])
            v[i, 32 * b + k[1]] = rng.choice(MAGS[:7]) * rng.choice([-1, 1])
    x = sig * ((2.0 ** -3 * v) @ h.T) / 128.0
    xt = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(xt.double().numpy(), x)
    q = oracle.mx_quantize(_bits(xt), axis=0, rht=True, rht_seed=rht_seed)
    np.testing.assert_array_equal(q.scales, 127 - 3)
    back = oracle.mx_dequantize(q.codes, q.scales, rht=True, rht_seed=rht_seed)
    np.testing.assert_array_equal(back.astype(np.float64), x)


@pytest.mark.parametrize("sr,rht", [(False, False), (True, False), (False, True), (True, True)])
def test_layout_and_scaling_invariants(sr, rht):
    x = workloads.c4(seed=8, shape=(256, 384))
    xb = _bits(x)
    col = oracle.mx_quantize(xb, axis=1, sr=sr, seed=2, rht=rht, rht_seed=3)
    row_t = oracle.mx_quantize(np.ascontiguousarray(xb.T), axis=0, sr=sr, seed=2, rht=rht,
                               rht_seed=3)
    # same values; the random stream of the column layout is its own (axis 1)
    if not sr:
        np.testing.assert_array_equal(col.codes, row_t.codes)
    np.testing.assert_array_equal(col.scales, row_t.scales)
    x2 = (x.double() * 2.0 ** 5).to(torch.bfloat16)
    q1 = oracle.mx_quantize(xb, axis=0, sr=sr, seed=2, rht=rht, rht_seed=3)
    q2 = oracle.mx_quantize(_bits(x2), axis=0, sr=sr, seed=2, rht=rht, rht_seed=3)
    np.testing.assert_array_equal(q2.codes, q1.codes)
    np.testing.assert_array_equal(q2.scales.astype(int), q1.scales.astype(int) + 5)


def test_sr_is_unbiased_fig9_method():
    """Mean of B SR passes: its error tracks mse/B (slope -1) to B = 256; RTN's plateaus."""
    x = workloads.c1()
    xb = _bits(x)
    xf = x.float().numpy().astype(np.float64)
    norm = (xf ** 2).sum()
    acc = np.zeros_like(xf)
    mse = 0.0
    for b in range(1, 257):
        q = oracle.mx_quantize(xb, axis=0, sr=True, seed=b, rht=True, rht_seed=b)
        back = oracle.mx_dequantize(q.codes, q.scales, rht=True, rht_seed=b)
        acc += back
        mse += ((back - xf) ** 2).sum() / norm
    bias = ((acc / 256 - xf) ** 2).sum() / norm
    mean_mse = mse / 256
    assert bias < 2.0 * mean_mse / 256            # unbiased: the mean's error is mse / B
    q = oracle.mx_quantize(xb, axis=0)
    rtn_err = ((oracle.mx_dequantize(q.codes, q.scales) - xf) ** 2).sum() / norm
    assert bias < 0.05 * rtn_err


def test_sr_draws_are_independent_per_element():
    """Elements halfway between two grid points round up with probability 1/2 each, and
    neighbouring elements decide independently (one random draw per element)."""
    rows, cols = 128, 1024
    x = np.full((rows, cols), 0.25)
    x[:, ::32] = 6.0                                   # each block's scale is 2^0
    xt = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
    q = oracle.mx_quantize(_bits(xt), axis=0, sr=True, seed=21)
    up = (oracle.unpack_codes(q.codes) & 7) == 1       # 0.25 -> 0.5 (up) or 0 (down)
    half = np.ones(cols, dtype=bool)
    half[::32] = False
    u = up[:, half]
    assert abs(u.mean() - 0.5) < 0.01
    agree = (u[:, 1:] == u[:, :-1]).mean()
    assert abs(agree - 0.5) < 0.01, agree


def test_k_tile_places_every_byte_by_its_index():
    """The K-tiled storage against its definition, one byte at a time: code byte j of vector v
    at flat offset (j // 64) * vecs * 64 + v * 64 + j % 64, scale byte s at
    (s // 4) * vecs * 4 + v * 4 + s % 4; and a shape that is not a multiple of 128 is refused."""
    rng = np.random.default_rng(3)
    vecs, n = 5, 384
    codes = rng.integers(0, 256, (vecs, n // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, (vecs, n // 32), dtype=np.uint8)
    tc, ts = oracle.mx_k_tile(codes, scales)
    assert tc.shape == (n // 128, vecs, 64) and ts.shape == (n // 128, vecs, 4)
    fc, fs = tc.reshape(-1), ts.reshape(-1)
    for v in range(vecs):
        for j in range(n // 2):
            assert fc[(j // 64) * vecs * 64 + v * 64 + j % 64] == codes[v, j]
        for k in range(n // 32):
            assert fs[(k // 4) * vecs * 4 + v * 4 + k % 4] == scales[v, k]
    with pytest.raises(ValueError):
        oracle.mx_k_tile(codes[:, :48], scales[:, :6])
