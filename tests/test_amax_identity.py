"""The identity phase 1 uses for the group maximum, checked on the oracle's transform.

Phase 1 wants only max |r| over each 128-element group.  The last butterfly stage (span 64)
outputs u + v and u - v; since max(|u + v|, |u - v|) = |u| + |v| and binary32 rounding is
monotone and symmetric in sign, max(|fl(u + v)|, |fl(u - v)|) = fl(|u| + |v|).  With s, d
the span-32 sum and difference of the first half and s', d' those of the second half, the
group's largest |r| is therefore the largest fl(|s_k| + |s'_k|) or fl(|d_k| + |d'_k|).

These tests run the unnormalized transform's first six stages in binary32 (spans 1..32, the
order of the oracle's transform), check that the last stage on top of them reproduces
oracle.fwht128 bit for bit, and then check the identity on inputs chosen to stress it:
random signs and magnitudes over the whole binary32 range the contract allows (|x| <= 2^56),
subnormals, exact zeros of both signs, and cancellations.
"""
import numpy as np
import pytest

import oracle


def stages_to_32(x: np.ndarray) -> np.ndarray:
    """Spans 1, 2, ..., 32 of the butterfly on each row of x (binary32, in place order)."""
    r = x.astype(np.float32).copy()
    s = 1
    while s < 64:
        idx = np.arange(128)
        lo = idx[(idx & s) == 0]
        u, v = r[:, lo].copy(), r[:, lo + s].copy()
        r[:, lo] = u + v
        r[:, lo + s] = u - v
        s <<= 1
    return r


def last_stage(r: np.ndarray) -> np.ndarray:
    out = r.copy()
    u, v = r[:, :64], r[:, 64:]
    out[:, :64] = u + v
    out[:, 64:] = u - v
    return out


def sum_form(r: np.ndarray) -> np.ndarray:
    """max over k of fl(|s_k| + |s'_k|) and fl(|d_k| + |d'_k|): 64 sums per group."""
    a, b = np.abs(r[:, :64]), np.abs(r[:, 64:])
    return (a + b).max(axis=1)                   # binary32 additions


def inputs(rng, n):
    kinds = []
    g = rng.standard_normal((n, 128)).astype(np.float32)
    kinds.append(g)
    e = rng.integers(-149, 57, size=(n, 128))
    m = rng.uniform(1, 2, size=(n, 128)) * rng.choice([-1.0, 1.0], size=(n, 128))
    kinds.append(np.ldexp(m, e).astype(np.float32))
    sub = (rng.integers(1, 1 << 23, size=(n, 128)).astype(np.uint32)
           | (rng.integers(0, 2, size=(n, 128)).astype(np.uint32) << 31)).view(np.float32)
    kinds.append(sub)
    z = g.copy()
    z[rng.random(z.shape) < 0.9] = 0.0
    z[rng.random(z.shape) < 0.5] *= -1.0         # zeros of both signs
    kinds.append(z)
    c = np.repeat(rng.standard_normal((n, 1)).astype(np.float32), 128, axis=1)
    c *= rng.choice([-1.0, 1.0], size=(n, 128)).astype(np.float32)
    kinds.append(c)                              # equal magnitudes: heavy cancellation
    big = np.ldexp(rng.uniform(1, 2, size=(n, 128)), 56).astype(np.float32)
    kinds.append(big * rng.choice([-1.0, 1.0], size=(n, 128)).astype(np.float32))
    return np.concatenate(kinds)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_stages_match_oracle_transform(seed):
    rng = np.random.default_rng(seed)
    x = inputs(rng, 64)
    full = last_stage(stages_to_32(x))
    for i in range(0, len(x), 37):
        np.testing.assert_array_equal(full[i], oracle.fwht128(x[i]), err_msg=f"row {i}")


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_group_max_from_64_sums(seed):
    rng = np.random.default_rng(100 + seed)
    x = inputs(rng, 2000)
    r = stages_to_32(x)
    want = np.abs(last_stage(r)).max(axis=1)
    got = sum_form(r)
    np.testing.assert_array_equal(got, want)


def test_identity_on_every_pair_of_small_floats():
    """Exhaustive over u, v from a set of binary32 values spanning normals, subnormals and
    both zeros: max(|fl(u+v)|, |fl(u-v)|) == fl(|u| + |v|)."""
    rng = np.random.default_rng(7)
    vals = np.concatenate([
        np.array([0.0, -0.0, 1.0, -1.0, 3.0, 2.0 ** -149, -(2.0 ** -149), 2.0 ** -126,
                  2.0 ** 56, -(2.0 ** 56)], dtype=np.float32),
        rng.standard_normal(200).astype(np.float32),
        (rng.integers(1, 1 << 23, 100).astype(np.uint32)).view(np.float32),
        np.ldexp(rng.uniform(1, 2, 100), rng.integers(-140, 50, 100)).astype(np.float32),
    ])
    u, v = np.meshgrid(vals, vals)
    lhs = np.maximum(np.abs(u + v), np.abs(u - v))
    rhs = np.abs(u) + np.abs(v)
    np.testing.assert_array_equal(lhs, rhs)
