"""Pins of the oracle's margins (CPU only).

A margin is the distance, in units in the last place, from a pre-rounding value to the
boundary of the rounding it feeds; the parity rule may excuse a GPU/oracle mismatch only
within 2 ulp of such a boundary.  Each margin is checked here against its meaning, by brute
force: step the value one float at a time (np.nextafter) up and down, holding every other
input fixed, and count the steps until the oracle's own rounding function (itself pinned
against torch and brute force in test_oracle_primitives.py) returns a different result.  For
a margin m that count is m or m + 1 (whether the boundary value itself rounds up or down);
for the element SR margin, whose boundary is not a binary32 value, it is within 1 of m.
"""
import numpy as np

import oracle

CAP = 48                         # steps tried in each direction
E2M1_THRESH = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)


def _around(points, k=40, lo=None, hi=None):
    """Values within k ulps of each point."""
    pts = np.asarray(points, dtype=np.float32)
    out = [pts]
    up, dn = pts.copy(), pts.copy()
    for _ in range(k):
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(0))
        out += [up.copy(), dn.copy()]
    v = np.concatenate(out)
    if lo is not None:
        v = v[v >= lo]
    if hi is not None:
        v = v[v < hi]
    return v


def _steps(fn, v):
    """Smallest number of one-ulp steps, up or down, after which fn changes (CAP + 1 if
    none within CAP)."""
    base = fn(v)
    best = np.full(v.shape, CAP + 1, dtype=np.int64)
    for direction in (np.float32(np.inf), np.float32(-np.inf)):
        cur = v.copy()
        for k in range(1, CAP + 1):
            cur = np.nextafter(cur, direction)
            hit = (fn(cur) != base) & (best > k)
            best[hit] = k
    return best


def _check(m, s, slack_low=0):
    m = m.astype(np.int64)
    near = m < CAP - 1
    assert near.sum() > 100, "the sample must hold values near the boundaries"
    ok = (s[near] >= m[near] - slack_low) & (s[near] <= m[near] + 1)
    bad = np.flatnonzero(~ok)
    assert ok.all(), f"{bad.size} margins disagree, e.g. m={m[near][bad[:5]]} steps={s[near][bad[:5]]}"
    # far from every boundary nothing changes within the steps tried
    assert np.all(s[~near] >= CAP - 1)


def test_e2m1_margin():
    rng = np.random.default_rng(0)
    v = np.concatenate([_around(E2M1_THRESH),
                        rng.uniform(0, 8, 20000).astype(np.float32)])
    v = np.concatenate([v, -v])                      # the margin is of |v|
    m = oracle.margin_n("e2m1", v)
    s = _steps(lambda a: oracle.e2m1_rtn_mag_n(np.abs(a)), v)
    _check(m, s)


def _e4m3_values():
    return np.array([oracle.e4m3_value(c) for c in range(127)], dtype=np.float32)


def test_e4m3_rne_margin():
    vals = _e4m3_values()
    mids = (vals[:-1] + vals[1:]) / 2
    rng = np.random.default_rng(1)
    v = np.concatenate([_around(mids, lo=0), _around(vals[1:], k=3, lo=0),
                        rng.uniform(0, 470, 20000).astype(np.float32),
                        np.exp2(rng.uniform(-12, 9, 20000)).astype(np.float32)])
    v = v[v > 0]
    m = oracle.margin_n("e4m3_rne", v)
    s = _steps(oracle.e4m3_rne_sat_n, v)
    _check(m, s)


def test_e4m3_up_margin():
    vals = _e4m3_values()
    rng = np.random.default_rng(2)
    v = np.concatenate([_around(vals[1:], lo=0), _around([448.0, 460.0]),
                        rng.uniform(0, 470, 20000).astype(np.float32),
                        np.exp2(rng.uniform(-12, 9, 20000)).astype(np.float32)])
    v = v[v > 0]
    m = oracle.margin_n("e4m3_up", v)
    s = _steps(oracle.e4m3_up_n, v)
    _check(m, s)


def test_scale_sr_margin():
    """Scale SR of c in [2^-6, 448) with a fixed word w: c one float at a time."""
    rng = np.random.default_rng(3)
    n = 600
    w = rng.integers(0, 2**32, n, dtype=np.uint64).astype(np.uint32)
    c = np.exp2(rng.uniform(-5.5, 8.5, n)).astype(np.float32)
    # half of the samples put bits(c) + (w >> 12) within a few units of a carry
    near = np.arange(n) < n // 2
    low = (c.view(np.uint32) & 0xFFFFF).astype(np.int64)
    target = (1 << 20) - (w.astype(np.int64) >> 12) + rng.integers(-30, 31, n)
    newlow = np.clip(target, 0, (1 << 20) - 1)
    bits = (c.view(np.uint32).astype(np.int64) & ~0xFFFFF) | np.where(near, newlow, low)
    c = bits.astype(np.uint32).view(np.float32)
    m = oracle.margin_n("scale_sr", c, w)

    def fn(cc):
        return np.array([oracle.scale_sr(float(a), int(b)) for a, b in zip(cc, w)])

    s = _steps(fn, c)
    _check(m, s)


def test_elem_sr_margin():
    """Element SR of a in [0, 6) with a fixed random word (draw v = word >> 10)."""
    rng = np.random.default_rng(4)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)
    n = 600
    u = rng.integers(0, 2**32, n, dtype=np.uint64).astype(np.uint32)
    lo = rng.integers(0, 7, n)
    point = grid[lo] + (1 - (u >> 10) / 2**22) * (grid[lo + 1] - grid[lo])   # the boundary
    a = point.astype(np.float32)
    a = np.where(np.arange(n) % 3 == 0, rng.uniform(0, 5.99, n).astype(np.float32), a)
    offs = rng.integers(-30, 31, n)
    for i in range(n):                   # move each sample a few floats off its boundary
        for _ in range(abs(int(offs[i]))):
            a[i] = np.nextafter(a[i], np.float32(np.inf if offs[i] > 0 else 0))
    a = np.minimum(a, np.float32(5.99))
    m = oracle.margin_n("elem_sr", a, u)

    def fn(aa):
        aa = np.minimum(np.maximum(aa, 0), np.float32(6.0))
        return np.array([oracle.elem_sr_mag(float(x), int(d)) for x, d in zip(aa, u)])

    s = _steps(fn, a)
    _check(m, s, slack_low=1)


def test_ulp_distance():
    """The ulp distance between two non-negative floats is the number of nextafter steps
    from one to the other."""
    rng = np.random.default_rng(5)
    a = np.exp2(rng.uniform(-20, 20, 3000)).astype(np.float32)
    k = rng.integers(0, 60, a.size)
    b = a.copy()
    for step in range(60):
        b = np.where(k > step, np.nextafter(b, np.float32(np.inf)), b)
    m = oracle.margin_n("ulp", a, b.view(np.uint32))
    assert np.array_equal(m.astype(np.int64), k)
    m2 = oracle.margin_n("ulp", b, a.view(np.uint32))
    assert np.array_equal(m2.astype(np.int64), k)
