"""Pins of the oracle's primitives against sources other than itself (CPU only).

* Philox4x32-10: rocRAND's engine (an independent implementation, called through its public
  API from a small host program) and the known-answer vectors of the Random123 release.
* Hadamard transform: the Sylvester matrix built with np.kron; exact on integer inputs.
* E4M3: torch's float8_e4m3fn cast (a library routine) and brute-force nearest / round-up
  over the 127 non-negative finite values.
* E2M1: brute-force nearest over the 8 magnitudes.
* SR steps: enumeration of every random draw.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


# ----------------------------------------------------------------------------- Philox

def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append([int(t, 16) for t in line.split()])
    return rows


def test_philox_known_answers(oracle_mod):
    # Random123 known-answer vectors for philox4x32 with 10 rounds (cited in the file).
    for row in _read_golden("philox4x32_10_kat.txt"):
        ctr, key, expect = row[0:4], row[4:6], row[6:10]
        got = oracle_mod.philox4x32_10(key[0] | (key[1] << 32), ctr)
        assert [int(v) for v in got] == expect


@pytest.fixture(scope="module")
def rocrand_dump(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND helper")
    exe = str(tmp_path_factory.mktemp("rocrand") / "philox_dump")
    src = os.path.join(ROOT, "tests", "helpers", "rocrand_philox_dump.cpp")
    subprocess.check_call([hipcc, "-O1", "-o", exe, src], cwd="/tmp")
    return exe


def test_philox_matches_rocrand(oracle_mod, rocrand_dump):
    rng = np.random.default_rng(123)
    cases = []
    for i in range(400):
        key = int(rng.integers(0, 2**64, dtype=np.uint64))
        ctr = [int(v) for v in rng.integers(0, 2**32, size=4, dtype=np.uint64)]
        if i % 4 == 0:  # the counters the quantizers actually use: small indices, streams 1..3
            ctr = [int(rng.integers(0, 2**24)), 0, int(rng.integers(1, 4)), int(rng.integers(0, 2))]
        cases.append((key, ctr))
    text = "".join(f"{k} {c[0]} {c[1]} {c[2]} {c[3]}\n" for k, c in cases)
    out = subprocess.run([rocrand_dump], input=text, capture_output=True, text=True, check=True)
    lines = out.stdout.strip().splitlines()
    assert len(lines) == len(cases)
    for (key, ctr), line in zip(cases, lines):
        expect = [int(t) for t in line.split()]
        assert [int(v) for v in oracle_mod.philox4x32_10(key, ctr)] == expect


def test_signs_are_bits_of_the_sign_stream(oracle_mod, rocrand_dump):
    # sigma_j = -1 iff bit (j mod 32) of word j/32 of the block at counter (0, 0, 1, 0).
    for seed in (0, 1, 7, 2**63 + 5):
        out = subprocess.run([rocrand_dump], input=f"{seed} 0 0 1 0\n", capture_output=True,
                             text=True, check=True)
        words = [int(t) for t in out.stdout.split()]
        bits = np.array([(words[j >> 5] >> (j & 31)) & 1 for j in range(128)])
        expect = np.where(bits == 1, -1.0, 1.0).astype(np.float32)
        np.testing.assert_array_equal(oracle_mod.signs(seed), expect)
    assert not np.array_equal(oracle_mod.signs(1), oracle_mod.signs(2))


# ----------------------------------------------------------------------------- Hadamard

def _sylvester(n=128):
    h = np.array([[1]], dtype=np.int64)
    while h.shape[0] < n:
        h = np.kron(np.array([[1, 1], [1, -1]], dtype=np.int64), h)
    return h


def test_sylvester_orthogonality():
    h = _sylvester()
    np.testing.assert_array_equal(h @ h.T, 128 * np.eye(128, dtype=np.int64))


def test_fwht_columns_are_sylvester(oracle_mod):
    h = _sylvester()
    for k in range(128):
        e = np.zeros(128, dtype=np.float32)
        e[k] = 1.0
        np.testing.assert_array_equal(oracle_mod.fwht128(e), h[:, k].astype(np.float32))


def test_fwht_exact_on_integers(oracle_mod):
    h = _sylvester()
    rng = np.random.default_rng(5)
    for _ in range(50):
        x = rng.integers(-1000, 1000, size=128)
        np.testing.assert_array_equal(oracle_mod.fwht128(x.astype(np.float32)),
                                      (h @ x).astype(np.float32))
        # applying it twice gives 128 x (H H = 128 I)
        twice = oracle_mod.fwht128(oracle_mod.fwht128(x.astype(np.float32)))
        np.testing.assert_array_equal(twice, (128 * x).astype(np.float32))


def test_fwht_rounding_bound(oracle_mod):
    # 7 rounded levels: |fl - exact| <= gamma_7 * sum |x_j|, gamma_7 = 7u / (1 - 7u).
    h = _sylvester().astype(np.float64)
    rng = np.random.default_rng(6)
    u = 2.0 ** -24
    gamma = 7 * u / (1 - 7 * u)
    for _ in range(200):
        x = (rng.standard_normal(128) * np.exp(rng.uniform(-8, 8, 128))).astype(np.float32)
        exact = h @ x.astype(np.float64)
        got = oracle_mod.fwht128(x).astype(np.float64)
        assert np.all(np.abs(got - exact) <= gamma * np.abs(x.astype(np.float64)).sum())


# ----------------------------------------------------------------------------- E4M3

def _e4m3_table():
    codes = np.arange(0x7F, dtype=np.uint8)
    vals = np.array([float(torch.tensor([c], dtype=torch.uint8).view(torch.float8_e4m3fn)
                           .to(torch.float64)) for c in codes])
    return codes, vals


def test_e4m3_values_match_torch(oracle_mod):
    codes, vals = _e4m3_table()
    for c, v in zip(codes, vals):
        assert oracle_mod.e4m3_value(int(c)) == v
    assert vals[0x7E] == 448.0 and vals[0x08] == 2.0 ** -6 and vals[1] == 2.0 ** -9


def _probe_values(points, spread=4096, extra=None, seed=0):
    """Every fp32 within +-spread ulps of each point, plus random fp32 in the range."""
    pts = []
    for p in points:
        b = np.array([p], dtype=np.float32).view(np.uint32)[0].astype(np.int64)
        lo = max(b - spread, 0)
        pts.append(np.arange(lo, b + spread + 1, dtype=np.int64))
    bits = np.concatenate(pts).astype(np.uint32)
    vals = bits.view(np.float32)
    if extra is not None:
        vals = np.concatenate([vals, extra.astype(np.float32)])
    return vals[np.isfinite(vals) & (vals >= 0)]


def _brute_nearest_even(t, vals):
    """Index of the nearest table value to t (float64), ties to the even index."""
    t = t.astype(np.float64)[:, None]
    d = np.abs(vals[None, :] - t)
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    idx = np.argmax(cand, axis=1)
    two = cand.sum(axis=1) > 1
    idx[two & (idx % 2 == 1)] += 1
    return idx


def test_e4m3_rne_against_torch_and_brute_force(oracle_mod):
    codes, vals = _e4m3_table()
    mids = (vals[:-1] + vals[1:]) / 2
    rng = np.random.default_rng(0)
    rand_bits = rng.integers(0, np.float32(470.0).view(np.uint32), 2_000_000, dtype=np.uint64)
    extra = rand_bits.astype(np.uint32).view(np.float32)
    t = _probe_values(list(vals) + list(mids) + [448.0, 464.0], extra=extra)
    got = oracle_mod.e4m3_rne_sat_n(t)
    # torch: round to nearest even; NaN at and above 464 where ours saturates to 448
    under = t < 464.0
    ref = torch.from_numpy(t[under]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(got[under], ref)
    assert np.all(got[~under] == 0x7E)
    # brute force over the 127 values (chunked), saturating
    sample = t[:: max(1, t.size // 200_000)]
    bf = np.concatenate([_brute_nearest_even(c, vals) for c in np.array_split(sample, 20)])
    bf = np.where(sample >= 448.0, 0x7E, bf)
    np.testing.assert_array_equal(oracle_mod.e4m3_rne_sat_n(sample), bf.astype(np.uint8))


def test_e4m3_up_brute_force(oracle_mod):
    codes, vals = _e4m3_table()
    rng = np.random.default_rng(1)
    extra = rng.integers(0, np.float32(460.0).view(np.uint32), 1_000_000,
                         dtype=np.uint64).astype(np.uint32).view(np.float32)
    t = _probe_values(list(vals), spread=2048, extra=extra)
    got = oracle_mod.e4m3_up_n(t)
    idx = np.searchsorted(vals, t.astype(np.float64), side="left")   # first value >= t
    idx = np.minimum(idx, 0x7E)
    np.testing.assert_array_equal(got, idx.astype(np.uint8))
    # rounding up never lands below t (away from the cap)
    below = t <= 448.0
    up_vals = vals[got[below]]
    assert np.all(up_vals >= t[below])


# ----------------------------------------------------------------------------- E2M1

def test_e2m1_rtn_brute_force(oracle_mod):
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)
    mids = (mags[:-1] + mags[1:]) / 2
    rng = np.random.default_rng(2)
    extra = np.concatenate([
        rng.uniform(0, 8, 2_000_000),
        rng.integers(0, np.float32(8.0).view(np.uint32), 1_000_000, dtype=np.uint64)
        .astype(np.uint32).view(np.float32).astype(np.float64),
        np.array([6.0, 7.0, 100.0, 1e30, 3.4e38]),
    ])
    a = _probe_values(list(mags) + list(mids), spread=8192, extra=extra)
    got = oracle_mod.e2m1_rtn_mag_n(a)
    ref = _brute_nearest_even(a, mags)
    ref = np.where(a > 6.0, 7, ref)
    np.testing.assert_array_equal(got, ref.astype(np.uint8))
    for c in range(16):
        v = oracle_mod.e2m1_value(c)
        assert abs(v) == mags[c & 7] and (np.signbit(v) == bool(c & 8))


# ----------------------------------------------------------------------------- SR steps

def test_scale_sr_enumeration(oracle_mod):
    """Over all 2^20 values of the used random bits, #up = the dropped 20 bits, so the
    expectation of the stochastically rounded scale is exactly c."""
    codes, vals = _e4m3_table()
    rng = np.random.default_rng(3)
    words = (np.arange(2 ** 20, dtype=np.uint64) << 12).astype(np.uint32)
    cs = list(rng.uniform(2.0 ** -6, 447.9, 40).astype(np.float32))
    cs += [np.float32(2.0 ** -6), np.float32(416.0), np.nextafter(np.float32(448.0), 0,
                                                                   dtype=np.float32)]
    for c in cs:
        c = np.float32(c)
        out = oracle_mod.scale_sr_n(float(c), words)
        lo_bits = int(np.array([c]).view(np.uint32)[0]) & 0xFFF00000
        lo = float(np.uint32(lo_bits).view(np.float32))
        hi_idx = int(np.searchsorted(vals, lo)) + 1
        hi = vals[min(hi_idx, 0x7E)]
        o = vals[out]
        assert set(np.unique(o)).issubset({lo, hi})
        n_up = int((o == hi).sum()) if hi != lo else 0
        low20 = int(np.array([c]).view(np.uint32)[0]) & 0xFFFFF
        assert n_up == low20
        assert lo + (hi - lo) * n_up / 2 ** 20 == float(c)   # exact in float64
    # low bits ignored: words differing only in bits 0..11 give identical results
    c = np.float32(3.3)
    assert np.array_equal(oracle_mod.scale_sr_n(float(c), words),
                          oracle_mod.scale_sr_n(float(c), words | np.uint32(0xFFF)))


def test_elem_sr_enumeration(oracle_mod):
    """Over all 2^22 draws v (the top 22 bits of the word), the magnitude moves up exactly
    for the floor(frac * 2^22) largest draws: add-and-round-down stochastic rounding, whose
    mean lands on a within one 2^-22 step of the grid spacing.  The ten bits below the draw
    never matter."""
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)
    v = np.arange(2 ** 22, dtype=np.uint32)
    words = v << np.uint32(10)
    rng = np.random.default_rng(4)
    low = rng.integers(0, 1024, v.size).astype(np.uint32)
    for a in list(rng.uniform(0, 6, 12).astype(np.float32)) + [np.float32(0.0),
                                                              np.float32(1.5),
                                                              np.float32(5.999),
                                                              np.float32(0.3),
                                                              np.float32(1e-9)]:
        a64 = float(a)
        got = oracle_mod.elem_sr_mag_n(float(a), words)
        lo = int(np.searchsorted(mags, a64, side="right") - 1)
        frac = (a64 - mags[lo]) / (mags[lo + 1] - mags[lo])
        n_up = int(np.floor(frac * 2 ** 22))
        want = np.where(v >= 2 ** 22 - n_up, lo + 1, lo)
        assert np.array_equal(got, want)
        assert np.array_equal(oracle_mod.elem_sr_mag_n(float(a), words | low), want)
        mean = mags[lo] + (mags[lo + 1] - mags[lo]) * n_up / 2 ** 22
        assert 0 <= a64 - mean < (mags[lo + 1] - mags[lo]) * 2.0 ** -22
    assert oracle_mod.elem_sr_mag(6.0, 0) == 7
