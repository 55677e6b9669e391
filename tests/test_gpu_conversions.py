"""The quantizers' scalar device functions on the GPU against the oracle, over every input
the contract feeds them (tests/helpers/conv_check.hip runs the functions of
unbiased_nvfp4_gradient_amd/csrc/nvfp4_device.h, the code the kernels include):

* E2M1 encode (v_cvt_scalef32_pk_fp4_f32 with scale 1, two codes per byte at each of the four
  byte positions of a word): every binary32 with |y| < 8, both signs, +-0, against the
  oracle's nearest-even magnitude with the sign of y; the other three bytes stay untouched;
* E4M3 nearest-even (v_cvt_pk_fp8_f32 after the clamp at 448) and E4M3 round-up: every
  binary32 in [0, 448], and sampled values above 448, infinities and NaN;
* E2M1 decode (v_cvt_scalef32_pk_f32_fp4): all 256 code bytes at all four byte positions,
  bit for bit (so -0 for code 8);
* E4M3 values of the 128 codes;
* element SR on every binary32 in [0, 6] with the draw at its rounding threshold, and on
  sampled inputs; scale SR and Philox4x32-10 on sampled inputs;
* the MXFP4 block-scale exponent over every non-negative finite binary32.

These roundings are the whole of the contract's element and scale decisions (Telegram digest
quant_prune_distill post 640, "Method": round-to-nearest onto the +-6 grid, FP8 scales; the
itsolotime.com summary, Q1: the scale SR and its skip)."""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "helpers", "libconv_check.so")
CHUNK = 1 << 28


@pytest.fixture(scope="module")
def conv():
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is missing: build it with __graft_entry__.build()")
    h = ctypes.CDLL(LIB)
    P, u32, u64 = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64
    for name, args in (("conv_fp4_encode", [u32, u64, P, P, P]), ("conv_e4m3_rne", [u32, u64, P, P]),
                       ("conv_e4m3_up", [u32, u64, P, P]), ("conv_fp4_decode", [P, P]),
                       ("conv_e4m3_val", [P, P]), ("conv_scale_sr", [P, P, u64, P, P]),
                       ("conv_elem_sr", [P, P, u64, P, P]), ("conv_philox", [P, P, u64, P, P]),
                       ("conv_mx_exp", [u32, u64, P, P])):
        getattr(h, name).argtypes = args
        getattr(h, name).restype = ctypes.c_int
    return h


def _stream():
    return torch.cuda.current_stream(DEV).cuda_stream


def _bits(start, count):
    return np.arange(start, start + count, dtype=np.uint64).astype(np.uint32)


def _unpack(b):
    return np.stack([b & 15, b >> 4], axis=-1).reshape(-1)


@pytest.mark.parametrize("sign", [0, 1])
def test_e2m1_encode_every_float_below_8(conv, sign):
    base = 0x80000000 if sign else 0
    end = 0x41000000                                   # bits of 8.0: every |y| < 8
    print(f"case: E2M1 encode, sign {sign}, {end} floats", flush=True)
    buf = torch.empty(CHUNK // 2, dtype=torch.uint8, device=DEV)
    touched = torch.zeros(1, dtype=torch.int32, device=DEV)
    checked = 0
    for lo in range(0, end, CHUNK):
        n = min(CHUNK, end - lo)
        assert n % 2 == 0 and n // 2 <= buf.numel()
        assert conv.conv_fp4_encode(base + lo, n, buf.data_ptr(), touched.data_ptr(),
                                    _stream()) == 0
        got = buf[:n // 2].cpu().numpy()
        assert int(touched.item()) == 0, "a conversion touched another byte of its word"
        mags = _bits(lo, n).view(np.float32)           # |y|
        want = oracle.e2m1_rtn_mag_n(mags) | np.uint8(8 * sign)
        gu = _unpack(got)
        bad = np.flatnonzero(gu != want)
        assert bad.size == 0, (f"{bad.size} codes differ, first at bits "
                               f"{base + lo + int(bad[0]):#010x}: {gu[bad[0]]} vs {want[bad[0]]}")
        checked += n
    assert checked == end


@pytest.mark.parametrize("kind", ["rne", "up"])
def test_e4m3_every_float_to_448(conv, kind):
    fn = conv.conv_e4m3_rne if kind == "rne" else conv.conv_e4m3_up
    ref = oracle.e4m3_rne_sat_n if kind == "rne" else oracle.e4m3_up_n
    end = 0x43E00001                                   # every binary32 in [0, 448]
    print(f"case: E4M3 {kind}, {end} floats", flush=True)
    buf = torch.empty(CHUNK, dtype=torch.uint8, device=DEV)
    for lo in range(0, end, CHUNK):
        n = min(CHUNK, end - lo)
        assert fn(lo, n, buf.data_ptr(), _stream()) == 0
        got = buf[:n].cpu().numpy()
        want = ref(_bits(lo, n).view(np.float32))
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, (f"{bad.size} differ, first at bits {lo + int(bad[0]):#010x}: "
                               f"{got[bad[0]]:#04x} vs {want[bad[0]]:#04x}")
    # above 448: saturation, up to +inf, and NaN inputs (outside the contract) stay in range
    rng = np.random.default_rng(0)
    starts = np.concatenate([[0x43E00001, 0x7F800000, 0x7F800001, 0x7FC00000],
                             rng.integers(0x43E00001, 0x7F800000, 2000)])
    for st in starts:
        assert fn(int(st), 16, buf.data_ptr(), _stream()) == 0
        got = buf[:16].cpu().numpy()
        vals = _bits(int(st), 16).view(np.float32)
        want = np.where(np.isnan(vals), 0x7E, ref(np.where(np.isnan(vals), 448, vals)))
        assert np.array_equal(got, want), hex(int(st))


def test_e2m1_decode_every_code(conv):
    out = torch.empty(2048, dtype=torch.float32, device=DEV)
    assert conv.conv_fp4_decode(out.data_ptr(), _stream()) == 0
    got = out.cpu().numpy().reshape(4, 256, 2)
    vals = np.array([oracle.e2m1_value(c) for c in range(16)], dtype=np.float32)
    want = np.stack([vals[np.arange(256) & 15], vals[np.arange(256) >> 4]], axis=-1)
    for sel in range(4):
        assert np.array_equal(got[sel].view(np.uint32), want.view(np.uint32)), sel


def test_e4m3_values(conv):
    out = torch.empty(128, dtype=torch.float32, device=DEV)
    assert conv.conv_e4m3_val(out.data_ptr(), _stream()) == 0
    want = np.array([oracle.e4m3_value(c) for c in range(127)], dtype=np.float32)
    assert np.array_equal(out.cpu().numpy()[:127].view(np.uint32), want.view(np.uint32))


def test_scale_sr_sampled(conv):
    rng = np.random.default_rng(1)
    n = 1 << 22
    # every normal in [2^-6, 448) is equally likely by bit pattern; half the draws sit
    # within 4 units of a carry out of the 20 dropped bits
    c_bits = rng.integers(0x3C800000, 0x43E00000, n).astype(np.uint32)
    w = rng.integers(0, 2**32, n, dtype=np.uint64).astype(np.uint32)
    low = (c_bits & 0xFFFFF).astype(np.int64)
    near = np.arange(n) % 2 == 0
    add = np.clip((1 << 20) - low + rng.integers(-4, 5, n), 0, (1 << 20) - 1)
    w = np.where(near, (add << 12).astype(np.uint32) | (w & 0xFFF), w).astype(np.uint32)
    c = c_bits.view(np.float32)
    cd, wd = torch.from_numpy(c).to(DEV), torch.from_numpy(w.view(np.int32)).to(DEV)
    out = torch.empty(n, dtype=torch.uint8, device=DEV)
    assert conv.conv_scale_sr(cd.data_ptr(), wd.data_ptr(), n, out.data_ptr(), _stream()) == 0
    assert np.array_equal(out.cpu().numpy(), oracle.scale_sr_pairs_n(c, w))


def _elem_sr_codes(y, w):
    """Oracle codes of signed y with words w: magnitude of min(|y|, 6), sign bit iff y < 0."""
    mag = oracle.elem_sr_pairs_n(np.minimum(np.abs(y), np.float32(6)), w)
    return mag | ((y < 0).astype(np.uint8) << 3)


def test_elem_sr_sampled(conv):
    """Signed inputs, both element positions of the conversion, saturation above 6."""
    rng = np.random.default_rng(2)
    n = 1 << 22
    a = np.concatenate([rng.uniform(0, 6, n - 80).astype(np.float32),
                        np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6] * 8, dtype=np.float32),
                        np.array([6.5, 7, 8, 100, 1e30, 2.0**-130, 1e-9, 5.9999995] * 2,
                                 dtype=np.float32)])
    # every grid point and its float neighbours
    grid_nb = np.concatenate([np.nextafter(a[-80:-16], np.float32(0)),
                              np.nextafter(a[-80:-16], np.float32(7))])
    a[: grid_nb.size] = np.minimum(grid_nb, np.float32(6))
    perm = rng.permutation(n)                         # spread the specials over both positions
    a = a[perm]
    y = np.where((rng.integers(0, 2, n) == 1) & (a != 0), -a, a).astype(np.float32)
    w = rng.integers(0, 2**32, n, dtype=np.uint64).astype(np.uint32)
    yd, wd = torch.from_numpy(y).to(DEV), torch.from_numpy(w.view(np.int32)).to(DEV)
    out = torch.empty(n, dtype=torch.uint8, device=DEV)
    assert conv.conv_elem_sr(yd.data_ptr(), wd.data_ptr(), n, out.data_ptr(), _stream()) == 0
    got, want = out.cpu().numpy(), _elem_sr_codes(y, w)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, (f"{bad.size} mismatches from y = {y[bad[0]]!r}, w = {w[bad[0]]:#x}, "
                           f"position {bad[0] % 2}: {got[bad[0]]} != {want[bad[0]]}")


def test_elem_sr_every_magnitude_at_its_threshold(conv):
    """Element SR on every binary32 a in [0, 6], each with the draw just below the smallest
    draw that rounds it up (stays) or at it (goes up), the two alternating in pairs so that
    both element positions of the conversion see both: the decision at the exact boundary,
    for every input.  The threshold 2^22 - floor(frac * 2^22) only picks the draw; the
    expected magnitude comes from the oracle."""
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    top = 0x40C00000                                   # bits of 6.0, included
    end = (top + 1 + 7) // 8 * 8                       # whole groups of 8 (the tail repeats 6.0)
    chunk = 1 << 26
    rng = np.random.default_rng(5)
    print(f"case: element SR, {top + 1} magnitudes", flush=True)
    out = torch.empty(chunk, dtype=torch.uint8, device=DEV)
    for lo in range(0, end, chunk):
        n = min(chunk, end - lo)
        a = np.minimum(_bits(lo, n), np.uint32(top)).view(np.float32)
        ad = a.astype(np.float64)
        k = np.minimum(np.searchsorted(grid, ad, side="right") - 1, 6)
        first_up = 2**22 - np.floor((ad - grid[k]) / (grid[k + 1] - grid[k]) * 2.0**22)
        v = np.clip(first_up - 1 + ((np.arange(n) >> 1) & 1), 0, 2**22 - 1).astype(np.uint32)
        w = (v << np.uint32(10)) | rng.integers(0, 1024, n, dtype=np.uint32)
        ad_t, wd = torch.from_numpy(a).to(DEV), torch.from_numpy(w.view(np.int32)).to(DEV)
        assert conv.conv_elem_sr(ad_t.data_ptr(), wd.data_ptr(), n, out.data_ptr(),
                                 _stream()) == 0
        got = out[:n].cpu().numpy()
        want = oracle.elem_sr_pairs_n(a, w)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (f"{bad.size} mismatches from a = {a[bad[0]]!r}, v = {v[bad[0]]}, "
                               f"position {bad[0] % 2}: {got[bad[0]]} != {want[bad[0]]}")


def test_philox_sampled(conv):
    rng = np.random.default_rng(3)
    n = 1 << 18
    keys = rng.integers(0, 2**64, n, dtype=np.uint64)
    ctr = rng.integers(0, 2**32, (n, 4), dtype=np.uint64).astype(np.uint32)
    ctr[: n // 2, 1] = 0                      # the quantizers' counters: small indices,
    ctr[: n // 2, 2] = rng.integers(1, 4, n // 2)          # streams 1..3, axis 0 or 1
    ctr[: n // 2, 3] = rng.integers(0, 2, n // 2)
    kd = torch.from_numpy(keys.view(np.int64)).to(DEV)
    cd = torch.from_numpy(ctr.view(np.int32)).to(DEV)
    out = torch.empty((n, 4), dtype=torch.int32, device=DEV)
    assert conv.conv_philox(kd.data_ptr(), cd.data_ptr(), n, out.data_ptr(), _stream()) == 0
    assert np.array_equal(out.cpu().numpy().view(np.uint32), oracle.philox_n(keys, ctr))


def test_mx_scale_exponent_every_float(conv):
    """The MXFP4 block-scale exponent (frexp on the device) over every non-negative finite
    binary32, subnormals included, against the oracle's definition (the smallest e with
    6 * 2^e >= m, clamped to [-127, 127])."""
    end = 0x7F800000
    print(f"case: MXFP4 scale exponent, {end} floats", flush=True)
    buf = torch.empty(CHUNK, dtype=torch.uint8, device=DEV)
    for lo in range(0, end, CHUNK):
        n = min(CHUNK, end - lo)
        assert conv.conv_mx_exp(lo, n, buf.data_ptr(), _stream()) == 0
        got = buf[:n].cpu().numpy()
        want = oracle.mx_scale_byte_n(_bits(lo, n).view(np.float32))
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, (f"{bad.size} differ, first at bits {lo + int(bad[0]):#010x}: "
                               f"{got[bad[0]]} vs {want[bad[0]]}")
