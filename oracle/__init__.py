"""CPU oracle for the NVFP4 quantizers (MS-EDEN, SR, RTN, 4/6) -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package.  The product path (``unbiased_nvfp4_gradient_amd``) never imports it.

The arithmetic lives in ``nvfp4_oracle.c`` (plain C, IEEE binary32, no FMA contraction);
this module only compiles it with gcc and marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import NamedTuple, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libnvfp4_oracle.so")

MODE_RTN, MODE_SR, MODE_EDEN, MODE_FP46 = 0, 1, 2, 3
MODES = {"rtn": MODE_RTN, "sr": MODE_SR, "eden": MODE_EDEN, "fp46": MODE_FP46}
MARGIN_NONE = 0xFFFFFFFF

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, no FMA contraction, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
             "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"]
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # NVFP4_ORACLE_LIB names another build of nvfp4_oracle.c to load instead (the mutation
    # tests use it to check that the pins reject planted mistakes)
    other = os.environ.get("NVFP4_ORACLE_LIB")
    if not other:
        build()
    lib = ctypes.CDLL(other or _LIB_PATH)
    c = ctypes
    P = c.c_void_p
    i64, u64, i32, f32 = c.c_int64, c.c_uint64, c.c_int, c.c_float
    lib.oracle_philox4x32_10.argtypes = [u64, P, P]
    lib.oracle_signs.argtypes = [u64, P]
    lib.oracle_fwht128.argtypes = [P]
    lib.oracle_e4m3_value.argtypes = [c.c_uint8]
    lib.oracle_e4m3_value.restype = f32
    lib.oracle_e4m3_rne_sat.argtypes = [f32]
    lib.oracle_e4m3_rne_sat.restype = c.c_uint8
    lib.oracle_e4m3_up.argtypes = [f32]
    lib.oracle_e4m3_up.restype = c.c_uint8
    lib.oracle_e2m1_value.argtypes = [c.c_uint8]
    lib.oracle_e2m1_value.restype = f32
    lib.oracle_e2m1_rtn_mag.argtypes = [f32]
    lib.oracle_e2m1_rtn_mag.restype = i32
    lib.oracle_tensor_scale.argtypes = [i32, f32]
    lib.oracle_tensor_scale.restype = f32
    lib.oracle_amax.argtypes = [P, i64, i64, i32, i32, u64]
    lib.oracle_amax.restype = f32
    lib.oracle_quantize_vectors.argtypes = [i32, P, i64, i64, i32, i32, u64, u64, f32, P, i64,
                                            P, P, P, P]
    lib.oracle_quantize_vectors.restype = i32
    lib.oracle_quantize.argtypes = [i32, P, i64, i64, i32, i32, u64, u64, P, P, P, P, P]
    lib.oracle_quantize.restype = i32
    lib.oracle_quantize_strips.argtypes = [i32, P, i64, i64, i32, i32, u64, u64, i64, P, P, P,
                                           P, P]
    lib.oracle_quantize_strips.restype = i32
    lib.oracle_dequantize.argtypes = [P, P, f32, i64, i64, i32, u64, P]
    lib.oracle_dequantize.restype = i32
    lib.oracle_eden_internals.argtypes = [P, i64, i64, i32, u64, f32, i64, P, P, P, P]
    lib.oracle_eden_internals.restype = i32
    lib.oracle_scale_sr.argtypes = [f32, c.c_uint32]
    lib.oracle_scale_sr.restype = c.c_uint8
    lib.oracle_elem_sr_mag.argtypes = [f32, c.c_uint32]
    lib.oracle_elem_sr_mag.restype = i32
    for name in ("oracle_e4m3_rne_sat_n", "oracle_e4m3_up_n", "oracle_e2m1_rtn_mag_n"):
        getattr(lib, name).argtypes = [P, P, i64]
    lib.oracle_scale_sr_n.argtypes = [f32, P, P, i64]
    lib.oracle_elem_sr_mag_n.argtypes = [f32, P, P, i64]
    lib.oracle_margin_n.argtypes = [i32, P, P, P, i64]
    lib.oracle_mx_scale_exp.argtypes = [f32]
    lib.oracle_mx_scale_exp.restype = i32
    lib.oracle_mx_scale_exp_n.argtypes = [P, P, i64]
    lib.oracle_mx_quantize.argtypes = [i32, P, i64, i64, i32, i32, u64, u64, P, P]
    lib.oracle_mx_quantize.restype = i32
    lib.oracle_mx_dequantize.argtypes = [P, P, i64, i64, i32, u64, P]
    lib.oracle_mx_dequantize.restype = i32
    lib.oracle_scale_sr_pairs_n.argtypes = [P, P, P, i64]
    lib.oracle_elem_sr_pairs_n.argtypes = [P, P, P, i64]
    lib.oracle_philox_n.argtypes = [P, P, P, i64]
    lib.oracle_set_threads.argtypes = [i32]
    lib.oracle_get_threads.restype = i32
    _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _bf16_bits(x) -> np.ndarray:
    """Accept a uint16 array of bf16 bit patterns, or a torch bfloat16 tensor."""
    if isinstance(x, np.ndarray):
        assert x.dtype == np.uint16
        return np.ascontiguousarray(x)
    import torch  # only for the dtype reinterpretation of CPU tensors

    assert x.dtype == torch.bfloat16
    return np.ascontiguousarray(x.detach().cpu().contiguous().view(torch.int16).numpy()
                                .view(np.uint16))


# ---------------------------------------------------------------------------- primitives

def philox4x32_10(key: int, ctr) -> np.ndarray:
    lib = _load()
    c = np.asarray(ctr, dtype=np.uint32).copy()
    out = np.zeros(4, dtype=np.uint32)
    lib.oracle_philox4x32_10(key & (2**64 - 1), _ptr(c), _ptr(out))
    return out


def signs(rht_seed: int) -> np.ndarray:
    lib = _load()
    out = np.zeros(128, dtype=np.float32)
    lib.oracle_signs(rht_seed & (2**64 - 1), _ptr(out))
    return out


def fwht128(a) -> np.ndarray:
    lib = _load()
    v = np.ascontiguousarray(np.asarray(a, dtype=np.float32)).copy()
    assert v.shape == (128,)
    lib.oracle_fwht128(_ptr(v))
    return v


def e4m3_value(code: int) -> float:
    return float(_load().oracle_e4m3_value(code))


def e4m3_rne_sat(t: float) -> int:
    return int(_load().oracle_e4m3_rne_sat(t))


def e4m3_up(t: float) -> int:
    return int(_load().oracle_e4m3_up(t))


def e2m1_value(code: int) -> float:
    return float(_load().oracle_e2m1_value(code))


def e2m1_rtn_mag(a: float) -> int:
    return int(_load().oracle_e2m1_rtn_mag(a))


def scale_sr(c: float, w: int) -> int:
    return int(_load().oracle_scale_sr(c, w))


def elem_sr_mag(a: float, w: int) -> int:
    """Element SR magnitude of a in [0, 6] with random word w (the draw is w >> 10)."""
    return int(_load().oracle_elem_sr_mag(a, w))


def _map_u8(fn_name: str, values) -> np.ndarray:
    v = np.ascontiguousarray(np.asarray(values, dtype=np.float32))
    out = np.zeros(v.shape, dtype=np.uint8)
    getattr(_load(), fn_name)(_ptr(v), _ptr(out), v.size)
    return out


def e4m3_rne_sat_n(t) -> np.ndarray:
    return _map_u8("oracle_e4m3_rne_sat_n", t)


def e4m3_up_n(t) -> np.ndarray:
    return _map_u8("oracle_e4m3_up_n", t)


def e2m1_rtn_mag_n(a) -> np.ndarray:
    return _map_u8("oracle_e2m1_rtn_mag_n", a)


def scale_sr_n(c: float, words) -> np.ndarray:
    w = np.ascontiguousarray(np.asarray(words, dtype=np.uint32))
    out = np.zeros(w.shape, dtype=np.uint8)
    _load().oracle_scale_sr_n(c, _ptr(w), _ptr(out), w.size)
    return out


def elem_sr_mag_n(a: float, words) -> np.ndarray:
    u = np.ascontiguousarray(np.asarray(words, dtype=np.uint32))
    out = np.zeros(u.shape, dtype=np.uint8)
    _load().oracle_elem_sr_mag_n(a, _ptr(u), _ptr(out), u.size)
    return out


def scale_sr_pairs_n(c, words) -> np.ndarray:
    """Scale SR of each c[i] (normal, below 448) with its own random word words[i]."""
    cc = np.ascontiguousarray(np.asarray(c, dtype=np.float32))
    w = np.ascontiguousarray(np.asarray(words, dtype=np.uint32))
    out = np.zeros(cc.shape, dtype=np.uint8)
    _load().oracle_scale_sr_pairs_n(_ptr(cc), _ptr(w), _ptr(out), cc.size)
    return out


def elem_sr_pairs_n(a, words) -> np.ndarray:
    """Element SR magnitude of each a[i] in [0, 6] with its own random word words[i]."""
    aa = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = np.ascontiguousarray(np.asarray(words, dtype=np.uint32))
    out = np.zeros(aa.shape, dtype=np.uint8)
    _load().oracle_elem_sr_pairs_n(_ptr(aa), _ptr(u), _ptr(out), aa.size)
    return out


def philox_n(keys, ctrs) -> np.ndarray:
    """Philox4x32-10 words [n, 4] of keys [n] (uint64) and counters [n, 4] (uint32)."""
    k = np.ascontiguousarray(np.asarray(keys, dtype=np.uint64))
    c = np.ascontiguousarray(np.asarray(ctrs, dtype=np.uint32))
    out = np.zeros((k.size, 4), dtype=np.uint32)
    _load().oracle_philox_n(_ptr(k), _ptr(c), _ptr(out), k.size)
    return out


MARGIN_KINDS = {"e2m1": 0, "e4m3_rne": 1, "e4m3_up": 2, "scale_sr": 3, "elem_sr": 4, "ulp": 5}


def margin_n(kind: str, values, aux=None) -> np.ndarray:
    """Margin (ulps from the value to the boundary of the rounding it feeds) of each value:
    "e2m1" nearest of |v|, "e4m3_rne" / "e4m3_up" scale roundings of v >= 0, "scale_sr" of v
    with random word aux, "elem_sr" of v in [0, 6) with random word aux, "ulp" the distance
    between v and the float whose bits are aux."""
    v = np.ascontiguousarray(np.asarray(values, dtype=np.float32))
    a = np.zeros(v.shape, dtype=np.uint32) if aux is None else \
        np.ascontiguousarray(np.broadcast_to(np.asarray(aux, dtype=np.uint32), v.shape))
    out = np.zeros(v.shape, dtype=np.uint32)
    _load().oracle_margin_n(MARGIN_KINDS[kind], _ptr(v), _ptr(a), _ptr(out), v.size)
    return out


def tensor_scale(mode: str, amax: float) -> float:
    return float(_load().oracle_tensor_scale(MODES[mode], amax))


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def get_threads() -> int:
    return int(_load().oracle_get_threads())


# ---------------------------------------------------------------------------- quantizers

class Quantized(NamedTuple):
    codes: np.ndarray          # uint8 [vecs, n/2], low nibble = even position
    scales: np.ndarray         # uint8 [vecs, n/16], E4M3FN bits
    g: float                   # fp32 tensor scale
    elem_margin: Optional[np.ndarray]   # uint32 [vecs, n] (ulps to the rounding boundary)
    scale_margin: Optional[np.ndarray]  # uint32 [vecs, n/16]


def _uses_rht(mode: str, rht: bool) -> bool:
    return bool(rht) or mode == "eden"


def amax(x, axis: int, rht: bool, rht_seed: int) -> float:
    lib = _load()
    xb = _bf16_bits(x)
    rows, cols = xb.shape
    return float(lib.oracle_amax(_ptr(xb), rows, cols, axis, int(rht), rht_seed))


def quantize(mode: str, x, axis: int = 0, seed: int = 0, rht: bool = False, rht_seed: int = 0,
             margins: bool = True) -> Quantized:
    """Whole-layout quantization of a bf16 matrix (axis 0: rows, axis 1: columns)."""
    lib = _load()
    xb = _bf16_bits(x)
    rows, cols = xb.shape
    nvec, n = (rows, cols) if axis == 0 else (cols, rows)
    codes = np.zeros((nvec, n // 2), dtype=np.uint8)
    scales = np.zeros((nvec, n // 16), dtype=np.uint8)
    em = np.zeros((nvec, n), dtype=np.uint32) if margins else None
    sm = np.zeros((nvec, n // 16), dtype=np.uint32) if margins else None
    g = np.zeros(1, dtype=np.float32)
    rc = lib.oracle_quantize(MODES[mode], _ptr(xb), rows, cols, axis, int(rht), seed, rht_seed,
                             _ptr(codes), _ptr(scales), _ptr(g), _ptr(em), _ptr(sm))
    if rc != 0:
        raise ValueError(f"oracle_quantize: unsupported shape {xb.shape} for axis {axis}")
    return Quantized(codes, scales, float(g[0]), em, sm)


class StripQuantized(NamedTuple):
    codes: np.ndarray          # uint8 [vecs, n/2]
    scales: np.ndarray         # uint8 [vecs, n/16]
    g: np.ndarray              # fp32 [ceil(vecs / strip)]: strip s covers vectors s*strip ..
    elem_margin: Optional[np.ndarray]
    scale_margin: Optional[np.ndarray]


def quantize_strips(mode: str, x, axis: int = 0, seed: int = 0, rht: bool = False,
                    rht_seed: int = 0, strip: int = 128, margins: bool = True) -> StripQuantized:
    """Strip-local quantization: each run of `strip` consecutive vectors of the layout takes
    its FP32 scale from its own maximum (the CTA-local variant)."""
    lib = _load()
    xb = _bf16_bits(x)
    rows, cols = xb.shape
    nvec, n = (rows, cols) if axis == 0 else (cols, rows)
    codes = np.zeros((nvec, n // 2), dtype=np.uint8)
    scales = np.zeros((nvec, n // 16), dtype=np.uint8)
    em = np.zeros((nvec, n), dtype=np.uint32) if margins else None
    sm = np.zeros((nvec, n // 16), dtype=np.uint32) if margins else None
    g = np.zeros(-(-nvec // strip), dtype=np.float32)
    rc = lib.oracle_quantize_strips(MODES[mode], _ptr(xb), rows, cols, axis, int(rht), seed,
                                    rht_seed, strip, _ptr(codes), _ptr(scales), _ptr(g), _ptr(em),
                                    _ptr(sm))
    if rc != 0:
        raise ValueError(f"oracle_quantize_strips: unsupported shape {xb.shape} for axis {axis}")
    return StripQuantized(codes, scales, g, em, sm)


def dequantize_strips(codes: np.ndarray, scales: np.ndarray, g: np.ndarray, strip: int = 128,
                      rht: bool = False, rht_seed: int = 0) -> np.ndarray:
    """Decode strip-local outputs: vectors s*strip .. with g[s]."""
    nvec = codes.shape[0]
    parts = [dequantize(codes[v0:v0 + strip], scales[v0:v0 + strip], float(g[v0 // strip]),
                        rht, rht_seed) for v0 in range(0, nvec, strip)]
    if not parts:
        return np.zeros((0, codes.shape[1] * 2), dtype=np.float32)
    return np.concatenate(parts, axis=0)


def quantize_vectors(mode: str, x, axis: int, vec_ids, g: float, seed: int = 0,
                     rht: bool = False, rht_seed: int = 0, margins: bool = True) -> Quantized:
    """Quantize only the listed vectors of a layout, given the tensor scale g."""
    lib = _load()
    xb = _bf16_bits(x)
    rows, cols = xb.shape
    n = cols if axis == 0 else rows
    ids = np.ascontiguousarray(np.asarray(vec_ids, dtype=np.int64))
    nv = ids.shape[0]
    codes = np.zeros((nv, n // 2), dtype=np.uint8)
    scales = np.zeros((nv, n // 16), dtype=np.uint8)
    em = np.zeros((nv, n), dtype=np.uint32) if margins else None
    sm = np.zeros((nv, n // 16), dtype=np.uint32) if margins else None
    rc = lib.oracle_quantize_vectors(MODES[mode], _ptr(xb), rows, cols, axis,
                                     int(_uses_rht(mode, rht)), seed, rht_seed, g, _ptr(ids), nv,
                                     _ptr(codes), _ptr(scales), _ptr(em), _ptr(sm))
    if rc != 0:
        raise ValueError("oracle_quantize_vectors: bad shape or vector id")
    return Quantized(codes, scales, float(g), em, sm)


def dequantize(codes: np.ndarray, scales: np.ndarray, g: float, rht: bool = False,
               rht_seed: int = 0) -> np.ndarray:
    lib = _load()
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    nvec, n = codes.shape[0], codes.shape[1] * 2
    out = np.zeros((nvec, n), dtype=np.float32)
    rc = lib.oracle_dequantize(_ptr(codes), _ptr(scales), g, nvec, n, int(rht), rht_seed,
                               _ptr(out))
    if rc != 0:
        raise ValueError("oracle_dequantize: bad shape")
    return out


def eden_internals(x, axis: int, rht_seed: int, g: float, vec: int):
    """r, q (rotated values and their RTN dequantization), S per group, c per block."""
    lib = _load()
    xb = _bf16_bits(x)
    rows, cols = xb.shape
    n = cols if axis == 0 else rows
    r = np.zeros(n, dtype=np.float32)
    q = np.zeros(n, dtype=np.float32)
    S = np.zeros(n // 128, dtype=np.float32)
    c = np.zeros(n // 16, dtype=np.float32)
    rc = lib.oracle_eden_internals(_ptr(xb), rows, cols, axis, rht_seed, g, vec, _ptr(r), _ptr(q),
                                   _ptr(S), _ptr(c))
    if rc != 0:
        raise ValueError("oracle_eden_internals: bad shape")
    return r, q, S, c


def unpack_codes(codes: np.ndarray) -> np.ndarray:
    """[vecs, n/2] packed bytes -> [vecs, n] 4-bit codes (low nibble first)."""
    lo = codes & 0x0F
    hi = codes >> 4
    return np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)


# ---------------------------------------------------------------------------- MXFP4 contract

class MXQuantized(NamedTuple):
    codes: np.ndarray          # uint8 [vecs, n/2], low nibble = even position
    scales: np.ndarray         # uint8 [vecs, n/32], E8M0: 2^(byte - 127)


def mx_scale_exp(m: float) -> int:
    """Smallest e with 6 * 2^e >= m (clamped to [-127, 127]; -127 for m = 0)."""
    return int(_load().oracle_mx_scale_exp(m))


def mx_scale_byte_n(m) -> np.ndarray:
    """E8M0 bytes (e + 127) of the MXFP4 block scale for each block maximum m."""
    return _map_u8("oracle_mx_scale_exp_n", m)


def mx_quantize(x, axis: int = 0, sr: bool = False, seed: int = 0, rht: bool = False,
                rht_seed: int = 0) -> MXQuantized:
    """MXFP4 (E2M1 elements, one E8M0 scale per 32) of one layout, RTN or SR."""
    lib = _load()
    xb = _bf16_bits(x)
    rows, cols = xb.shape
    nvec, n = (rows, cols) if axis == 0 else (cols, rows)
    codes = np.zeros((nvec, n // 2), dtype=np.uint8)
    scales = np.zeros((nvec, n // 32), dtype=np.uint8)
    rc = lib.oracle_mx_quantize(int(bool(sr)), _ptr(xb), rows, cols, axis, int(bool(rht)), seed,
                                rht_seed, _ptr(codes), _ptr(scales))
    if rc != 0:
        raise ValueError(f"oracle_mx_quantize: unsupported shape {xb.shape} for axis {axis}")
    return MXQuantized(codes, scales)


def mx_k_tile(codes: np.ndarray, scales: np.ndarray):
    """The K-tiled storage of an MXFP4 layout (the same bytes, rearranged; n a multiple of 128):
    code byte j of vector v goes to [j // 64][v][j % 64] and scale byte s to [s // 4][v][s % 4],
    so each 128-element step of K holds every vector's 64 code bytes, then every vector's 4
    scale bytes, in one piece."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    vecs, half = codes.shape
    if half % 64 or scales.shape != (vecs, half // 16):
        raise ValueError("mx_k_tile: n must be a multiple of 128 with n/32 scale bytes per vector")
    tiles = half // 64
    tc = np.ascontiguousarray(codes.reshape(vecs, tiles, 64).transpose(1, 0, 2))
    ts = np.ascontiguousarray(scales.reshape(vecs, tiles, 4).transpose(1, 0, 2))
    return tc, ts


def mx_dequantize(codes: np.ndarray, scales: np.ndarray, rht: bool = False,
                  rht_seed: int = 0) -> np.ndarray:
    lib = _load()
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    nvec, n = codes.shape[0], codes.shape[1] * 2
    out = np.zeros((nvec, n), dtype=np.float32)
    rc = lib.oracle_mx_dequantize(_ptr(codes), _ptr(scales), nvec, n, int(bool(rht)), rht_seed,
                                  _ptr(out))
    if rc != 0:
        raise ValueError("oracle_mx_dequantize: bad shape")
    return out
