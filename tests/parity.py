"""Parity rule between the GPU library and the oracle.

Packed codes and scales must match bit for bit, except where the oracle's pre-rounding fp32
value lies within 2 ulp of the boundary of the rounding it feeds (the oracle exports that
distance per code and per scale).  Outputs that depend on an excused mismatch are excused
too: every code of a block whose scale rounding is within the band, and (MS-EDEN) every
scale of a group in which a code mismatch was excused, since the EDEN ratio then moves.
Excused mismatches must stay at or below 1e-5 of each output kind; unexcused ones at 0.
The tensor scale is an exact function of the exact amax and must match exactly.

The kernels compute the contract's binary32 steps in the oracle's order, so the tests hold
them to the stricter bar: no mismatch at all (STRICT).  The band is still computed, so a
failure report says whether the differing outputs sit on a rounding boundary.
"""
from dataclasses import dataclass

import numpy as np

import oracle

BAND = 2
EXCUSED_RATE = 1e-5
STRICT = True


@dataclass
class Report:
    codes: int
    scales: int
    code_mismatch: int
    code_excused: int
    scale_mismatch: int
    scale_excused: int

    def ok(self) -> bool:
        if STRICT:
            return self.code_mismatch == 0 and self.scale_mismatch == 0
        return (self.code_mismatch == self.code_excused and
                self.scale_mismatch == self.scale_excused and
                self.code_excused <= EXCUSED_RATE * self.codes + 0 and
                self.scale_excused <= max(EXCUSED_RATE * self.scales, 0))


def compare(mode: str, codes: np.ndarray, scales: np.ndarray, ref: oracle.Quantized) -> Report:
    assert codes.shape == ref.codes.shape and scales.shape == ref.scales.shape
    gc = oracle.unpack_codes(codes)
    rc = oracle.unpack_codes(ref.codes)
    cm = gc != rc
    sm = scales != ref.scales
    em = ref.elem_margin
    smg = ref.scale_margin
    block_band = smg <= BAND                                  # [vecs, nblk]
    code_exc = cm & ((em <= BAND) | np.repeat(block_band, 16, axis=1))
    scale_exc = sm & block_band
    if mode == "eden" and code_exc.any():
        nv, n = gc.shape
        grp_hit = code_exc.reshape(nv, n // 128, 128).any(axis=2)     # [vecs, groups]
        scale_exc |= sm & np.repeat(grp_hit, 8, axis=1)
    return Report(int(gc.size), int(scales.size), int(cm.sum()), int(code_exc.sum()),
                  int(sm.sum()), int(scale_exc.sum()))


def assert_parity(mode, codes, scales, g, ref: oracle.Quantized, what=""):
    assert np.float32(g) == np.float32(ref.g), f"{what}: tensor scale {g!r} != oracle {ref.g!r}"
    rep = compare(mode, codes, scales, ref)
    assert rep.ok(), f"{what}: {rep}"
    return rep


def assert_same_floats(got: np.ndarray, ref: np.ndarray, what="", zero_sign_free=False):
    """Bit patterns equal.  With zero_sign_free, a zero may carry either sign (the rotated
    dequantizer carries a per-lane sign through its butterfly, so a zero output's sign follows
    its own order of operations, not the oracle's); every nonzero value must still match bit
    for bit."""
    g = np.ascontiguousarray(got, dtype=np.float32).view(np.uint32)
    r = np.ascontiguousarray(ref, dtype=np.float32).view(np.uint32)
    same = g == r
    if zero_sign_free:
        same |= ((g & 0x7FFFFFFF) == 0) & ((r & 0x7FFFFFFF) == 0)
    bad = np.flatnonzero(~same)
    assert bad.size == 0, (f"{what}: {bad.size} values differ, first at {bad[0]}: "
                           f"{got.reshape(-1)[bad[0]]!r} vs {ref.reshape(-1)[bad[0]]!r}")
