"""Exact reference for the NVFP4 GEMM consumer: operand values from the codes and scales in
fp64 (sign * E4M3(scale) * magnitude; the tensor scales apart), and the bound of FP32
accumulation, |dC| <= 2 K u sum_k |a_k b_k| + 4 u |C| (u = 2^-24)."""
import numpy as np

import oracle

U = 2.0 ** -24
E2M1 = np.array([oracle.e2m1_value(c) for c in range(16)], dtype=np.float64)
E4M3 = np.array([oracle.e4m3_value(c) for c in range(127)] + [np.nan], dtype=np.float64)


def exact_rows(t, rows):
    """fp64 values of the listed vectors of a device NVFP4 layout (tensor scale apart)."""
    codes = oracle.unpack_codes(t.codes[rows].cpu().numpy())
    scales = E4M3[t.scales[rows].cpu().numpy()]
    return E2M1[codes] * np.repeat(scales, 16, axis=1)


def check_entries(c, a, b, rows, cols, f, strips=False):
    """C[rows][cols] of C = f * gA * gB * A B^T against the exact product, within the bound.
    With strips=True, gA and gB are per 128 rows of each operand (strip-local scales)."""
    rows, cols = np.asarray(rows), np.asarray(cols)
    if strips:
        ga = a.tensor_scale.cpu().numpy().astype(np.float64)[rows // 128][:, None]
        gb = b.tensor_scale.cpu().numpy().astype(np.float64)[cols // 128][None, :]
    else:
        ga, gb = float(a.tensor_scale.cpu()[0]), float(b.tensor_scale.cpu()[0])
    A = exact_rows(a, rows)
    B = exact_rows(b, cols)
    ref = (A @ B.T) * ga * gb * f
    mag = (np.abs(A) @ np.abs(B).T) * ga * gb * f
    K = A.shape[1]
    got = c[np.ix_(rows, cols)].cpu().numpy().astype(np.float64)
    bound = 2 * K * U * mag + 4 * U * np.abs(ref) + 1e-30
    assert np.all(np.abs(got - ref) <= bound), np.max(np.abs(got - ref) / bound)
    return got, ref


def mx_exact(codes, scales):
    """fp64 values of row-major MXFP4 vectors: sign * magnitude * 2^(scale byte - 127)."""
    c = oracle.unpack_codes(np.asarray(codes))
    sc = np.exp2(np.asarray(scales).astype(np.float64) - 127)
    return E2M1[c] * np.repeat(sc, 32, axis=1)


def check_mx_entries(c, a_codes, a_scales, b_codes, b_scales, f):
    """Every entry of C = f * A B^T of two MXFP4 operands (row-major numpy codes and scales)
    against the exact product, within the bound of FP32 accumulation."""
    A, B = mx_exact(a_codes, a_scales), mx_exact(b_codes, b_scales)
    ref = (A @ B.T) * f
    mag = (np.abs(A) @ np.abs(B).T) * f
    K = A.shape[1]
    got = c.cpu().numpy().astype(np.float64)
    bound = 2 * K * U * mag + 4 * U * np.abs(ref) + 1e-300
    assert np.all(np.abs(got - ref) <= bound), np.max(np.abs(got - ref) / bound)
    return got, ref
