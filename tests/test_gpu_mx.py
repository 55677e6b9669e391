"""The MXFP4 recipe on the GPU: the producer (mxfp4_quantize) against the oracle's MXFP4
quantizer bit for bit, in the row-major and the K-tiled layout, and the native FP4 matrix-core
consumer (mxfp4_gemm) against an fp64 product of the exact operand values, within the bound of
FP32 accumulation (|dC| <= 2 K u sum_k |a_k b_k| + 4 u |C|, u = 2^-24); K-tiled operands give
the row-major operands' C bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import unbiased_nvfp4_gradient_amd as nv
import workloads
from guards import MARGIN, SENTINEL

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
U = 2.0 ** -24
E2M1 = np.array([oracle.e2m1_value(c) for c in range(16)], dtype=np.float64)


def _guarded_mx(vecs, n, k_tiled=False):
    """An MXFP4 layout whose two tensors sit inside sentinel margins."""
    bufs = []
    views = []
    shapes = ((n // 128, vecs, 64), (n // 128, vecs, 4)) if k_tiled else \
        ((vecs, n // 2), (vecs, n // 32))
    for shape in shapes:
        nbytes = int(np.prod(shape))
        buf = torch.full((MARGIN + nbytes + MARGIN,), SENTINEL, dtype=torch.uint8, device=DEV)
        bufs.append((buf, nbytes))
        views.append(buf[MARGIN:MARGIN + nbytes].view(shape))
    return nv.MXFP4(*views, k_tiled), bufs


def _intact(bufs):
    return all(bool((b[:MARGIN] == SENTINEL).all()) and bool((b[MARGIN + n:] == SENTINEL).all())
               for b, n in bufs)


def check_mx(x, layouts, sr, rht, seed=5, rht_seed=7, what="", k_tiled=False):
    xd = x.to(DEV)
    rows, cols = xd.shape
    row, bufs_r = _guarded_mx(rows, cols, k_tiled) if "row" in layouts else (None, [])
    col, bufs_c = _guarded_mx(cols, rows, k_tiled) if "col" in layouts else (None, [])
    q = nv.mxfp4_quantize(xd, sr=sr, seed=seed, rht=rht, rht_seed=rht_seed, layouts=layouts,
                          out=nv.MXQuantized(row, col))
    torch.cuda.synchronize()
    assert _intact(bufs_r + bufs_c), f"{what}: a write landed outside an output buffer"
    xb = workloads.bf16_bits(x)
    for axis, t in ((0, q.row), (1, q.col)):
        if t is None:
            continue
        ref = oracle.mx_quantize(xb, axis=axis, sr=sr, seed=seed, rht=rht, rht_seed=rht_seed)
        rc, rs = oracle.mx_k_tile(ref.codes, ref.scales) if k_tiled else (ref.codes, ref.scales)
        codes, scales = t.codes.cpu().numpy(), t.scales.cpu().numpy()
        cm = int(np.count_nonzero(codes != rc))
        sm = int(np.count_nonzero(scales != rs))
        assert cm == 0 and sm == 0, f"{what} axis={axis}: {cm} code bytes, {sm} scales differ"
    return q


@pytest.mark.parametrize("sr,rht", [(False, False), (True, False), (False, True), (True, True)])
@pytest.mark.parametrize("layouts", [("row",), ("col",), ("row", "col")])
def test_mx_quantize_config1(sr, rht, layouts):
    print(f"case: MXFP4 c1 sr={sr} rht={rht} {layouts}", flush=True)
    check_mx(workloads.c1(), layouts, sr, rht, what="c1")


@pytest.mark.parametrize("shape,sr,rht,layouts", [
    ((200, 256), True, True, ("row",)),            # ragged rows: partial tiles
    ((256, 200), False, False, ("col",)),          # n = 256, rows % 128 != 0 elsewhere
    ((96, 160), True, False, ("row", "col")),      # n % 128 != 0: partial groups, odd n/32
    ((32, 32), False, False, ("row", "col")),      # one block
    ((384, 640), True, True, ("row", "col")),      # several tiles
])
def test_mx_quantize_ragged(shape, sr, rht, layouts):
    print(f"case: MXFP4 {shape} sr={sr} rht={rht} {layouts}", flush=True)
    check_mx(workloads.normal(shape, seed=sum(shape)), layouts, sr, rht, what=f"{shape}")


def test_mx_quantize_extremes_and_zeros():
    """Per-row magnitudes 1e-30..1e30 (scale exponents at the clamp), all-zero rows, -0."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((256, 512)) * 10.0 ** rng.uniform(-30, 30, (256, 1))
    x[:16] = 0.0
    x[16:32] = -0.0
    xt = workloads.to_bf16(x)
    print("case: MXFP4 extremes and zeros", flush=True)
    for sr, rht in ((False, False), (True, True), (True, False)):
        check_mx(xt, ("row", "col"), sr, rht, what=f"extremes sr={sr} rht={rht}")


@pytest.mark.parametrize("sr,rht", [(True, True), (False, True), (True, False)])
def test_mx_quantize_config4_full(sr, rht):
    """16384 x 8192, both layouts in one call: every output."""
    print(f"case: MXFP4 c4 sr={sr} rht={rht} both layouts, every output", flush=True)
    check_mx(workloads.c4(), ("row", "col"), sr, rht, seed=1, rht_seed=1, what="c4")


@pytest.mark.parametrize("shape,sr,rht,layouts", [
    ((256, 1024), False, False, ("row", "col")),
    ((256, 1024), True, True, ("row", "col")),
    ((200, 256), True, True, ("row",)),            # ragged vectors: partial tiles
    ((384, 640), False, True, ("row", "col")),     # several tiles along both dims
    ((128, 384), True, False, ("col",)),           # one K tile of 128 vectors' columns
])
def test_mx_quantize_k_tiled(shape, sr, rht, layouts):
    """The K-tiled layout: the oracle's codes and scales rearranged by its definition, every
    byte, with sentinel margins around both tensors."""
    print(f"case: MXFP4 K-tiled {shape} sr={sr} rht={rht} {layouts}", flush=True)
    check_mx(workloads.normal(shape, seed=sum(shape) + 1), layouts, sr, rht, what=f"{shape}",
             k_tiled=True)


def test_mx_quantize_k_tiled_config4_full():
    """16384 x 8192, both layouts K-tiled (the benchmark GEMM's A takes the row layout)."""
    print("case: MXFP4 c4 K-tiled sr=True rht=True both layouts, every output", flush=True)
    check_mx(workloads.c4(), ("row", "col"), True, True, seed=1, rht_seed=1, what="c4 K-tiled",
             k_tiled=True)


def _exact(t, rows):
    codes = oracle.unpack_codes(t.codes[rows].cpu().numpy())
    scale = np.exp2(t.scales[rows].cpu().numpy().astype(np.float64) - 127)
    return E2M1[codes] * np.repeat(scale, 32, axis=1)


def check_gemm(c, a, b, rows, cols, f):
    A, B = _exact(a, rows), _exact(b, cols)
    ref = (A @ B.T) * f
    mag = (np.abs(A) @ np.abs(B).T) * f
    K = A.shape[1]
    got = c[np.ix_(rows, cols)].cpu().numpy().astype(np.float64)
    bound = 2 * K * U * mag + 4 * U * np.abs(ref) + 1e-300
    worst = float(np.max(np.abs(got - ref) / bound))
    assert worst <= 1.0, worst
    return got, ref


# K % 512 == 0 takes the 256-wide K step kernel (512, 1024, 1536, 2048), other K the 128-step
# one; M and N that are not multiples of 256 exercise the clamped rows of partial tiles
@pytest.mark.parametrize("M,N,K", [(256, 256, 128), (512, 256, 384), (96, 160, 256),
                                   (288, 544, 1024), (256, 256, 512), (64, 96, 1536),
                                   (544, 288, 2048)])
def test_mx_gemm_small(M, N, K):
    print(f"case: MXFP4 gemm M={M} N={N} K={K}", flush=True)
    x = workloads.normal((M, K), seed=M + K).to(DEV)
    w = workloads.normal((N, K), seed=N + K + 1, scale=0.02).to(DEV)
    a = nv.mxfp4_quantize(x, sr=True, seed=3, rht=True, rht_seed=9).row
    b = nv.mxfp4_quantize(w, rht=True, rht_seed=9).row
    c = nv.mxfp4_gemm(a, b, rotated_pair=True)
    torch.cuda.synchronize()
    got, _ = check_gemm(c, a, b, np.arange(M), np.arange(N), 2.0 ** -7)
    xw = (x.float() @ w.float().T).cpu().numpy()
    assert np.linalg.norm(got - xw) / np.linalg.norm(xw) < 0.25


@pytest.mark.parametrize("M,N,K", [(256, 256, 128), (96, 160, 256), (288, 544, 1024),
                                   (64, 96, 1536), (544, 288, 2048), (512, 256, 384)])
def test_mx_gemm_k_tiled_matches_row_major(M, N, K):
    """K-tiled operands (the same quantization stored K-tiled) give C bit for bit equal to the
    row-major operands' (both kernels add the 64-element products over K in the same order),
    so the row-major GEMM's bound check covers them too; checked against the bound as well."""
    print(f"case: MXFP4 gemm K-tiled M={M} N={N} K={K}", flush=True)
    x = workloads.normal((M, K), seed=M + K + 2).to(DEV)
    w = workloads.normal((N, K), seed=N + K + 3, scale=0.02).to(DEV)
    a = nv.mxfp4_quantize(x, sr=True, seed=3, rht=True, rht_seed=9).row
    b = nv.mxfp4_quantize(w, rht=True, rht_seed=9).row
    at = nv.mxfp4_quantize(x, sr=True, seed=3, rht=True, rht_seed=9, k_tiled=True).row
    bt = nv.mxfp4_quantize(w, rht=True, rht_seed=9, k_tiled=True).row
    c = nv.mxfp4_gemm(a, b, rotated_pair=True)
    ct = nv.mxfp4_gemm(at, bt, rotated_pair=True)
    torch.cuda.synchronize()
    tc, ts = oracle.mx_k_tile(a.codes.cpu().numpy(), a.scales.cpu().numpy())
    assert np.array_equal(at.codes.cpu().numpy(), tc) and np.array_equal(at.scales.cpu().numpy(), ts)
    assert torch.equal(c.view(torch.int32), ct.view(torch.int32))
    check_gemm(ct, a, b, np.arange(M), np.arange(N), 2.0 ** -7)


def test_mx_gemm_k_tiled_config4_full():
    """The benchmark's shape, 16384 x 8192 x 8192: the K-tiled GEMM equals the row-major one on
    every entry of C, bit for bit."""
    print("case: MXFP4 gemm c4 K-tiled against row-major, every entry", flush=True)
    x, w = workloads.c4().to(DEV), workloads.c4w().to(DEV)
    c = nv.mxfp4_gemm(nv.mxfp4_quantize(x, sr=True, seed=1, rht=True, rht_seed=1).row,
                      nv.mxfp4_quantize(w, rht=True, rht_seed=1).row, rotated_pair=True)
    ct = nv.mxfp4_gemm(nv.mxfp4_quantize(x, sr=True, seed=1, rht=True, rht_seed=1,
                                         k_tiled=True).row,
                       nv.mxfp4_quantize(w, rht=True, rht_seed=1, k_tiled=True).row,
                       rotated_pair=True)
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int32), ct.view(torch.int32))


def test_mx_gemm_wide_scales():
    """Operands whose 32-blocks span 2^-60..2^60: the matrix core applies every block's own
    power-of-two scale (no tensor scale to hide a wrong one)."""
    print("case: MXFP4 gemm with wide block scales", flush=True)
    rng = np.random.default_rng(8)
    x = rng.standard_normal((128, 512)) * np.exp2(rng.integers(-30, 30, (128, 16))).repeat(32, 1)
    w = rng.standard_normal((96, 512)) * np.exp2(rng.integers(-30, 30, (96, 16))).repeat(32, 1)
    a = nv.mxfp4_quantize(workloads.to_bf16(x).to(DEV)).row
    b = nv.mxfp4_quantize(workloads.to_bf16(w).to(DEV)).row
    c = nv.mxfp4_gemm(a, b)
    torch.cuda.synchronize()
    check_gemm(c, a, b, np.arange(128), np.arange(96), 1.0)


def test_mx_gemm_config4_sampled():
    """M = 16384, N = 8192, K = 8192 (the benchmark's GEMM shape): SR+RHT activations against
    an RTN+RHT weight, sampled rows and columns of C."""
    print("case: MXFP4 gemm c4 M=16384 N=8192 K=8192 sampled", flush=True)
    a = nv.mxfp4_quantize(workloads.c4().to(DEV), sr=True, seed=1, rht=True, rht_seed=1).row
    b = nv.mxfp4_quantize(workloads.c4w().to(DEV), rht=True, rht_seed=1).row
    c = nv.mxfp4_gemm(a, b, rotated_pair=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([[0, 16383], rng.choice(16384, 40, replace=False)]))
    cols = np.unique(np.concatenate([[0, 8191], rng.choice(8192, 40, replace=False)]))
    check_gemm(c, a, b, rows, cols, 2.0 ** -7)


def test_mx_errors():
    print("case: MXFP4 argument errors", flush=True)
    x = workloads.normal((256, 200), seed=1).to(DEV)
    with pytest.raises(nv.NVFP4Error) as e:
        nv.mxfp4_quantize(x, rht=True)                     # 200 % 128 != 0
    assert e.value.status == nv.ERR_SHAPE
    q = nv.mxfp4_quantize(workloads.normal((64, 256), seed=2).to(DEV)).row
    r = nv.MXFP4(q.codes[:, :64].contiguous(), q.scales[:, :4].contiguous())  # K = 128
    with pytest.raises(nv.NVFP4Error):
        nv.mxfp4_gemm(q, nv.MXFP4(q.codes[:48].contiguous(), q.scales[:48].contiguous()))
    c = nv.mxfp4_gemm(r, r)
    torch.cuda.synchronize()
    assert c.shape == (64, 64)
    t = nv.mxfp4_quantize(workloads.normal((64, 256), seed=2).to(DEV), k_tiled=True).row
    with pytest.raises(ValueError):
        nv.mxfp4_gemm(q, t)                                # one row-major, one K-tiled
    with pytest.raises(ValueError):
        nv.mxfp4_quantize(x, k_tiled=True)                 # K-tiled needs n % 128 (200)


def test_mx_graph_capture_and_replay():
    """The MXFP4 path in a HIP graph: K-tiled SR quantization of both layouts of an input and of
    a weight, then the FP4 GEMM of the row layouts; each of four replays (outputs cleared and
    other work run eagerly in between) gives the eager results bit for bit."""
    print("case: HIP graph capture of mxfp4_quantize (K-tiled) + mxfp4_gemm, 4 replays",
          flush=True)
    x = workloads.normal((384, 512), seed=91).to(DEV)
    w = workloads.normal((256, 512), seed=92, scale=0.02).to(DEV)
    other = workloads.normal((256, 256), seed=93).to(DEV)
    qx = nv.MXQuantized(nv.empty_mx_layout(384, 512, DEV, True), nv.empty_mx_layout(512, 384, DEV, True))
    qw = nv.MXQuantized(nv.empty_mx_layout(256, 512, DEV, True), None)
    c = torch.empty((384, 256), dtype=torch.float32, device=DEV)
    rx = nv.mxfp4_quantize(x, sr=True, seed=4, rht=True, rht_seed=5, layouts=("row", "col"),
                           k_tiled=True)
    rw = nv.mxfp4_quantize(w, rht=True, rht_seed=5, k_tiled=True)
    rc = nv.mxfp4_gemm(rx.row, rw.row, rotated_pair=True)
    torch.cuda.synchronize()

    def work():
        nv.mxfp4_quantize(x, sr=True, seed=4, rht=True, rht_seed=5, layouts=("row", "col"),
                          out=qx)
        nv.mxfp4_quantize(w, rht=True, rht_seed=5, out=qw)
        nv.mxfp4_gemm(qx.row, qw.row, rotated_pair=True, out=c)

    s = torch.cuda.Stream(device=DEV)
    s.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(s):
        work()                                                # warm-up off the capture
    torch.cuda.current_stream(DEV).wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for rep in range(4):
        for t in (qx.row.codes, qx.row.scales, qx.col.codes, qx.col.scales, qw.row.codes,
                  qw.row.scales, c):
            t.zero_()
        nv.mxfp4_quantize(other, sr=True, seed=rep, layouts=("row", "col"))   # eager work between
        g.replay()
        torch.cuda.synchronize()
        for got, want in ((qx.row.codes, rx.row.codes), (qx.row.scales, rx.row.scales),
                          (qx.col.codes, rx.col.codes), (qx.col.scales, rx.col.scales),
                          (qw.row.codes, rw.row.codes), (qw.row.scales, rw.row.scales)):
            assert torch.equal(got, want), rep
        assert torch.equal(c.view(torch.int32), rc.view(torch.int32)), rep


@pytest.mark.parametrize("k_tiled", [False, True])
def test_mx_empty_shapes(k_tiled):
    """Zero vectors or zero length: the producer writes nothing and returns; the GEMM with an
    empty M or N returns an empty C, and with K = 0 a C of zeros."""
    print(f"case: MXFP4 empty shapes, k_tiled={k_tiled}", flush=True)
    q = nv.mxfp4_quantize(torch.empty((0, 256), dtype=torch.bfloat16, device=DEV),
                          k_tiled=k_tiled).row
    assert q.codes.numel() == 0 and q.scales.numel() == 0
    q = nv.mxfp4_quantize(torch.empty((256, 0), dtype=torch.bfloat16, device=DEV),
                          layouts=("col",), k_tiled=k_tiled).col
    assert q.codes.numel() == 0 and q.scales.numel() == 0
    x = workloads.normal((64, 256), seed=5).to(DEV)
    w = workloads.normal((96, 256), seed=6).to(DEV)
    a = nv.mxfp4_quantize(x, k_tiled=k_tiled).row
    b = nv.mxfp4_quantize(w, k_tiled=k_tiled).row
    empty_a = nv.empty_mx_layout(0, 256, DEV, k_tiled)
    c = nv.mxfp4_gemm(empty_a, b)
    assert c.shape == (0, 96)
    c = nv.mxfp4_gemm(a, nv.empty_mx_layout(0, 256, DEV, k_tiled))
    assert c.shape == (64, 0)
    za, zb = nv.empty_mx_layout(64, 0, DEV, k_tiled), nv.empty_mx_layout(96, 0, DEV, k_tiled)
    c = nv.mxfp4_gemm(za, zb, out=torch.full((64, 96), 7.0, device=DEV))
    torch.cuda.synchronize()
    assert c.shape == (64, 96) and bool((c == 0).all())
