"""GEMM check consumer: C = A B^T of two NVFP4 operands on the matrix cores, against an fp64
reference built directly from the codes and scales (exact operand values), within the
bound of FP32 accumulation, |dC| <= 2 K u sum_k |a_k b_k| (u = 2^-24)."""
import numpy as np
import pytest
import torch

import unbiased_nvfp4_gradient_amd as nv
import workloads
from gemm_ref import check_entries

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("M,N,K", [(256, 256, 128), (512, 256, 384), (96, 160, 64),
                                   (256, 512, 1024)])
def test_gemm_small_exhaustive(M, N, K):
    print(f"case: gemm M={M} N={N} K={K}", flush=True)
    x = workloads.normal((M, K), seed=M + K).to(DEV)
    w = workloads.normal((N, K), seed=N + K + 1, scale=0.02).to(DEV)
    rot = K % 128 == 0
    if rot:
        a = nv.eden_quantize(x, seed=3, rht_seed=9, layouts=("row",)).row
        b = nv.rtn_quantize(w, rht=True, rht_seed=9, layouts=("row",)).row
    else:
        a = nv.rtn_quantize(x, layouts=("row",)).row
        b = nv.rtn_quantize(w, layouts=("row",)).row
    c = nv.nvfp4_gemm_check(a, b, rotated_pair=rot)
    torch.cuda.synchronize()
    f = 2.0 ** -7 if rot else 1.0
    got, ref = check_entries(c, a, b, np.arange(M), np.arange(N), f)
    # the rotation cancels: C approximates the unquantized product
    xw = (x.float() @ w.float().T).cpu().numpy()
    rel = np.linalg.norm(got - xw) / np.linalg.norm(xw)
    assert rel < 0.2, rel


def test_gemm_zero_k_and_errors():
    print("case: gemm K=0 and bad shapes", flush=True)
    a = nv.NVFP4(torch.zeros((64, 0), dtype=torch.uint8, device=DEV),
                 torch.zeros((64, 0), dtype=torch.uint8, device=DEV),
                 torch.ones(1, device=DEV))
    c = nv.nvfp4_gemm_check(a, a)
    torch.cuda.synchronize()
    assert c.shape == (64, 64) and not c.any()
    x = workloads.normal((48, 128), seed=1).to(DEV)
    q = nv.rtn_quantize(x, layouts=("row",)).row
    with pytest.raises(nv.NVFP4Error):
        nv.nvfp4_gemm_check(q, q)          # M = 48 is not a multiple of 32


def test_gemm_config4_sampled():
    """16384 x 8192 MS-EDEN activations against an 8192 x 8192 RTN weight, both rotated with
    the same seed along K = 8192 (the bench's check configuration); sampled entries."""
    print("case: gemm c4 M=16384 N=8192 K=8192 sampled", flush=True)
    x = workloads.c4().to(DEV)
    w = workloads.c4w().to(DEV)
    a = nv.eden_quantize(x, seed=1, rht_seed=1, layouts=("row",)).row
    b = nv.rtn_quantize(w, rht=True, rht_seed=1, layouts=("row",)).row
    del x, w
    c = nv.nvfp4_gemm_check(a, b, rotated_pair=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([[0, 16383], rng.choice(16384, 62, replace=False)]))
    cols = np.unique(np.concatenate([[0, 8191], rng.choice(8192, 62, replace=False)]))
    check_entries(c, a, b, rows, cols, 2.0 ** -7)
    assert torch.isfinite(c).all()
