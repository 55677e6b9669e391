"""One training step's worth of linear-layer quantizations of a 1.9B-parameter Llama-style
model (hidden 2048, FFN 8192, 24 layers, 32768 tokens), batched on one stream: for each of
q/k/v/o/gate/up/down, 4/6 of the weight (both layouts) and of the activation (row layout)
for the forward GEMM, and MS-EDEN of the grad-output (both layouts) for the two backward
GEMMs -- 504 calls.  GEMM partners share a rotation seed along their contraction dim:
X row / W row (forward), dY row / W column (input gradient).

Inputs are drawn on the GPU (torch generator, seed 0): X ~ N(0,1), W ~ N(0, 0.02),
dY ~ N(0,1), one buffer per distinct shape reused by every layer.  Layer 0's outputs are
checked against the oracle in full (every code, scale and tensor scale of the weights, the
activations and the grad-outputs); the whole batch is timed."""
import numpy as np
import pytest
import torch

import oracle
import unbiased_nvfp4_gradient_amd as nv
import workloads
from parity import assert_parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOKENS, HIDDEN, FFN, LAYERS = 32768, 2048, 8192, 24
PROJ = [("q", HIDDEN, HIDDEN), ("k", HIDDEN, HIDDEN), ("v", HIDDEN, HIDDEN),
        ("o", HIDDEN, HIDDEN), ("gate", FFN, HIDDEN), ("up", FFN, HIDDEN), ("down", HIDDEN, FFN)]


def make_inputs():
    g = torch.Generator(device=DEV).manual_seed(0)

    def randn(shape, std):
        return (torch.randn(shape, generator=g, device=DEV) * std).to(torch.bfloat16)

    acts = {d: randn((TOKENS, d), 1.0) for d in (HIDDEN, FFN)}
    grads = {d: randn((TOKENS, d), 1.0) for d in (HIDDEN, FFN)}
    weights = {(o, i): randn((o, i), 0.02) for o, i in ((HIDDEN, HIDDEN), (FFN, HIDDEN),
                                                       (HIDDEN, FFN))}
    return acts, grads, weights


def outputs_for(acts, grads, weights):
    """Preallocated outputs, one set per distinct shape and role."""
    out = {}
    for (o, i), w in weights.items():
        out[("w", o, i)] = nv.Quantized(nv.empty_layout(o, i, DEV), nv.empty_layout(i, o, DEV))
    for d in (HIDDEN, FFN):
        out[("x", d)] = nv.Quantized(nv.empty_layout(TOKENS, d, DEV), None)
        out[("dy", d)] = nv.Quantized(nv.empty_layout(TOKENS, d, DEV),
                                      nv.empty_layout(d, TOKENS, DEV))
    return out


def run_projection(layer, p, acts, grads, weights, out, ws, stream):
    name, o, i = PROJ[p]
    rs = 1000 * layer + 10 * p               # rotation seed shared by the GEMM partners
    w, x, dy = weights[(o, i)], acts[i], grads[o]
    qw = nv.fp46_quantize(w, rht=True, rht_seed=rs, layouts=("row", "col"),
                          out=out[("w", o, i)], workspace=ws, stream=stream)
    qx = nv.fp46_quantize(x, rht=True, rht_seed=rs, layouts=("row",), out=out[("x", i)],
                          workspace=ws, stream=stream)
    qd = nv.eden_quantize(dy, seed=rs + 3, rht_seed=rs, layouts=("row", "col"),
                          out=out[("dy", o)], workspace=ws, stream=stream)
    return name, rs, (o, i), qw, qx, qd


def run_layer(layer, acts, grads, weights, out, ws, stream):
    for p in range(len(PROJ)):
        run_projection(layer, p, acts, grads, weights, out, ws, stream)


def _parity_full(mode, x_dev, q: nv.NVFP4, axis, seed, rs, what):
    """Every code, scale and the tensor scale of one layout against the oracle."""
    xb = workloads.bf16_bits(x_dev.cpu())
    ref = oracle.quantize(mode, xb, axis=axis, seed=seed, rht=True, rht_seed=rs, margins=False)
    g = float(q.tensor_scale.cpu()[0])
    assert np.float32(g) == np.float32(ref.g), what
    codes, scales = q.codes.cpu().numpy(), q.scales.cpu().numpy()
    cm = int(np.count_nonzero(codes != ref.codes))
    sm = int(np.count_nonzero(scales != ref.scales))
    assert cm == 0 and sm == 0, f"{what}: {cm} code bytes and {sm} scale bytes differ"


def test_config5_layer0_parity_and_batch_timing():
    print("case: config 5 layer 0 parity (21 quantizations)", flush=True)
    acts, grads, weights = make_inputs()
    out = outputs_for(acts, grads, weights)
    ws = torch.empty(nv.workspace_bytes(TOKENS, FFN, 3), dtype=torch.uint8, device=DEV)
    stream = torch.cuda.current_stream(DEV)
    for p in range(len(PROJ)):
        # projections of one shape share output buffers: check each before the next runs
        name, rs, (o, i), qw, qx, qd = run_projection(0, p, acts, grads, weights, out, ws,
                                                      stream)
        torch.cuda.synchronize()
        w, x, dy = weights[(o, i)], acts[i], grads[o]
        wb = workloads.bf16_bits(w.cpu())
        for axis, t in ((0, qw.row), (1, qw.col)):
            ref = oracle.quantize("fp46", wb, axis=axis, rht=True, rht_seed=rs)
            assert_parity("fp46", t.codes.cpu().numpy(), t.scales.cpu().numpy(),
                          float(t.tensor_scale.cpu()[0]), ref, f"{name} W axis={axis}")
        _parity_full("fp46", x, qx.row, 0, 0, rs, f"{name} X row")
        _parity_full("eden", dy, qd.row, 0, rs + 3, rs, f"{name} dY row")
        _parity_full("eden", dy, qd.col, 1, rs + 3, rs, f"{name} dY col")

    print("case: config 5 full step, 504 calls on one stream", flush=True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for layer in range(2):                                   # warm-up
        run_layer(layer, acts, grads, weights, out, ws, stream)
    torch.cuda.synchronize()
    e0.record(stream)
    for layer in range(LAYERS):
        run_layer(layer, acts, grads, weights, out, ws, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    read = 0
    written = 0
    for name, o, i in PROJ:
        read += 2 * (o * i + TOKENS * i + TOKENS * o)
        written += 2 * (o * i // 2 + o * i // 16) + (TOKENS * i // 2 + TOKENS * i // 16)
        written += 2 * (TOKENS * o // 2 + TOKENS * o // 16)
    read *= LAYERS
    written *= LAYERS
    print(f"config 5: {LAYERS * len(PROJ) * 3} calls in {ms:.2f} ms; algorithmic "
          f"{read / 1e9:.1f} GB read + {written / 1e9:.1f} GB written = "
          f"{(read + written) / (ms * 1e-3) / 1e9:.0f} GB/s", flush=True)
    assert ms > 0
