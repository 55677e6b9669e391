"""GPU parity: the HIP library (through its C ABI) against the CPU oracle, element by element,
on the same seeded inputs.  Codes and scales bit-exact outside the 2-ulp boundary band
(tests/parity.py), tensor scales exact, dequantized values within 1e-6 relative."""
import numpy as np
import pytest
import torch

import oracle
import unbiased_nvfp4_gradient_amd as nv
import workloads
from guards import guarded_outputs
from parity import assert_parity, assert_same_floats

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def run_gpu(mode, x, layouts, seed=1, rht=False, rht_seed=1, guard=False):
    """Quantize on the GPU; with guard, into outputs fenced by sentinel margins that must
    come back untouched."""
    xd = x.to(DEV)
    out, guards = (guarded_outputs(xd.shape[0], xd.shape[1], layouts, DEV) if guard
                   else (None, []))
    if mode == "eden":
        q = nv.eden_quantize(xd, seed, rht_seed, layouts=layouts, out=out)
    elif mode == "sr":
        q = nv.sr_quantize(xd, seed, rht=rht, rht_seed=rht_seed, layouts=layouts, out=out)
    elif mode == "rtn":
        q = nv.rtn_quantize(xd, rht=rht, rht_seed=rht_seed, layouts=layouts, out=out)
    else:
        q = nv.fp46_quantize(xd, rht=rht, rht_seed=rht_seed, layouts=layouts, out=out)
    torch.cuda.synchronize()
    assert all(g.intact() for g in guards), "a write landed outside an output buffer"
    out = {}
    for axis, t in ((0, q.row), (1, q.col)):
        if t is not None:
            out[axis] = (t.codes.cpu().numpy(), t.scales.cpu().numpy(),
                         float(t.tensor_scale.cpu()[0]), t)
    return out


def check_full(mode, x, layouts, seed=1, rht=False, rht_seed=1, what="", guard=True):
    got = run_gpu(mode, x, layouts, seed, rht, rht_seed, guard=guard)
    xb = workloads.bf16_bits(x)
    reps = []
    for axis, (codes, scales, g, _) in got.items():
        ref = oracle.quantize(mode, xb, axis=axis, seed=seed, rht=rht, rht_seed=rht_seed)
        reps.append(assert_parity(mode, codes, scales, g, ref, f"{what} axis={axis}"))
    return got, reps


# ----------------------------------------------------------------------------- small / config 1

@pytest.mark.parametrize("mode,rht", [("rtn", False), ("sr", False), ("eden", True),
                                      ("fp46", False), ("rtn", True), ("sr", True),
                                      ("fp46", True)])
@pytest.mark.parametrize("layouts", [("row",), ("col",), ("row", "col")])
def test_config1_all_modes(mode, rht, layouts):
    print(f"case: c1 256x1024 mode={mode} rht={rht} layouts={layouts}", flush=True)
    check_full(mode, workloads.c1(), layouts, seed=1, rht=rht, rht_seed=1,
               what=f"c1 {mode} rht={rht}")


@pytest.mark.parametrize("shape,mode,rht,layouts", [
    ((200, 256), "eden", True, ("row",)),          # ragged row count (partial tile)
    ((256, 200), "eden", True, ("col",)),          # ragged column count
    ((130, 144), "rtn", False, ("row",)),          # n % 128 != 0 without rotation
    ((48, 40), "sr", False, ("col",)),             # tiny, n = 48
    ((144, 48), "fp46", False, ("row", "col")),    # both layouts, ragged, no rotation
    ((384, 640), "eden", True, ("row", "col")),    # several tiles both ways
    ((128, 128), "sr", True, ("row", "col")),      # exactly one tile
])
def test_ragged_and_multi_tile(shape, mode, rht, layouts):
    print(f"case: shape={shape} mode={mode} rht={rht} layouts={layouts}", flush=True)
    x = workloads.normal(shape, seed=sum(shape))
    check_full(mode, x, layouts, seed=7, rht=rht, rht_seed=3, what=f"{shape} {mode}")


def test_zero_and_empty():
    print("case: zeros 256x256 and empty 0x256 / 256x0", flush=True)
    z = torch.zeros(256, 256, dtype=torch.bfloat16)
    got, _ = check_full("eden", z, ("row", "col"), what="zeros")
    for codes, scales, g, _ in got.values():
        assert g == 0.0 and not codes.any() and not scales.any()
    for shape, lay in (((0, 256), ("row",)), ((256, 0), ("col",))):
        x = torch.zeros(shape, dtype=torch.bfloat16, device=DEV)
        q = nv.eden_quantize(x, 1, 1, layouts=lay)
        torch.cuda.synchronize()
        t = q.row if q.row is not None else q.col
        assert t.codes.numel() == 0 and float(t.tensor_scale.cpu()[0]) == 0.0


def _zero_heavy(seed=5):
    """512 x 512 rows built to produce exact zeros and cancellations inside the rotation:
    small integers, constant rows, sparse rows filled with +-0, groups whose first half is
    zero, equal and opposite pairs, all -0 rows, and +-c patterns; N(0,1) rows in between."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((512, 512))
    x[0:64] = rng.integers(-2, 3, (64, 512))
    x[64:128] = rng.choice([-1.0, -0.5, 0.5, 1.0, 2.0], (64, 1))
    sparse = rng.random((64, 512)) < 0.05
    x[128:192] = np.where(sparse, rng.standard_normal((64, 512)),
                          rng.choice([0.0, -0.0], (64, 512)))
    x[192:256].reshape(64, 4, 128)[:, :, :64] = rng.choice([0.0, -0.0], (64, 4, 64))
    pairs = rng.standard_normal((64, 256))
    x[256:320, 0::2] = pairs
    x[256:320, 1::2] = pairs * rng.choice([-1.0, 1.0], (64, 256))
    x[384:448] = -0.0
    x[448:512] = rng.choice([-1.5, 1.5], (64, 512)) * rng.integers(1, 3, (64, 1))
    return workloads.to_bf16(x)


@pytest.mark.parametrize("mode,rht", [("eden", True), ("rtn", True), ("rtn", False),
                                      ("sr", True), ("sr", False), ("fp46", True),
                                      ("fp46", False)])
def test_exact_zeros_and_cancellations(mode, rht):
    print(f"case: zero-heavy 512x512 mode={mode} rht={rht}", flush=True)
    x = _zero_heavy()
    assert (workloads.bf16_bits(x) == 0x8000).any()
    check_full(mode, x, ("row", "col"), seed=4, rht=rht, rht_seed=6,
               what=f"zero-heavy {mode} rht={rht}")


def test_extreme_magnitudes():
    """Tiny values (subnormal products, scales below 2^-6 and zero scales) and large ones."""
    rng = np.random.default_rng(0)
    base = rng.standard_normal((256, 256))
    mags = 10.0 ** rng.uniform(-30, 30, (256, 1))
    x = workloads.to_bf16(base * mags)
    print("case: magnitudes 1e-30..1e30 per row", flush=True)
    for mode, rht in (("eden", True), ("rtn", False), ("sr", False), ("fp46", True)):
        check_full(mode, x, ("row", "col"), rht=rht, what=f"extreme {mode}")


def test_determinism():
    print("case: determinism eden c1 both layouts", flush=True)
    x = workloads.c1()
    a = run_gpu("eden", x, ("row", "col"))
    b = run_gpu("eden", x, ("row", "col"))
    for axis in a:
        assert np.array_equal(a[axis][0], b[axis][0]) and np.array_equal(a[axis][1], b[axis][1])


# ----------------------------------------------------------------------------- configs 2 and 3

def test_config2_fp46_both_layouts():
    print("case: c2 4096x4096 fp46 rht both layouts", flush=True)
    check_full("fp46", workloads.c2(), ("row", "col"), rht=True, rht_seed=1, what="c2")


def test_config3_eden_both_layouts():
    print("case: c3 16384x2048 eden both layouts", flush=True)
    check_full("eden", workloads.c3(), ("row", "col"), seed=1, rht_seed=1, what="c3")


# ----------------------------------------------------------------------------- config 4 (full)

def assert_identical(codes, scales, g, ref, what):
    """Every code byte, scale byte and the tensor scale equal to the oracle's."""
    assert np.float32(g) == np.float32(ref.g), f"{what}: tensor scale {g!r} != {ref.g!r}"
    assert codes.shape == ref.codes.shape and scales.shape == ref.scales.shape, what
    cm = int(np.count_nonzero(codes != ref.codes))
    sm = int(np.count_nonzero(scales != ref.scales))
    assert cm == 0 and sm == 0, f"{what}: {cm} code bytes and {sm} scale bytes differ"


@pytest.fixture(scope="module")
def config4():
    x = workloads.c4()
    return x, workloads.bf16_bits(x), x.to(DEV)


@pytest.mark.parametrize("mode,rht,seed,rht_seed", [
    ("eden", True, 1, 1),            # the benchmark's call
    ("sr", True, 3, 2), ("sr", False, 3, 2), ("rtn", True, 0, 2), ("rtn", False, 0, 2),
    ("fp46", True, 0, 2)])
def test_config4_full(config4, mode, rht, seed, rht_seed):
    """The full 16384 x 8192 input in the benchmark's launch configuration (both layouts in
    one call): every code, scale and tensor scale of both layouts against the oracle."""
    print(f"case: c4 16384x8192 {mode} rht={rht} both layouts, every output", flush=True)
    x, xb, xd = config4
    got = run_gpu(mode, xd, ("row", "col"), seed=seed, rht=rht, rht_seed=rht_seed)
    for axis in (0, 1):
        codes, scales, g, _ = got[axis]
        ref = oracle.quantize(mode, xb, axis=axis, seed=seed, rht=rht, rht_seed=rht_seed,
                              margins=False)
        assert_identical(codes, scales, g, ref, f"c4 {mode} rht={rht} axis={axis}")


# ----------------------------------------------------------------------------- dequantize

@pytest.mark.parametrize("mode,rht", [("eden", True), ("rtn", False), ("fp46", True)])
def test_dequantize_parity(mode, rht):
    print(f"case: dequantize {mode} rht={rht}", flush=True)
    x = workloads.c1()
    got = run_gpu(mode, x, ("row", "col"), rht=rht)
    rot = rht or mode == "eden"
    for axis, (codes, scales, g, t) in got.items():
        out = nv.dequantize(t, rht=rot, rht_seed=1)
        torch.cuda.synchronize()
        ref = oracle.dequantize(codes, scales, g, rht=rot, rht_seed=1)
        o = out.cpu().numpy()
        # the codes matched the oracle (checked above), so the decode must match too
        scale = np.maximum(np.abs(ref), np.sqrt((ref.reshape(ref.shape[0], -1, 16) ** 2)
                                                 .mean(-1)).repeat(16, -1))
        assert np.all(np.abs(o - ref) <= 1e-6 * scale), (mode, axis)
        # same operations in the same order: bit-exact (a zero's sign aside when rotated)
        assert_same_floats(o, ref, f"{mode} axis={axis}", zero_sign_free=rot)


@pytest.mark.parametrize("shape,mode", [((144, 48), "rtn"), ((112, 1040), "sr"),
                                        ((48, 208), "rtn"), ((144, 2064), "fp46")])
def test_dequantize_ragged_unrotated(shape, mode):
    """Vector lengths that end in a partial group (48, 112, 144 = 128 + 16, 208 = 128 + 80,
    1040 = 8 x 128 + 16, 2064 = 16 x 128 + 16; rows are the column layout's lengths): the
    unrotated decoder's lanes hold positions 4q..4q+3 and 64+4q..64+4q+3 of a group, so in a
    short last group some lanes store one quadruple and some none; both layouts, compared
    with the oracle bit for bit."""
    print(f"case: dequantize ragged {shape} {mode} without the rotation", flush=True)
    x = workloads.normal(shape, seed=11)
    got = run_gpu(mode, x, ("row", "col"), seed=5, rht=False, guard=True)
    for axis, (codes, scales, g, t) in got.items():
        vecs, n = codes.shape[0], codes.shape[1] * 2
        # the output is a view into a larger buffer whose margins must stay untouched
        fence = torch.full((1024 + vecs * n + 1024,), -7.0, dtype=torch.float32, device=DEV)
        out = fence[1024:1024 + vecs * n].view(vecs, n)
        nv.dequantize(t, rht=False, out=out)
        torch.cuda.synchronize()
        assert bool((fence[:1024] == -7.0).all()) and bool((fence[1024 + vecs * n:] == -7.0).all())
        ref = oracle.dequantize(codes, scales, g, rht=False, rht_seed=0)
        assert_same_floats(out.cpu().numpy(), ref, f"{shape} {mode} axis={axis}")


# ----------------------------------------------------------------------------- outside the contract

def test_nonfinite_inputs_complete():
    """NaN, infinities and values beyond 2^56 are outside the contract (their codes are
    unspecified), but every quantizer must still complete and write in-range scale bytes."""
    print("case: NaN / inf / huge inputs, every mode, both layouts", flush=True)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((256, 512)).astype(np.float32)
    x[rng.random(x.shape) < 0.01] = np.nan
    x[rng.random(x.shape) < 0.01] = np.inf
    x[rng.random(x.shape) < 0.01] = -np.inf
    x[rng.random(x.shape) < 0.01] = 3e38
    xd = torch.from_numpy(x).to(torch.bfloat16).to(DEV)
    bits = workloads.bf16_bits(xd.cpu())
    assert ((bits & 0x7FFF) > 0x7F80).any() and ((bits & 0x7FFF) == 0x7F80).any()
    for mode, rht in (("eden", True), ("sr", False), ("sr", True), ("rtn", False),
                      ("rtn", True), ("fp46", False), ("fp46", True)):
        got = run_gpu(mode, xd, ("row", "col"), seed=2, rht=rht, rht_seed=2)
        for axis, (codes, scales, g, _) in got.items():
            assert scales.max() <= 0x7E, (mode, rht, axis)


# ----------------------------------------------------------------------------- HIP graphs

@pytest.mark.parametrize("layouts", [("row", "col"), ("row",), ("col",)])
def test_workspace_contents_do_not_matter(layouts):
    """Phase 1 leaves one maximum per workgroup and layout in the workspace and phase 2
    reduces them: a workspace full of 0xFF bytes (larger than any maximum, compared as
    unsigned integers) must give the same result as a zeroed one, in every mode."""
    print(f"case: workspace filled with 0xFF, layouts {layouts}", flush=True)
    x = workloads.c4(seed=12, shape=(640, 768)).to(DEV)
    for name, fn, kw in (("eden", nv.eden_quantize, dict(seed=3, rht_seed=4)),
                         ("sr", nv.sr_quantize, dict(seed=3, rht=True, rht_seed=4)),
                         ("rtn", nv.rtn_quantize, dict(rht=False)),
                         ("fp46", nv.fp46_quantize, dict(rht=True, rht_seed=4))):
        outs = []
        for fill in (0, 255):
            ws = torch.full((nv.workspace_bytes(640, 768, 3),), fill, dtype=torch.uint8,
                            device=DEV)
            outs.append(fn(x, layouts=layouts, workspace=ws, **kw))
        torch.cuda.synchronize()
        for lay in layouts:
            a, b = getattr(outs[0], lay), getattr(outs[1], lay)
            for f in ("codes", "scales", "tensor_scale"):
                assert torch.equal(getattr(a, f), getattr(b, f)), (name, lay, f)


def test_graph_capture_and_replay():
    """The entry points allocate nothing and write every workspace slot they read (no
    memset), so a call can be captured in a HIP graph.  Each replay (with other quantizer work run eagerly in
    between) must give the eager result bit for bit."""
    print("case: HIP graph capture of eden_quantize + dequantize, 4 replays", flush=True)
    x = workloads.normal((384, 512), seed=77).to(DEV)
    other = workloads.normal((256, 256), seed=78).to(DEV)
    ws = torch.empty(nv.workspace_bytes(384, 512, 3), dtype=torch.uint8, device=DEV)
    out = nv.Quantized(nv.empty_layout(384, 512, DEV), nv.empty_layout(512, 384, DEV))
    back = torch.empty((384, 512), dtype=torch.float32, device=DEV)
    ref = nv.eden_quantize(x, 5, 6, layouts=("row", "col"))
    ref_back = nv.dequantize(ref.row, rht=True, rht_seed=6)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream(device=DEV)
    s.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(s):
        nv.eden_quantize(x, 5, 6, layouts=("row", "col"), out=out, workspace=ws)   # warm-up
        nv.dequantize(out.row, rht=True, rht_seed=6, out=back)
    torch.cuda.current_stream(DEV).wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        nv.eden_quantize(x, 5, 6, layouts=("row", "col"), out=out, workspace=ws)
        nv.dequantize(out.row, rht=True, rht_seed=6, out=back)
    for rep in range(4):
        for t in (out.row.codes, out.row.scales, out.col.codes, out.col.scales, back):
            t.zero_()
        nv.sr_quantize(other, seed=rep, layouts=("row", "col"))        # eager work between
        g.replay()
        torch.cuda.synchronize()
        for got, want in ((out.row.codes, ref.row.codes), (out.row.scales, ref.row.scales),
                          (out.col.codes, ref.col.codes), (out.col.scales, ref.col.scales),
                          (out.row.tensor_scale, ref.row.tensor_scale),
                          (out.col.tensor_scale, ref.col.tensor_scale), (back, ref_back)):
            assert torch.equal(got, want), rep


def test_concurrent_streams():
    """Calls on two streams at once, each with its own workspace and outputs, give the same
    results as one after the other: the library keeps no state between calls.  Calls run on
    the side streams while the default stream goes on; the inputs were made before them."""
    print("case: eden_quantize and nvfp4_quantize_strips on two streams at once", flush=True)
    xa = workloads.c4(seed=3, shape=(1024, 2048)).to(DEV)
    xb = workloads.normal((2048, 1024), seed=4).to(DEV)
    ref_a = nv.eden_quantize(xa, 1, 2, layouts=("row", "col"))
    ref_b = nv.nvfp4_quantize_strips("eden", xb, seed=3, rht_seed=4, layouts=("row", "col"))
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(device=DEV), torch.cuda.Stream(device=DEV)
    outs = []
    for rep in range(3):
        with torch.cuda.stream(sa):
            qa = nv.eden_quantize(xa, 1, 2, layouts=("row", "col"))
        # the stream argument alone: outputs and workspace are allocated on sb too
        qb = nv.nvfp4_quantize_strips("eden", xb, seed=3, rht_seed=4, layouts=("row", "col"),
                                      stream=sb)
        outs.append((qa, qb))
    torch.cuda.synchronize()
    for qa, qb in outs:
        for got, want in ((qa, ref_a), (qb, ref_b)):
            for lay in ("row", "col"):
                g, w = getattr(got, lay), getattr(want, lay)
                assert torch.equal(g.codes, w.codes) and torch.equal(g.scales, w.scales)
                assert torch.equal(g.tensor_scale, w.tensor_scale)
