"""The oracle's pins reject plausible mistakes.  Each case plants one mistake in a copy of
oracle/nvfp4_oracle.c (on the CPU; nothing here touches a GPU), builds it, and runs the pins
that should notice it against that build in a child process: they must fail.  A control
case builds the unmodified source the same way and runs every pin named below: they must
pass, so a failure of a mutated build comes from the planted mistake, not from the harness.
"""
import concurrent.futures
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "nvfp4_oracle.c")
PRIM = "tests/test_oracle_primitives.py::"
QUANT = "tests/test_oracle_quantizers.py::"
STRIP = "tests/test_oracle_strips.py::"
MX = "tests/test_oracle_mx.py::"
MARG = "tests/test_oracle_margins.py::"

# (name, text in the source, replacement, pins that must notice)
MUTATIONS = [
    ("butterfly difference reversed", "a[i + h] = u - v;", "a[i + h] = v - u;",
     [PRIM + "test_fwht_columns_are_sylvester"]),
    ("E4M3 ties away from zero", "double n = nearbyint(ldexp((double)t, -q));",
     "double n = round(ldexp((double)t, -q));",
     [PRIM + "test_e4m3_rne_against_torch_and_brute_force"]),
    ("E4M3 round-up rounds to nearest", "double n = ceil(ldexp((double)t, -q));",
     "double n = nearbyint(ldexp((double)t, -q));", [PRIM + "test_e4m3_up_brute_force"]),
    ("E2M1 tie at 0.25 goes up", "if (a <= 0.25f) return 0;", "if (a < 0.25f) return 0;",
     [PRIM + "test_e2m1_rtn_brute_force"]),
    ("scale SR draws one bit short", "uint32_t up_bits = (bits_of(c) + (w >> 12)) & 0xFFF00000u;",
     "uint32_t up_bits = (bits_of(c) + (w >> 13)) & 0xFFF00000u;",
     [PRIM + "test_scale_sr_enumeration"]),
    ("element SR compares with >", "return frac >= (float)(4194304u - v) / 4194304.0f ? lo + 1 : lo;",
     "return frac > (float)(4194304u - v) / 4194304.0f ? lo + 1 : lo;",
     [PRIM + "test_elem_sr_enumeration"]),
    ("Philox multiplier off by two", "0xD2511F53u", "0xD2511F55u",
     [PRIM + "test_philox_known_answers"]),
    ("rotation signs ignored", "a[j] = sigma[j] * v[g0 + j];", "a[j] = v[g0 + j];",
     [QUANT + "test_eden_ratio_is_one_on_grid"]),
    ("zero keeps its sign bit", "int neg = r[i] < 0.0f;", "int neg = signbit(r[i]) != 0;",
     [QUANT + "test_zero_encoding"]),
    ("skip threshold one binade low", "} else if (c < 0.015625f) {",
     "} else if (c < 0.0078125f) {", [QUANT + "test_skip_of_tiny_scales"]),
    ("EDEN ratio inverted", "float S = (den > 0.0f) ? num / den : 1.0f;\n            for (int b",
     "float S = (den > 0.0f) ? den / num : 1.0f;\n            for (int b",
     [QUANT + "test_unbiasedness_fig9_method"]),      # MSE ordering alone misses it
    ("MS-EDEN tensor scale divides by 4 * 448",
     "float d = (mode == MODE_FP46) ? 1792.0f : 2688.0f;",
     "float d = (mode == MODE_FP46) ? 1792.0f : 1792.0f;",
     [QUANT + "test_tensor_max_block_gets_top_scale"]),
    ("SR block scale rounded to nearest", "uint8_t s = oracle_e4m3_up(t);",
     "uint8_t s = oracle_e4m3_rne_sat(t);", [QUANT + "test_sr_scale_never_clips"]),
    ("4/6 keeps the worse option", "int pickA = errA <= errB;", "int pickA = errA >= errB;",
     [QUANT + "test_fp46_choice_against_fp64"]),
    ("strip scale from the whole layout", "v0, v1));", "0, total));",
     [STRIP + "test_power_of_two_equivariance_per_strip"]),
    ("MS-EDEN block scale rounded up", "                s[b] = oracle_e4m3_rne_sat(t);",
     "                s[b] = oracle_e4m3_up(t);", [QUANT + "test_rtn_codes_are_nearest"]),
    ("EDEN <r,q> uses r for q", "Q[i] = r[i] * q[i];", "Q[i] = r[i] * r[i];",
     [QUANT + "test_eden_ratio_against_fp64"]),
    ("EDEN <r,r> misses the square", "P[i] = r[i] * r[i];", "P[i] = r[i];",
     [QUANT + "test_eden_ratio_is_one_on_grid"]),
    ("pairwise sum drops the last term", "t[i] = t[2 * i] + t[2 * i + 1];",
     "t[i] = t[2 * i] + (2 * i + 1 < n - 1 ? t[2 * i + 1] : 0.0f);",
     [QUANT + "test_eden_ratio_against_fp64"]),
    ("4/6 error adds instead of subtracting", "float d = q[i] - r[i];",
     "float d = q[i] + r[i];", [QUANT + "test_fp46_choice_against_fp64"]),
    ("4/6 error is absolute, not squared", "d2[i] = d * d;", "d2[i] = fabsf(d);",
     [QUANT + "test_fp46_choice_against_fp64"]),
    ("E2M1 margin misses the top threshold", "for (int i = 0; i < 7; ++i) {\n        uint32_t d",
     "for (int i = 0; i < 6; ++i) {\n        uint32_t d", [MARG + "test_e2m1_margin"]),
    ("E4M3 round-up margin counts the saturated top", "if (c < 0x7E) best = ulp_dist(t, oracle_e4m3_value(c));",
     "best = ulp_dist(t, oracle_e4m3_value(c));", [MARG + "test_e4m3_up_margin"]),
    ("E4M3 nearest margin skips the midpoint above", "if (c < 0x7E) {\n        float mid",
     "if (c < 0x7D) {\n        float mid", [MARG + "test_e4m3_rne_margin"]),
    ("scale SR margin one bit short", "uint32_t sum = (bits_of(c) & 0xFFFFFu) + (w >> 12);",
     "uint32_t sum = (bits_of(c) & 0xFFFFFu) + (w >> 13);", [MARG + "test_scale_sr_margin"]),
    ("element SR margin from the wrong grid point",
     "double ab = E2M1_V[lo] + (1.0 - (double)(w >> 10) / 4194304.0) * (E2M1_V[lo + 1] - E2M1_V[lo]);",
     "double ab = E2M1_V[lo + 1] - (1.0 - (double)(w >> 10) / 4194304.0) * (E2M1_V[lo + 1] - E2M1_V[lo]);",
     [MARG + "test_elem_sr_margin"]),
    ("decoder drops the sign", "o[e] = (code & 8) ? -qv : qv;", "o[e] = qv;",
     [QUANT + "test_dequantize_round_trips_on_grid_inputs"]),
    ("decoder swaps the nibbles", "uint8_t code = (e % 2 == 0) ? (byte & 15) : (byte >> 4);",
     "uint8_t code = (e % 2 == 0) ? (byte >> 4) : (byte & 15);",
     [QUANT + "test_dequantize_round_trips_on_grid_inputs"]),
    ("MX scale one binade high on exact fits", "while (ldexp(6.0, e) < (double)m) ++e;",
     "while (ldexp(6.0, e) <= (double)m) ++e;", [MX + "test_scale_exponent_brute_force"]),
    ("MX elements scaled by the wrong power", "float p = ldexpf(1.0f, -e);",
     "float p = ldexpf(1.0f, 1 - e);", [MX + "test_rtn_codes_are_nearest_and_never_clip"]),
    ("MX decoder ignores the scale bias", "float s = ldexpf(1.0f, (int)scales[v * (n / 32) + pos / 32] - 127);",
     "float s = ldexpf(1.0f, (int)scales[v * (n / 32) + pos / 32] - 126);",
     [MX + "test_round_trip_on_grid_inputs"]),
    ("MX SR draws from the scale stream", "uint32_t w = rand_word(seed, (uint64_t)(vec * n + pos), STREAM_ELEM_SR,",
     "uint32_t w = rand_word(seed, (uint64_t)(vec * n + pos) / 4, STREAM_ELEM_SR,",
     [MX + "test_sr_draws_are_independent_per_element"]),
    ("4/6 tensor scale divides by 6 * 448",
     "float d = (mode == MODE_FP46) ? 1792.0f : 2688.0f;",
     "float d = (mode == MODE_FP46) ? 2688.0f : 2688.0f;",
     [QUANT + "test_tensor_max_block_gets_top_scale"]),
]


def _build(src_text, out_dir):
    c_path = os.path.join(out_dir, "oracle.c")
    so_path = os.path.join(out_dir, "liboracle.so")
    with open(c_path, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                    "-fPIC", "-shared", "-o", so_path, c_path, "-lm"], check=True,
                   capture_output=True)
    return so_path


def _run_pins(so_path, pins):
    env = dict(os.environ, NVFP4_ORACLE_LIB=so_path, OMP_NUM_THREADS="2")
    p = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *pins], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return p.returncode, p.stdout[-2000:]


def _case(name, old, new, pins, source):
    with tempfile.TemporaryDirectory() as d:
        if old is not None:
            assert source.count(old) == 1, f"{name}: the text to replace must occur once"
            source = source.replace(old, new)
        so = _build(source, d)
        return _run_pins(so, pins)


def test_pins_reject_planted_mistakes():
    source = open(SRC).read()
    all_pins = sorted({p for _, _, _, pins in MUTATIONS for p in pins})
    jobs = [("control", None, None, all_pins)] + MUTATIONS
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        futs = {name: ex.submit(_case, name, old, new, pins, source)
                for name, old, new, pins in jobs}
        results = {name: f.result() for name, f in futs.items()}
    rc, out = results.pop("control")
    assert rc == 0, f"the unmodified oracle must pass its pins:\n{out}"
    escaped = {name: out for name, (rc, out) in results.items() if rc != 1}
    assert not escaped, f"mistakes the pins did not reject (or that broke the run): {escaped}"


@pytest.mark.parametrize("name,old,new,pins", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_text_occurs_once(name, old, new, pins):
    assert open(SRC).read().count(old) == 1
