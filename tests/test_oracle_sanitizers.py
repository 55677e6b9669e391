"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

tests/helpers/oracle_sanitize_driver.c calls every entry point of oracle/nvfp4_oracle.c over
the inputs its pins use (every mode, layout and rotation setting, ragged and empty shapes,
vector sub-sets, strip-local scales, the decoder, the EDEN internals, the scalar roundings
at their edges); built with -fsanitize=address,undefined and no recovery, any out-of-bounds
access, leak or undefined operation ends the run with a report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_is_clean_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.fail("gcc is needed to build the sanitized oracle")
    exe = str(tmp_path / "oracle_sanitized")
    subprocess.run([gcc, "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
                    "-ffp-contract=off", "-fno-fast-math",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-o", exe, os.path.join(ROOT, "oracle", "nvfp4_oracle.c"),
                    os.path.join(ROOT, "tests", "helpers", "oracle_sanitize_driver.c"), "-lm"],
                   check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    p = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    report = (p.stdout + p.stderr)[-4000:]
    assert p.returncode == 0, report
    assert "runtime error" not in p.stderr and "AddressSanitizer" not in p.stderr, report
    assert "all calls behaved" in p.stdout
