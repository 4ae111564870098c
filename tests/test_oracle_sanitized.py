"""Host-side sanitizer run of the fp64 oracle (CPU only).

Compiles oracle/kron_delta_oracle.c together with tests/native/oracle_sanitize.c
under gcc's AddressSanitizer and UndefinedBehaviorSanitizer and runs the oracle's
entry points (forward, backward, Gated Delta Rule-2 forward) on small seeded
inputs with the parity tests' edge cases: an empty sequence, one token, a
ragged tail, gates at exactly 0 and 1, with and without S0 and dS_T.  Any
out-of-bounds access, leak or undefined operation aborts the program.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = tmp_path / "oracle_sanitize"
    cmd = [gcc, "-O1", "-g", "-std=c99", "-fopenmp", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           os.path.join(ROOT, "tests", "native", "oracle_sanitize.c"),
           os.path.join(ROOT, "oracle", "kron_delta_oracle.c"), "-o", str(exe), "-lm"]
    built = subprocess.run(cmd, capture_output=True, text=True)
    if built.returncode != 0 and "sanitize" in built.stderr and "cannot find" in built.stderr:
        pytest.skip("sanitizer runtime not installed")
    assert built.returncode == 0, built.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="2")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stderr[-4000:]
