"""The oracle and the synthetic generator under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

Both C sources are rebuilt with -fsanitize=address,undefined (no recovery) and
tests/sanitize/exercise.py runs them over small cases reaching every entry
point, in a child process with the sanitizer runtime preloaded; any finding
aborts it.  Leak checking is off: the interpreter itself keeps memory to the
end.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _gcc(src, out):
    cmd = ["gcc", *SAN, "-std=c99", "-D_DEFAULT_SOURCE", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
           "-shared", "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True)


def test_oracle_and_generator_are_clean_under_asan_and_ubsan(tmp_path):
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("no AddressSanitizer runtime for gcc")
    olib, slib = str(tmp_path / "liboracle_san.so"), str(tmp_path / "libsynth_san.so")
    _gcc(os.path.join(ROOT, "oracle", "csa2_oracle.c"), olib)
    _gcc(os.path.join(ROOT, "sparse_long_context_amd", "synth_c", "csa2_synth.c"), slib)
    env = dict(os.environ, CSA2_ORACLE_LIB=olib, CSA2_SYNTH_LIB=slib, LD_PRELOAD=asan, OMP_NUM_THREADS="4",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "sanitize", "exercise.py")], env=env,
                       capture_output=True, text=True, timeout=600)
    log = r.stdout + r.stderr
    assert r.returncode == 0, log[-4000:]
    assert "exercise: done" in r.stdout
    assert "runtime error" not in log and "AddressSanitizer" not in log, log[-4000:]
