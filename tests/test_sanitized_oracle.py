"""The oracle and the input generator built with AddressSanitizer and
UndefinedBehaviorSanitizer (host code only), and the oracle pins and generator tests run
against those builds in a child process: an out-of-bounds access, a use after free or
undefined behaviour in either library fails the run. CPU only."""
import os
import shutil
import subprocess
import sys

import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name: str) -> str:
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True, check=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else ""


@pytest.mark.slow
def test_oracle_and_generator_clean_under_sanitizers(tmp_path):
    asan = _runtime("libasan.so")
    if not asan or shutil.which("gcc") is None or shutil.which("g++") is None:
        pytest.skip("no gcc AddressSanitizer runtime")
    olib = oracle.build(out=str(tmp_path / "liboracle_san.so"), sanitize=True)
    slib = synth.build(out=str(tmp_path / "libsynth_san.so"), sanitize=True)
    env = dict(os.environ)
    env.update({
        "MOE_ORACLE_LIB": olib,
        "MOE_SYNTH_LIB": slib,
        # the sanitizer runtime must come first in a Python that is not itself instrumented;
        # the interpreter's own allocations are not checked for leaks
        "LD_PRELOAD": ":".join(p for p in (asan, _runtime("libubsan.so")) if p),
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:verify_asan_link_order=0",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
        "OMP_NUM_THREADS": "4",
    })
    tests = [os.path.join(ROOT, "tests", n) for n in ("test_oracle_pins.py", "test_synth.py", "test_golden.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu and not slow", "-p", "no:cacheprovider", "-s",
                        *tests], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
    assert " passed" in r.stdout, tail
