"""The oracle's pins, run against an AddressSanitizer + UndefinedBehavior-
Sanitizer build of oracle.c (every finding fatal), in a child process with the
ASan runtime preloaded.  Checks that the reference checker itself reads and
writes only inside its arrays and executes no undefined behaviour on the
pinned inputs (out-of-range labels, empty rows, -inf log-weights, tails,
causal, GQA, permutations, token sets, sampler cases)."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_FILES = ["test_oracle_attn.py", "test_oracle_csr_sched.py", "test_oracle_crm.py", "test_oracle_sampler.py",
             "test_oracle_tok.py", "test_oracle_mcsparse.py", "test_oracle_spectral.py", "test_metrics.py"]


def _libasan():
    try:
        out = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True, check=True)
    except (OSError, subprocess.CalledProcessError):
        return None
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_sanitizers(tmp_path):
    asan = _libasan()
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    so = oracle.build_sanitized(str(tmp_path / "liboracle_san.so"))
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": asan,
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "BSA_ORACLE_LIB": so,
        "OMP_NUM_THREADS": "4",
    })
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider"] + \
          [os.path.join(ROOT, "tests", f) for f in PIN_FILES]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = "\n".join((res.stdout + res.stderr).splitlines()[-40:])
    assert res.returncode == 0, "oracle pins failed under sanitizers:\n" + tail
    assert "passed" in res.stdout, tail
    # the sanitized library (not the plain one) was the one loaded
    assert "ERROR: AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr, tail
