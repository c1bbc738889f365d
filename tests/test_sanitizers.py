"""Host-only builds under AddressSanitizer and UndefinedBehaviorSanitizer of
the C ABI's argument checks (with the self-test's reference values) and of
the CPU oracle, run on small and edge-case inputs. Needs no GPU: the
validator is plain C++ and the oracle plain C; each harness is built with gcc
or g++ into a temporary directory and must exit 0 with no sanitizer report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dsa_top_sparse_amd", "csrc")
SAN = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                                reason="needs gcc and g++")


def _build_and_run(cmd, exe):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"build failed:\n{r.stderr}"
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=120)
    assert r.returncode == 0 and "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr
    return r.stdout


def test_validator_under_sanitizers(tmp_path):
    exe = str(tmp_path / "validate_harness")
    cmd = ["g++", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "sanitize", "validate_harness.cpp"), os.path.join(CSRC, "validate.cpp"),
           "-o", exe]
    assert "validate harness: ok" in _build_and_run(cmd, exe)


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_harness")
    cmd = ["gcc", "-std=c11", *SAN, os.path.join(ROOT, "tests", "sanitize", "oracle_harness.c"),
           os.path.join(ROOT, "oracle", "dsa_oracle.c"), "-o", exe, "-lm"]
    assert "oracle harness: ok" in _build_and_run(cmd, exe)
