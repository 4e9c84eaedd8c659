"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

The oracle (plain C) is rebuilt with both sanitizers and its pin tests run
against that build in a child process.  The library's host code (descriptor
validation, size accounting, plan checks) runs under them when its sanitizer
build exists (`python -m ternary_weight_amd.build --sanitize`, a few minutes
of compilation, so not part of every run): then the ABI's CPU tests run
against it.  Any sanitizer report fails the child."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(env_extra, tests):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"   # the interpreter itself leaks by design
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        *tests], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


def test_oracle_under_sanitizers(tmp_path):
    import oracle
    so = oracle.build(sanitize=True, out=str(tmp_path / "liboracle_san.so"))
    libasan = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    libubsan = subprocess.check_output(["gcc", "-print-file-name=libubsan.so"], text=True).strip()
    out = _run({"TQ_ORACLE_LIB": so, "LD_PRELOAD": libasan + ":" + libubsan},
               ["tests/test_oracle_pins.py", "tests/test_oracle_chain.py", "tests/test_oracle_ternarize.py"])
    assert " passed" in out


def test_library_host_code_under_sanitizers():
    so = os.path.join(ROOT, "_build", "asan", "libtq.so")
    if not os.path.exists(so):
        pytest.skip("no sanitizer build of libtq (python -m ternary_weight_amd.build --sanitize)")
    rt = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("the compiler's AddressSanitizer runtime is not installed")
    out = _run({"TQ_LIB": so, "LD_PRELOAD": rt[-1]}, ["tests/test_abi.py", "tests/test_b3_layout.py"])
    assert " passed" in out
