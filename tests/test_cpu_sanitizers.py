"""The CPU code under AddressSanitizer and UndefinedBehaviorSanitizer.

Two builds, made here in a temporary directory:
  * the C oracle (``oracle/gdr_oracle.c``) by clang with -fsanitize=address,undefined;
  * the library with its host code instrumented the same way (the argument
    validation, workspace sizing and planning of the C ABI; device code is
    compiled as usual and never runs here).
A child process with clang's ASan runtime preloaded then runs the oracle's pins
(``test_oracle_pins.py``) against the instrumented oracle and the host-side ABI
tests (``test_abi_cpu.py``) against the instrumented library.  Any memory error
or undefined behaviour ends that process with an error, failing this test."""
import glob
import os
import subprocess
import sys

import pytest

from gated_delta_rule_85_amd import build as hip_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.slow
def test_oracle_and_host_code_under_asan_and_ubsan(tmp_path):
    rt = _asan_runtime()
    if rt is None or not os.path.exists(CLANG) or not os.path.exists(hip_build.HIPCC):
        pytest.skip("ROCm clang toolchain with its ASan runtime not found")
    oracle_lib = str(tmp_path / "liboracle_san.so")
    subprocess.run([CLANG, "-O1", "-g", "-std=c99", "-fPIC", "-shared", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    os.path.join(ROOT, "oracle", "gdr_oracle.c"), "-o", oracle_lib], check=True)
    host_lib = hip_build.build(out=str(tmp_path / "libgdr_san.so"), sanitize=True,
                               build_dir=str(tmp_path / "obj"))
    env = dict(os.environ, LD_PRELOAD=rt, GDR_LIB=host_lib, GDR_ORACLE_LIB=oracle_lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "tests/test_abi_cpu.py", "tests/test_oracle_pins.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
