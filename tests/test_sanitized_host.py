"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the oracle and the HIP library's host pass with both sanitizers
(clang; one sanitizer runtime for the process; GPU code as usual), then runs
the C-ABI checks and the oracle's pins against those builds in a child
process with the runtime preloaded.  Any report fails the test.  CPU only."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ASAN_RT = "/opt/rocm/llvm/lib/clang/%s/lib/linux/libclang_rt.asan-x86_64.so"


def _asan_runtime():
    base = "/opt/rocm/llvm/lib/clang"
    for v in sorted(os.listdir(base)) if os.path.isdir(base) else []:
        p = ASAN_RT % v
        if os.path.exists(p):
            return p
    return None


def test_host_code_clean_under_asan_ubsan():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("clang's sanitizer runtime is not installed")
    import oracle
    from free_sparse_swiglu_stage1_amd import build as hip_build

    lib = hip_build.build(sanitize=True)
    olib = oracle.build_sanitized()
    env = dict(os.environ, LD_PRELOAD=rt, PROX_LIB=lib, PROX_ORACLE_LIB=olib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=87")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        "tests/test_abi.py", "tests/test_oracle_pins.py"],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=900)
    tail = r.stdout[-4000:]
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in r.stdout and "runtime error:" not in r.stdout, tail
    assert " passed" in tail, tail
