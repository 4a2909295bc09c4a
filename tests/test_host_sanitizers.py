"""The host side of the C ABI (argument validation, size queries, workspace
carving in api.cpp) under AddressSanitizer and UndefinedBehaviorSanitizer:
the ABI tests run in a child process against the sanitizer build of the
library, with the clang ASan runtime preloaded.  No GPU is used: every call
the ABI tests make is rejected or answered before any HIP work is issued."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CLANG = "/opt/rocm/llvm/bin/clang"


def test_abi_tests_under_host_sanitizers():
    if not os.path.exists(CLANG):
        pytest.skip("ROCm clang not found")
    rt = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                        text=True).stdout.strip()
    if not os.path.exists(rt):
        pytest.skip("clang ASan runtime not found")
    sys.path.insert(0, os.path.dirname(HERE))
    from gpt_decoder_block_amd import build
    lib = build.build_sanitized()
    env = dict(os.environ, GDB_LIB=lib, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_abi.py")], env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, out
    assert " passed" in r.stdout, out
