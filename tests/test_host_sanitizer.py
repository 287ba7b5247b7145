"""The host code of the library under AddressSanitizer and UndefinedBehaviorSanitizer.

host.cpp (argument validation, the column-interval descriptor builders, the chunk-pair
descriptors, the Variable Block expansion, the tile-index and workspace layouts) is
compiled with g++ -fsanitize=address,undefined -fno-sanitize-recover=all and linked
against launcher stand-ins that abort (tests/sanitize/launch_stubs.cpp). The CPU tests
of the C ABI then run against that build in a child process (MLCT_ATTN_LIB names it,
libasan is preloaded because the Python interpreter is not instrumented): any
out-of-bounds access, use of freed memory, signed overflow, misaligned access or other
undefined behaviour aborts the run, and so does a launch reached on an error path."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST = os.path.join(ROOT, "masked_long_context_tiled_amd", "csrc", "host.cpp")
STUBS = os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp")
ABI_TESTS = ["tests/test_abi.py", "tests/test_abi_select.py", "tests/test_oracle_chunks.py"]


def _gxx(*args):
    return subprocess.run(["g++", *args], capture_output=True, text=True)


@pytest.mark.timeout(900)
def test_abi_tests_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "libattn_host_asan.so")
    r = _gxx("-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all", "-fPIC", "-shared", HOST, STUBS, "-o", lib)
    assert r.returncode == 0, r.stderr
    asan = _gxx("-print-file-name=libasan.so").stdout.strip()
    assert os.path.exists(asan), asan
    env = dict(os.environ)
    env.update(MLCT_ATTN_LIB=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                        *ABI_TESTS], cwd=ROOT, env=env, capture_output=True, text=True)
    tail = (r.stdout[-3000:] + r.stderr[-3000:])
    assert r.returncode == 0, tail
    assert " passed" in r.stdout and "failed" not in r.stdout, tail
