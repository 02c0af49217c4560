"""The C-ABI validation tests (tests/test_abi.py) again, against a build whose
host code (argument checks, status codes, workspace and size arithmetic) is
instrumented with AddressSanitizer and UndefinedBehaviorSanitizer.  Runs in a
child process with the ASan runtime preloaded; any sanitizer report fails the
test.  No GPU: every call fails validation before any HIP call."""
import os
import subprocess
import sys

import pytest

from nvfp4_post_quantization_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def san_env():
    try:
        rt = B.asan_runtime()
    except Exception as e:                               # no hipcc / clang runtime in this image
        pytest.skip(f"sanitizer toolchain unavailable: {e}")
    if not os.path.exists(os.path.join(B.BUILD, "quant.o")):
        B.build()
    lib = B.build_sanitized()
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, NVFP4MI_LIB=lib, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    return env, lib


def _run(cmd, env):
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    return r, out


def test_sanitized_library_is_the_one_loaded(san_env):
    env, lib = san_env
    code = ("import nvfp4_post_quantization_amd as nq; nq.load(); "
            "print(any(l.rstrip().endswith('libnvfp4mi_san.so') for l in open('/proc/self/maps')))")
    r, out = _run([sys.executable, "-c", code], env)
    assert r.returncode == 0, out[-4000:]
    assert r.stdout.strip().endswith("True"), out[-4000:]
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_" in syms and "__ubsan_" in syms


def test_abi_validation_under_sanitizers(san_env):
    env, _ = san_env
    r, out = _run([sys.executable, "-m", "pytest", "tests/test_abi.py", "-q", "-p", "no:cacheprovider"], env)
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out and "skipped" not in out, out[-2000:]
