"""The ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

build.py --sanitize-host compiles the same sources with host-only -fsanitize=address
and -fsanitize=undefined (recovery off, so any finding aborts) into
_build/sanitize/libsmol.so; tests/test_abi_cpu.py then runs in a child process that
loads that copy, with clang's ASan runtime preloaded. Every argument check, workspace
computation and status path those tests drive runs instrumented; the child must pass
with no sanitizer report. The product library is built with -Werror."""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "llama_decoder_only_amd", "csrc")
sys.path.insert(0, CSRC)
import build as BUILD  # noqa: E402


def _hipcc_ok():
    try:
        return subprocess.run([BUILD.HIPCC, "--version"], capture_output=True).returncode == 0
    except OSError:
        return False


def test_product_build_treats_warnings_as_errors():
    assert "-Werror" in BUILD.FLAGS and "-Wall" in BUILD.FLAGS


def test_sanitizer_flags_are_host_only():
    flags = BUILD.SAN_FLAGS
    for i, f in enumerate(flags):
        if f.startswith("-fsanitize"):
            assert i > 0 and flags[i - 1] == "-Xarch_host", f


@pytest.mark.skipif(not _hipcc_ok(), reason="hipcc not available")
def test_abi_host_checks_clean_under_asan_and_ubsan():
    srcs = glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h")) + \
        [os.path.join(ROOT, "include", "smol.h"), os.path.join(CSRC, "build.py")]
    lib = BUILD.SAN_LIB
    if not os.path.exists(lib) or os.path.getmtime(lib) < max(os.path.getmtime(p) for p in srcs):
        BUILD.build(jobs=min(8, os.cpu_count() or 1), sanitize_host=True)
    env = dict(os.environ)
    env["LD_PRELOAD"] = " ".join(p for p in (BUILD.sanitizer_runtime(), env.get("LD_PRELOAD", "")) if p)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"  # the interpreter itself is not instrumented
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["SMOL_LIB_PATH"] = lib
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "Sanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
