"""Build libsmol.so (all HIP kernels + the C ABI) for gfx950 with hipcc, in-tree.

    python llama_decoder_only_amd/csrc/build.py [--jobs N] [--sanitize-host]

Objects go to _build/ at the repository root; the library lands next to the
Python binding (llama_decoder_only_amd/libsmol.so). Warnings are errors.

--sanitize-host builds a separate copy, _build/sanitize/libsmol.so, whose host code
(argument checks, workspace layout, launch sequencing) carries AddressSanitizer and
UndefinedBehaviorSanitizer; the device code is compiled as usual. It is meant for
the CPU tests of the ABI: load it with the clang ASan runtime preloaded
(SANITIZER_RUNTIME below) and SMOL_LIB_PATH pointing at it.
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsmol.so")
SAN_BUILD = os.path.join(BUILD, "sanitize")
SAN_LIB = os.path.join(SAN_BUILD, "libsmol.so")

SOURCES = ["api.hip", "gemm.hip", "attention.hip", "decode_attention.hip", "decode_xcd.hip", "norm_embed.hip", "sample.hip", "backward.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else "hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-mcode-object-version=5",
    # keep hipcc from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Werror",
    "-Wno-unused-variable",
    "-Wno-unused-function",
    "-I", INCLUDE,
    "-I", HERE,
]


# Host-only sanitizers: every -fsanitize= goes to the host compilation alone
# (-Xarch_host), so the gfx950 code objects are the ones of the normal build.
SAN_FLAGS = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
    "-Xarch_host", "-g",
]


def sanitizer_runtime() -> str:
    """Path of clang's shared ASan runtime (it carries the UBSan handlers too)."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("clang ASan runtime not found")
    return path


def _compile(src: str, sanitize: bool = False) -> str:
    out = SAN_BUILD if sanitize else BUILD
    obj = os.path.join(out, src + ".o")
    cmd = [HIPCC, *FLAGS, *(SAN_FLAGS if sanitize else []), "-c", os.path.join(HERE, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    noise = "is not a recognized feature for this target"
    for line in (r.stderr or "").splitlines():
        if line.strip() and noise not in line:
            sys.stderr.write(line + "\n")
    return obj


def build(jobs: int = 8, sanitize_host: bool = False) -> str:
    """Compile every source and link the library; returns its path. With
    sanitize_host, the sanitizer copy (SAN_LIB) instead of the product library. The
    sanitizer copy leaves its ASan/UBSan symbols to the preloaded runtime."""
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError("hipcc not found")
    out, lib = (SAN_BUILD, SAN_LIB) if sanitize_host else (BUILD, LIB)
    os.makedirs(out, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize_host), SOURCES))
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc link failed")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--sanitize-host", action="store_true",
                    help="build _build/sanitize/libsmol.so with host-side ASan + UBSan")
    args = ap.parse_args()
    print(build(args.jobs, args.sanitize_host))
