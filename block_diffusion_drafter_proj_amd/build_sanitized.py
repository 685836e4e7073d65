"""Builds a host-sanitized copy of libdflash.so for the CPU tests.

Usage: python -m block_diffusion_drafter_proj_amd.build_sanitized

The host code of every source under csrc/ (argument validation, the
workspace carve-up, the launch sequences) is compiled with AddressSanitizer
and UndefinedBehaviorSanitizer; the device code is compiled as usual and is
never run from this copy (it is for tests without a GPU).  The library goes
to _build/host_sanitized/libdflash.so and is loaded with the sanitizer
runtime preloaded (see `runtime_path`).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

from .build import ARCH, HIPCC, ROOT, sources

OUT_DIR = os.path.join(ROOT, "_build", "host_sanitized")
LIB = os.path.join(OUT_DIR, "libdflash.so")
# -Xarch_host before each sanitizer flag: host code only
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer"]
CFLAGS = [f"--offload-arch={ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-I", os.path.join(ROOT, "include")] + SAN


def runtime_path() -> str:
    """The AddressSanitizer runtime of the toolchain (to be preloaded)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return r.stdout.strip()


def _compile(src):
    obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
    r = subprocess.run([HIPCC, *CFLAGS, "-c", src, "-o", obj], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(jobs: int = 8) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    with ThreadPoolExecutor(max(1, jobs)) as ex:
        objs = list(ex.map(_compile, sources()))
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *SAN, *objs, "-o", LIB],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    return LIB


if __name__ == "__main__":
    print(build(min(16, os.cpu_count() or 4)))
    sys.exit(0)
