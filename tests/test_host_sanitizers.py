"""The host runtime under AddressSanitizer and UndefinedBehaviorSanitizer.

A host-sanitized copy of the library (device code unchanged, never run here)
is built, and the CPU ABI tests (validation of every entry point, handle
creation, binding, the size queries, error paths) run against it in a child
process with the sanitizer runtime preloaded; any report aborts the child.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import ctypes, sys
sys.path.insert(0, {tests!r}); sys.path.insert(0, {root!r})
ctypes.CDLL(None).__asan_init  # the sanitizer runtime is in the process
import block_diffusion_drafter_proj_amd.binding as B
B.LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main([{abi!r}, "-q", "-x", "-p", "no:cacheprovider"]))
"""


def test_abi_tests_pass_under_host_sanitizers():
    if not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("no hipcc")
    from block_diffusion_drafter_proj_amd import build_sanitized as S
    rt = S.runtime_path()
    if not rt or not os.path.exists(rt):
        pytest.skip("no AddressSanitizer runtime in the toolchain")
    lib = S.build(jobs=8)
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = CHILD.format(tests=os.path.join(ROOT, "tests"), root=ROOT, lib=lib,
                        abi=os.path.join(ROOT, "tests", "test_abi_cpu.py"))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout
