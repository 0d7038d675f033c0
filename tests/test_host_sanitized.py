"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds ``_build/libdflash_san.so`` (api.cpp instrumented on the host, device code as
usual) and runs the host-only ABI suites against it in a child process with the
ASan runtime preloaded: the validation tests and the randomised argument checks.
Any out-of-bounds host access, use of freed memory or undefined arithmetic aborts
the child.  CPU only: the child's calls never reach a device.
"""
import os
import shutil
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0 or not (shutil.which("hipcc") or
                                                                       os.path.exists("/opt/rocm/bin/hipcc")),
                                reason="host-only: needs hipcc and no visible GPU")


def test_abi_suites_under_host_sanitizers():
    from block_diffusion_draft_proj_amd import build_sanitized as S
    lib = S.build()
    env = dict(os.environ, LD_PRELOAD=S.asan_runtime(), DFLASH_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    check = "from block_diffusion_draft_proj_amd import dflash as d; assert d.LIB_PATH.endswith('libdflash_san.so')"
    r = subprocess.run([sys.executable, "-c", check], env=env, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "tests/test_abi_cpu.py", "tests/test_abi_fuzz_cpu.py"],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    tail = (r.stdout[-3000:] + "\n" + r.stderr[-3000:])
    assert r.returncode == 0, tail
    assert "Sanitizer" not in r.stderr, tail
    assert " passed" in r.stdout, tail
