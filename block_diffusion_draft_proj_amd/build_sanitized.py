"""Host-sanitizer build of the C ABI: ``_build/libdflash_san.so``.

``api.cpp`` (the C entry points: argument checks, planning, launches) is compiled
with AddressSanitizer and UndefinedBehaviorSanitizer on its host code only and
linked with the device objects that ``build.py`` left under ``_build/``.  Device
code is not instrumented.  The library is loaded with the clang ASan runtime
preloaded (``asan_runtime()``) and ``DFLASH_LIB`` naming it; it is for host-side
tests of the validation code (no GPU needed), never for the GPU path.
"""
from __future__ import annotations

import glob
import os
import subprocess

from block_diffusion_draft_proj_amd import build as B

LIB = os.path.join(B.BUILD, "libdflash_san.so")
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def _host(flags):
    out = []
    for f in flags:  # every sanitizer flag applies to the host pass only
        out += ["-Xarch_host", f]
    return out


def asan_runtime() -> str:
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise RuntimeError("clang ASan runtime not found under /opt/rocm/llvm")
    return found[-1]


def build() -> str:
    hipcc = B._hipcc()
    objs = [os.path.join(B.BUILD, os.path.splitext(s)[0] + ".o") for s in B.SOURCES if s != "api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        B.build()
    api = os.path.join(B.BUILD, "api_san.o")
    flags = [f for f in B.HIP_FLAGS if f != "-O3"] + ["-O1", "-g"]
    cmd = [hipcc, "-x", "hip", *flags, *_host(SAN), "-c", os.path.join(B.CSRC, "api.cpp"), "-o", api]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"sanitized compile failed:\n{r.stderr}")
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *_host(SAN[:2]), "-shared-libasan", api, *objs,
           "-o", LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"sanitized link failed:\n{r.stderr}")
    return LIB


if __name__ == "__main__":
    print(build())
