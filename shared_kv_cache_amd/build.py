"""Build the gfx950 library (``_lib/libhogwild.so``) with hipcc, in-tree.

Usage: ``python -m shared_kv_cache_amd.build`` (or ``__graft_entry__.build()``).
Always recompiles. The library exports the C ABI of ``include/hogwild.h`` and
``include/hogwild_debug.h``.

``--asan-host OUT``: build a copy at OUT whose host code (not the device code) carries
AddressSanitizer, for the CPU tests of the host logic; load it with the sanitizer runtime
preloaded (``clang -print-file-name=libclang_rt.asan-x86_64.so``).
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB_DIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIB_DIR, "libhogwild.so")
SOURCES = [os.path.join(PKG, "csrc", "hw_host.cpp"), os.path.join(PKG, "csrc", "hw_kernels.hip")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 arithmetic off on the device: plain scalar fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # leading scalar kernel arguments preloaded into scalar registers at dispatch (gfx950):
    # the merge kernel's; kernels whose first argument is a struct preload nothing
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall", "-Wno-unused-result",
    "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(PKG, "csrc"),
    "-Wl,-rpath,/opt/rocm/lib",
]


ASAN_HOST = ["-O1", "-g", "-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer"]


def build(verbose: bool = True, out: str = LIB, extra=()) -> str:
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    if len(sys.argv) == 3 and sys.argv[1] == "--asan-host":
        build(verbose=True, out=os.path.abspath(sys.argv[2]), extra=ASAN_HOST)
    else:
        build(verbose=True)
    sys.exit(0)
