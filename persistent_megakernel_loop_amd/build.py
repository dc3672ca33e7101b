"""Compile the HIP library (libmk.so) for gfx950, in-tree.

    python -m persistent_megakernel_loop_amd.build
    python -m persistent_megakernel_loop_amd.build --host-sanitizers OUT.so

The second form builds the same sources with AddressSanitizer and
UndefinedBehaviorSanitizer on the host side only (the device code is built as
usual): a check of the library's host code, loaded through MK_LIBRARY with the
sanitizer runtime preloaded (see ``sanitizer_env``).

Every HIP source is compiled with packed-fp32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmk.so")
SOURCES = ["mk_kernel.hip", "mk_phased.hip", "mk_aux.hip", "mk_prefill.hip", "mk_pprefill.hip", "mk_bench.hip", "mk_api.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libmk.so")
    os.replace(tmp, LIB)
    return LIB


def build_host_sanitized(out: str, verbose: bool = False) -> str:
    """The library with ASan + UBSan on its host code (-Xarch_host before each flag)."""
    tmp = out + ".tmp"
    san = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"):
        san += ["-Xarch_host", f]
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", "-shared", "-shared-libsan",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *san,
           "-I", INCLUDE, "-I", CSRC, *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building the host-sanitized library")
    os.replace(tmp, out)
    return out


def sanitizer_env(lib_path: str) -> dict:
    """Environment that loads lib_path through MK_LIBRARY with the ASan runtime preloaded."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang++")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang++"
    rt = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                        text=True).stdout.strip()
    env = dict(os.environ)
    env.update(MK_LIBRARY=lib_path, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    return env


if __name__ == "__main__":
    if len(sys.argv) > 2 and sys.argv[1] == "--host-sanitizers":
        print(build_host_sanitized(sys.argv[2], verbose=True))
    else:
        print(build(verbose=True))
