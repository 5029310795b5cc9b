"""Builds libolmo3attn.so in-tree with hipcc for gfx950.

Each HIP source is compiled to an object in ``_build/`` (in parallel), then
linked into ``global_hybrid_causal_amd/libolmo3attn.so``.  The library is
written under a temporary name and renamed, so a reader never sees a
half-written file.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libolmo3attn.so")
SOURCES = ["api.hip", "prologue.hip", "attn.hip", "prefill.hip"]
ARCH = "gfx950"

# -packed-fp32-ops: keep hipcc from emitting packed fp32 VALU operations.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libolmo3attn.so")
    return path


# The prefill kernel's maxima never see a NaN (masked scores are -inf), so
# fmax needs no NaN quieting there.
PER_FILE_FLAGS = {"prefill.hip": ["-fno-honor-nans"]}


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *PER_FILE_FLAGS.get(src, []), *extra, "-c",
           os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(extra_flags: list[str] | None = None, verbose: bool = False) -> str:
    """Compile every HIP source and link the shared library; returns its path."""
    extra = list(extra_flags or [])
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


# Host-side AddressSanitizer + UBSan build of the same sources, for running
# the argument validation (sizes, 128-bit byte counts, overlap spans) under
# the sanitizers on the CPU.  Only the host code is instrumented
# (-Xarch_host): device code is built as usual and never runs there.
SAN_BUILD = os.path.join(PKG, "_build_san")
SAN_LIB = os.path.join(SAN_BUILD, "libolmo3attn_san.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
             "-fno-omit-frame-pointer", "-g"]


def sanitizer_runtime() -> str | None:
    """The clang AddressSanitizer runtime the sanitized library links to
    (it must be preloaded into a process that loads that library)."""
    res = subprocess.run([hipcc(), "--print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
        return path
    import glob
    found = sorted(glob.glob("/opt/rocm*/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def build_host_sanitized(verbose: bool = False) -> str:
    """Compile the library with host-only ASan/UBSan into SAN_LIB."""
    os.makedirs(SAN_BUILD, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(SAN_BUILD, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc(), *COMMON_FLAGS, *PER_FILE_FLAGS.get(src, []), *SAN_FLAGS, "-c",
               os.path.join(CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc (host sanitizers) failed on {src}:\n{res.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = SAN_LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host",
           "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host",
           "-shared-libsan", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link (host sanitizers) failed:\n{res.stderr}")
    os.replace(tmp, SAN_LIB)
    if verbose:
        print(f"built {SAN_LIB}", file=sys.stderr)
    return SAN_LIB


if __name__ == "__main__":
    build(verbose=True)
