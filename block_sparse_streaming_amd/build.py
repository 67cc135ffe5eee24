"""Build the SSA HIP library (libssa.so) in-tree for gfx950.

Every source is compiled with hipcc for gfx950 only; packed-fp32 instructions
are disabled in device code. Objects are built in parallel and linked into
``block_sparse_streaming_amd/libssa.so``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libssa.so")
SOURCES = ["api.cpp", "prefill.hip", "backward.hip", "decode.hip"]
ARCH = "gfx950"
# decode.hip's MFMA kernel and the backward kernels keep their accumulators in
# VGPRs (scores feed VALU work) and their read-only operands in AGPRs; the VGPR
# form of MFMA lets the compiler do that without copying accumulators around.
EXTRA_FLAGS = {"decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "backward.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the SSA library needs ROCm to build")
    return path


def common_flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fno-strict-aliasing",
            "-Wall", "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include")]


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libssa.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmd = [cc, *common_flags(), *EXTRA_FLAGS.get(src, []), "-x", "hip", "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # The host pass does not know the packed-fp32 feature; that note is noise.
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]
        if lines and (verbose or p.returncode):
            print(f"[{src}]\n" + "\n".join(lines), file=sys.stderr)
        if p.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB + ".tmp"
    subprocess.check_call([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


SANITIZE_DIR = os.path.join(BUILD_DIR, "sanitize")
SANITIZED_LIB = os.path.join(SANITIZE_DIR, "libssa_host_asan.so")


def build_host_sanitized() -> str:
    """A second libssa.so whose host code (api.cpp: argument checks, planning,
    workspace layout) is built with AddressSanitizer and UBSan; the kernels
    are the normal objects (device code is not sanitized). Loaded only when
    SSA_LIB names it, with the clang ASan runtime preloaded."""
    if not all(os.path.exists(os.path.join(BUILD_DIR, os.path.splitext(x)[0] + ".o")) for x in SOURCES):
        build()
    os.makedirs(SANITIZE_DIR, exist_ok=True)
    cc = hipcc()
    obj = os.path.join(SANITIZE_DIR, "api.o")
    host_flags = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
              "-fno-omit-frame-pointer", "-g"):
        host_flags += ["-Xarch_host", f]
    subprocess.check_call([cc, *common_flags(), *host_flags, "-x", "hip", "-c",
                           os.path.join(CSRC, "api.cpp"), "-o", obj],
                          stderr=subprocess.DEVNULL)
    objs = [obj] + [os.path.join(BUILD_DIR, os.path.splitext(x)[0] + ".o") for x in SOURCES if x != "api.cpp"]
    tmp = SANITIZED_LIB + ".tmp"
    subprocess.check_call([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, SANITIZED_LIB)
    return SANITIZED_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
