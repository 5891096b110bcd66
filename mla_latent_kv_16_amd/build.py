"""Builds libmla.so (the gfx950 HIP kernels and their C ABI) in-tree with hipcc.

Usage: python -m mla_latent_kv_16_amd.build [--save-temps DIR]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmla.so")
SOURCES = ["mla_api.hip", "mla_kernels.hip", "mla_splitkv8.hip", "mla_splitkvq.hip",
           "mla_append.hip", "mla_project.hip"]
# the achievable-peak microbenchmarks the benchmark measures its denominators with
PEAKS_LIB = os.path.join(PKG, "libmla_peaks.so")
PEAKS_SOURCES = ["mla_peaks.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # gfx950 packed-fp32 instructions stay off; ordinary float code is used instead
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; ROCm is required to build libmla.so")


# libmla.so again with its host code under AddressSanitizer (the device code is the
# same), for the CPU tests of the C ABI's host-side checks; the ASan runtime is loaded
# by the test process, not linked in
HOSTCHECK_LIB = os.path.join(PKG, "libmla_hostcheck.so")
HOSTCHECK_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
                   "-shared-libasan"]


def build(verbose: bool = True, extra=()) -> str:
    """Compiles libmla.so (the attention path), libmla_peaks.so (the peak
    microbenchmarks) and libmla_hostcheck.so (libmla.so with AddressSanitizer on its
    host code) next to this file; returns the path of libmla.so."""
    _build_one(PEAKS_LIB, PEAKS_SOURCES, verbose, extra)
    _build_one(HOSTCHECK_LIB, SOURCES, verbose, [*extra, *HOSTCHECK_FLAGS])
    return _build_one(LIB, SOURCES, verbose, extra)


def asan_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (for LD_PRELOAD)."""
    res = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the AddressSanitizer runtime of hipcc's clang was not found")
    return path


def _build_one(lib: str, sources, verbose: bool, extra) -> str:
    tmp = lib + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-I", os.path.join(ROOT, "include"),
           *[os.path.join(CSRC, s) for s in sources], "-o", tmp]
    if verbose:
        print("[build]", " ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    extra = []
    if len(sys.argv) > 2 and sys.argv[1] == "--save-temps":
        os.makedirs(sys.argv[2], exist_ok=True)
        extra = ["-save-temps=obj", "-o"]  # placeholder, handled below
        cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"),
               "--cuda-device-only", "-S"]
        for s in SOURCES + PEAKS_SOURCES:
            out = os.path.join(sys.argv[2], s.replace(".hip", ".s"))
            subprocess.run(cmd + [os.path.join(CSRC, s), "-o", out], check=True)
            print(out)
    else:
        print(build())
