"""Build libpkv.so (HIP for gfx950) in-tree with hipcc.

    python -m paged_kv_cache_190_amd.build      # or __graft_entry__.build()

Objects go to _build/ at the repository root, the libraries to paged_kv_cache_190_amd/lib/:
libpkv.so, and the debug and host-sanitizer variants of it (see VARIANTS). Every call compiles
from scratch.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libpkv.so")
OBJDIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

SOURCES = ["api.cpp", "block_manager.cpp", "kv_write.hip", "decode.hip", "prefill.hip",
           "blocks.hip", "debug.hip"]

# Packed-fp32 VALU instructions are disabled for the device pass; hipcc -O3 would otherwise
# form them from plain float code. The host pass warns that it does not know the feature.
# MFMA accumulators are kept in ordinary VGPRs: the softmax rescales them every few tiles, and
# in AGPRs each rescale would cost a read, a multiply and a write per element.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-mfma-vgpr-form=1"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include")]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found (ROCm is required to build libpkv)")
    return exe


# Library variants built from the same sources:
#   release  libpkv.so          what the binding, tests and benchmark load
#   debug    libpkv_debug.so    PKV_DEBUG=1: device-array checks before every call
#   hostsan  libpkv_hostsan.so  host code under AddressSanitizer and UndefinedBehaviorSanitizer
#                               (device code unchanged); loaded only by a CPU test, with the
#                               sanitizer runtime preloaded
VARIANTS = {
    "release": ("libpkv.so", []),
    "debug": ("libpkv_debug.so", ["-DPKV_DEBUG=1"]),
    "hostsan": ("libpkv_hostsan.so",
                ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
                 "-fno-omit-frame-pointer", "-Xarch_host", "-g"]),
}


def lib_path(variant: str = "release") -> str:
    return os.path.join(LIBDIR, VARIANTS[variant][0])


def _compile(job) -> str:
    variant, src = job
    flags = VARIANTS[variant][1]
    obj = os.path.join(OBJDIR, variant, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, *DEVICE_FLAGS, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    return obj


def _link(variant: str, objs) -> str:
    out = lib_path(variant)
    tmp = out + ".tmp"
    vf = VARIANTS[variant][1]
    flags = []  # the link takes the sanitizer selections (each after its -Xarch_host)
    for i in range(len(vf) - 1):
        if vf[i] == "-Xarch_host" and vf[i + 1].startswith("-fsanitize="):
            flags += vf[i:i + 2]
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *flags, *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    if variant != "hostsan":
        # Load the result with every symbol resolved now, so an unresolved kernel stub fails
        # the build rather than the first test (dlopen needs no GPU). (The sanitized variant
        # loads only with its runtime preloaded.)
        import ctypes
        try:
            ctypes.CDLL(tmp, mode=os.RTLD_NOW)
        except OSError as e:
            raise RuntimeError(f"built library does not load: {e}") from e
    os.replace(tmp, out)
    return out


def build(verbose: bool = True, variants=("release", "debug", "hostsan")) -> str:
    """Compile every source for each variant (all compilations in one pool) and link them.
    Returns the release library's path."""
    for v in variants:
        os.makedirs(os.path.join(OBJDIR, v), exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    jobs = [(v, src) for v in variants for src in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, jobs))
    for v in variants:
        out = _link(v, [o for (vv, _), o in zip(jobs, objs) if vv == v])
        if verbose:
            print(f"built {out}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
