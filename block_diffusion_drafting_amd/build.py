"""Builds libdflash.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m block_diffusion_drafting_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = ["api.hip", "gemm.hip", "gemm_qkv.hip", "gemm_swiglu.hip", "gemm_part.hip", "gemm_argmax.hip",
           "gemm_proj.hip", "attention.hip", "misc.hip", "persist.hip",
           "loss.hip", "adapt.hip"]
LIB = os.path.join(HERE, "libdflash.so")
ARCH = os.environ.get("DFLASH_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from emitting packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
NOISE = "is not a recognized feature for this target"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.sep not in c or os.path.exists(c)):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stderr or "").splitlines() if NOISE not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False) -> str:
    """Compiles every source to an object (in parallel) and links the
    shared library; objects go to a build folder beside the sources."""
    from concurrent.futures import ThreadPoolExecutor
    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    cc = hipcc()
    jobs = []
    for src in SOURCES:
        obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
        jobs.append((obj, [cc, *HIPCC_FLAGS, "-c", os.path.join(HERE, "csrc", src), "-o", obj]))
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        errs = list(ex.map(lambda j: _run(j[1]), jobs))
    tmp = LIB + ".tmp"
    errs.append(_run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *[o for o, _ in jobs], "-o", tmp]))
    if verbose:
        for e in errs:
            if e.strip():
                print(e, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


# Host code with AddressSanitizer and UndefinedBehaviorSanitizer (every
# sanitizer flag applies to the host compilation only; the device code is
# built as usual and never runs in the tests that use this copy).
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def build_host_sanitized(out_dir: str) -> str:
    """Builds a copy of the library with sanitized host code into out_dir
    (objects and libdflash_san.so) and returns the library's path.  It
    needs the shared ASan runtime (asan_runtime()) preloaded in the process
    that loads it."""
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(out_dir, exist_ok=True)
    cc = hipcc()
    flags = [f"--offload-arch={ARCH}", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *HOST_SANITIZE]
    jobs = []
    for src in SOURCES:
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        jobs.append((obj, [cc, *flags, "-c", os.path.join(HERE, "csrc", src), "-o", obj]))
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        list(ex.map(lambda j: _run(j[1]), jobs))
    lib = os.path.join(out_dir, "libdflash_san.so")
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *[o for o, _ in jobs], "-o", lib])
    return lib


def asan_runtime() -> str:
    """Path of the compiler's shared ASan runtime (its UBSan handlers
    included), to be preloaded in a process that loads build_host_sanitized()."""
    import glob
    root = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    for base in (os.path.join(root, "llvm", "lib", "clang"), os.path.join(root, "lib", "llvm", "lib", "clang")):
        hits = sorted(glob.glob(os.path.join(base, "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
        if hits:
            return hits[-1]
    raise RuntimeError("the shared ASan runtime of the compiler was not found")


if __name__ == "__main__":
    print(build(verbose=True))
