"""Build libtt_emb.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: python -m tensor_train_compressed_amd.build   (or build() from Python)

Each .hip source is compiled to an object in parallel, then linked into
tensor_train_compressed_amd/libtt_emb.so next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libtt_emb.so")
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

# -packed-fp32-ops keeps the compiler from emitting packed-FP32 VALU ops.
# -munsafe-fp-atomics turns float atomicAdd into the hardware global float add
# (device memory from hipMalloc is coarse-grained, where that instruction is valid).
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-munsafe-fp-atomics",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC,
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer flags: every
# -fsanitize goes to the host compilation only (device code is not
# instrumented). A process that loads this library must preload clang's ASan
# runtime (asan_runtime()) and point TT_EMB_LIBRARY at it.
HOST_SANITIZE = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
]


def asan_runtime() -> str:
    """clang's shared ASan runtime (it also carries the UBSan handlers)."""
    llvm = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm")
    hits = sorted(glob.glob(os.path.join(llvm, "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise RuntimeError("clang's ASan runtime was not found next to hipcc")
    return os.path.realpath(hits[-1])


def build_host_sanitized(out_dir: str) -> str:
    """Build the same sources with host-side sanitizers (device code at -O1,
    never run by the host checks) into out_dir/libtt_emb_san.so."""
    os.makedirs(out_dir, exist_ok=True)
    flags = [a for a in COMMON if a != "-O3"] + ["-O1", "-g"] + HOST_SANITIZE

    def one(src):
        obj = os.path.join(out_dir, os.path.basename(src) + ".o")
        r = subprocess.run([HIPCC, *flags, "-c", src, "-o", obj], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(sources()))) as ex:
        objs = list(ex.map(one, sources()))
    lib = os.path.join(out_dir, "libtt_emb_san.so")
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", lib],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    return lib


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
