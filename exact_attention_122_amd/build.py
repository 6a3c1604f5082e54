"""Compile the HIP sources under csrc/ into libfa.so for gfx950 (in-tree).

Usage: python -m exact_attention_122_amd.build [-v] [--sanitize]

``--sanitize`` builds a second library, _build_san/libfa_san.so, whose host
code is instrumented with AddressSanitizer and UndefinedBehaviorSanitizer
(device code is compiled as usual). Loaded into a process that preloads the
ASan runtime, it checks the boundary's host logic: argument validation,
stride and size arithmetic, workspace and scratch bookkeeping.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfa.so")
ARCH = "gfx950"
SAN_BUILD = os.path.join(PKG, "_build_san")
SAN_LIB = os.path.join(SAN_BUILD, "libfa_san.so")


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; a ROCm toolchain is required to build libfa.so")
    return path


COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no NaN-quieting before max/min: every NaN the kernels could see comes
    # from NaN inputs, whose outputs are meaningless either way
    "-fno-honor-nans",
    "-Wall", "-Wno-unused-result",
    "-I", INCLUDE, "-I", CSRC,
]


# host-only sanitizers: each -fsanitize= is scoped to the host pass
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-fno-omit-frame-pointer", "-g"]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, verbose: bool, out_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(out_dir, os.path.basename(src)[:-4] + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *extra, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    """Always recompiles every source, then links libfa.so. Returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def asan_runtime() -> str:
    """Path of the shared ASan runtime that must be preloaded (LD_PRELOAD)
    into a process loading the sanitized library."""
    llvm = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc()))), "llvm")
    hits = sorted(glob.glob(os.path.join(llvm, "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    if not hits:
        hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("the shared ASan runtime (libclang_rt.asan-x86_64.so) was not found")
    return hits[-1]


def _sources_digest(extra) -> str:
    h = hashlib.sha256(" ".join([*COMMON_FLAGS, *extra]).encode())
    for path in sorted(sources() + glob.glob(os.path.join(CSRC, "*.h")) + glob.glob(os.path.join(INCLUDE, "*.h"))):
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def build_host_sanitized(verbose: bool = False) -> str:
    """Build _build_san/libfa_san.so (host code under ASan + UBSan), unless
    one built from the same sources and flags is already there. Returns its
    path."""
    os.makedirs(SAN_BUILD, exist_ok=True)
    stamp = os.path.join(SAN_BUILD, "sources.sha256")
    digest = _sources_digest(SAN_FLAGS)
    if os.path.exists(SAN_LIB) and os.path.exists(stamp) and open(stamp).read().strip() == digest:
        return SAN_LIB
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, SAN_BUILD, SAN_FLAGS), srcs))
    tmp = SAN_LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libsan",
           *SAN_FLAGS[:4], *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, SAN_LIB)
    with open(stamp, "w") as f:
        f.write(digest + "\n")
    return SAN_LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_host_sanitized(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
