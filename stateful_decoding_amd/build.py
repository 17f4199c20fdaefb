"""Build the gfx950 C-ABI library ``librlt.so`` in-tree with hipcc.

Usage: ``python -m stateful_decoding_amd.build`` (or ``build()`` from Python). Every call
compiles from source; nothing is cached.
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
LIB = os.path.join(PKG, "librlt.so")

SOURCES = ["api.cpp", "gemm.hip", "attention.hip", "misc.hip", "parallel.hip", "backward.hip",
           "head.hip", "noalloc.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep packed fp32 instructions out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build librlt.so")
    return exe


def build(verbose: bool = False, jobs: int = 4, out_dir: str | None = None,
          defines: tuple = ()) -> str:
    """Compile every source to an object, then link ``librlt.so`` (in the package, or in
    ``out_dir``; ``defines`` are extra ``NAME=VALUE`` preprocessor definitions). Returns the
    library path."""
    objdir = os.path.join(out_dir or PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    lib = os.path.join(out_dir, "librlt.so") if out_dir else LIB
    dflags = [f"-D{x}" for x in defines]
    cc = hipcc()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc, *HIPCC_FLAGS, *dflags, "-I", INCLUDE, "-I", CSRC, *lang, "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                            stderr=subprocess.STDOUT, text=True)))
        if len(procs) >= jobs:
            _wait(procs.pop(0), verbose)
    for p in procs:
        _wait(p, verbose)
    tmp = lib + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}")
    os.replace(tmp, lib)
    return lib


def build_host_asan(main_src: str, exe: str, jobs: int = 8) -> str:
    """Compile every library source and ``main_src`` with AddressSanitizer on the host code
    only (the device code is built as usual) and link the executable ``exe``. For checks of
    the host logic that run without a GPU; nothing here is part of ``librlt.so``."""
    objdir = os.path.join(os.path.dirname(os.path.abspath(exe)), "obj")
    os.makedirs(objdir, exist_ok=True)
    asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = [f for f in HIPCC_FLAGS if f != "-O3"] + ["-O1", "-g", *asan]
    cc = hipcc()
    procs, objs = [], []
    for src in [os.path.join(CSRC, s) for s in SOURCES] + [os.path.abspath(main_src)]:
        obj = os.path.join(objdir, os.path.splitext(os.path.basename(src))[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc, *flags, "-I", INCLUDE, "-I", CSRC, *lang, "-c", src, "-o", obj]
        procs.append((os.path.basename(src), subprocess.Popen(
            cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        if len(procs) >= jobs:
            _wait(procs.pop(0), False)
    for p in procs:
        _wait(p, False)
    r = subprocess.run([cc, "--offload-arch=gfx950", *asan, *objs, "-o", exe],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}")
    return exe


def _wait(item, verbose):
    src, p = item
    out, _ = p.communicate()
    if p.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{out}")
    if verbose and out.strip():
        print(_filter(out), flush=True)


def _filter(text: str) -> str:
    # hipcc's host pass does not know the packed-fp32 target feature; that note is harmless.
    return "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
