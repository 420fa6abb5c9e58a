"""Build libpda.so (HIP kernels for gfx950 + the C-ABI host code) in-tree.

    python -m decode_attention_paged_02_amd.build

Compiles csrc/*.hip and csrc/*.cpp with hipcc into
decode_attention_paged_02_amd/libpda.so.  Packed-FP32 instruction selection
is disabled for the device code; kernel-argument preloading is enabled.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpda.so")
ARCH = os.environ.get("PDA_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the first kernel arguments arrive in scalar registers at wave start
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source to an object in parallel, then link libpda.so."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        procs.append((src, subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True)))
        if len(procs) >= jobs:
            _wait(procs.pop(0))
    for p in procs:
        _wait(p)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


EXAMPLE_SRC = os.path.join(HERE, "examples", "c_abi_decode.cpp")
EXAMPLE_BIN = os.path.join(HERE, "examples", "c_abi_decode")
EXAMPLE_LIB = os.path.join(HERE, "examples", "libc_abi_decode.so")


def build_example(verbose: bool = False) -> str:
    """The C-ABI example (host code only, linked against libpda.so): the
    program, and the same code as a shared library for in-process tests."""
    common = [HIPCC, "-O2", "-std=c++17", "-Wall", "-I", os.path.join(ROOT, "include"),
              EXAMPLE_SRC, "-L", HERE, "-lpda", "-Wl,-rpath,$ORIGIN/.."]
    for out, extra in ((EXAMPLE_BIN, []),
                       (EXAMPLE_LIB, ["-shared", "-fPIC", "-DPDA_EXAMPLE_LIBRARY"])):
        cmd = common + extra + ["-o", out + ".tmp"]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        subprocess.run(cmd, check=True)
        os.replace(out + ".tmp", out)
    return EXAMPLE_BIN


def _wait(item):
    src, p = item
    _, err = p.communicate()
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (err or "").splitlines() if noise not in l]
    if msgs:
        print("\n".join(msgs), file=sys.stderr)
    if p.returncode != 0:
        raise RuntimeError("hipcc failed on %s" % src)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_example(verbose="-v" in sys.argv))
