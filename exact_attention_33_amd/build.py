"""Build the HIP library ``lib/libfa_mi355x.so`` for gfx950 with hipcc.

Usage: ``python -m exact_attention_33_amd.build`` (or ``build()`` from Python).
Every call recompiles every source: it is the "does it build" check as well
as the build.  Objects go to ``_build/`` at the repository root.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libfa_mi355x.so")
OBJDIR = os.path.join(ROOT, "_build")

SOURCES = ["shim.cpp", "plan.cpp", "prefill_bf16.hip", "mask_prep.hip", "fwd_f32.hip", "decode_bf16.hip",
           "bwd_bf16.hip", "kvouter_bf16.hip",
           "prefill_fp8.hip", "noalloc.hip"]

ARCH = "gfx950"
# Packed fp32 instructions are switched off for device code (the host pass
# warns that it does not know the feature; that warning is harmless).
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-command-line-argument"]


def hipcc():
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # drop the host pass's notice about the device-only feature flag
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose=False, jobs=8):
    """Compile all sources and link the shared library; returns its path."""
    os.makedirs(OBJDIR, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"]
        out = _run([hipcc(), *lang, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and out.strip():
            print(out)
        return obj

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
