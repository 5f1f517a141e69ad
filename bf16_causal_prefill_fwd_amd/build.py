"""Build libattn_prefill.so in-tree with hipcc for gfx950.

Usage: ``python -m bf16_causal_prefill_fwd_amd.build`` (or ``build()``).
The library lands next to this file; the ctypes binding loads it from there.
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
LIB_NAME = "libattn_prefill.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["api.hip", "quantize.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed-FP32 VALU instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libattn_prefill.so)")


def build(verbose: bool = False, extra_flags: list[str] | None = None, out: str | None = None) -> str:
    """Compile every HIP source into the shared library; returns its path."""
    out = out or LIB_PATH
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building %s" % LIB_NAME)
    os.replace(tmp, out)
    return out


C_CALLER_SRC = os.path.join(ROOT, "tests", "c_abi", "abi_caller.cpp")
C_CALLER = os.path.join(ROOT, "tests", "c_abi", "abi_caller")


def build_c_caller(verbose: bool = False) -> str:
    """Compile the plain C++ ABI caller used by the tests (host code only),
    linked against the in-tree library; returns its path."""
    tmp = C_CALLER + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-O2", "-std=c++17", "-Wno-unused-command-line-argument", "-I", INCLUDE, C_CALLER_SRC,
           "-L", PKG, "-lattn_prefill", "-Wl,-rpath,$ORIGIN/../../bf16_causal_prefill_fwd_amd", "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building the ABI caller")
    os.replace(tmp, C_CALLER)
    return C_CALLER


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_c_caller(verbose=True))
