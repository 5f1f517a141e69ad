"""The C ABI's host-side argument checks under AddressSanitizer (no GPU).

The library is built from the same sources with AddressSanitizer on its host
code only (the device code is built as usual and never launched here), and a
plain C++ program, tests/c_abi/abi_checks.cpp, calls every entry point with
arguments that the host checks reject. Each call must return its error code
before any HIP call, and the sanitizer must report nothing. The build takes
about a minute and is kept under _build/asan/ keyed by a hash of its inputs,
so later runs reuse it.
"""

import hashlib
import os
import shutil
import subprocess

import pytest

from bf16_causal_prefill_fwd_amd import build as build_mod

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bf16_causal_prefill_fwd_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
CHECKS_SRC = os.path.join(ROOT, "tests", "c_abi", "abi_checks.cpp")
FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17"]


def _inputs_hash() -> str:
    h = hashlib.sha256(" ".join(FLAGS).encode())
    files = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".h", ".hip")))
    for p in files + [os.path.join(INCLUDE, "attn_prefill.h"), CHECKS_SRC]:
        with open(p, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _run(cmd, cwd):
    res = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, timeout=900)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed: {' '.join(cmd)}\n{res.stdout}{res.stderr}")


@pytest.fixture(scope="module")
def asan_program() -> str:
    try:
        hipcc = build_mod.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not found")
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "llvm", "bin", "amdclang++")
    if not os.path.exists(clang):
        clang = shutil.which("amdclang++") or ""
    if not (os.path.exists(hipcc) and clang and os.path.exists(clang)):
        pytest.skip("hipcc / amdclang++ not found")
    out = os.path.join(ROOT, "_build", "asan", _inputs_hash())
    exe = os.path.join(out, "abi_checks")
    if os.path.exists(exe):
        return exe
    tmp = out + ".tmp%d" % os.getpid()
    os.makedirs(tmp, exist_ok=True)
    lib = os.path.join(tmp, "libattn_prefill.so")
    srcs = [os.path.join(CSRC, "api.hip"), os.path.join(CSRC, "quantize.hip")]
    # the sanitizer on the host pass only
    _run([hipcc, "--offload-arch=gfx950", *FLAGS, "-fPIC", "-shared", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-Wno-unused-command-line-argument", "-w",
          "-Xarch_host", "-fsanitize=address",
          "-I", INCLUDE, "-I", CSRC, *srcs, "-o", lib], tmp)
    # the caller: host C++ only, no HIP source
    rocm = os.path.realpath(os.path.join(os.path.dirname(os.path.realpath(hipcc)), ".."))
    _run([clang, *FLAGS, "-fsanitize=address", "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE,
          "-I", os.path.join(rocm, "include"), CHECKS_SRC, "-L", tmp, "-lattn_prefill", "-Wl,-rpath,$ORIGIN",
          "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(rocm, "lib"),
          "-o", os.path.join(tmp, "abi_checks")], tmp)
    if os.path.exists(out):
        shutil.rmtree(out)
    os.replace(tmp, out)
    return exe


def test_abi_host_checks_under_address_sanitizer(asan_program):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0")
    res = subprocess.run([asan_program], env=env, capture_output=True, text=True, timeout=300)
    assert "AddressSanitizer" not in res.stderr, res.stderr
    assert res.returncode == 0, res.stdout + res.stderr
    assert "abi checks: OK" in res.stdout
