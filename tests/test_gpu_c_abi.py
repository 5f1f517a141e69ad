"""The C ABI from a plain C++ caller (tests/c_abi/abi_caller.cpp): HIP
runtime calls and include/attn_prefill.h only, no torch and no Python
binding. It runs the FP8 and BF16 paths on Q = 0, where O is the running
mean of the dequantized V prefix and LSE = ln(i+1), and checks an invalid
call is rejected. Built by __graft_entry__.build()."""

import os
import subprocess

import pytest

from bf16_causal_prefill_fwd_amd.build import C_CALLER

pytestmark = pytest.mark.gpu


def test_plain_cpp_caller():
    assert os.path.exists(C_CALLER), f"{C_CALLER} is not built: run __graft_entry__.build()"
    print("case c-abi caller (FP8 and BF16, Q = 0 closed form)", flush=True)
    r = subprocess.run([C_CALLER], capture_output=True, text=True, timeout=120)
    print(r.stdout + r.stderr, flush=True)
    assert r.returncode == 0 and "c-abi caller: OK" in r.stdout
