"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function include/attn_prefill.h
declares, and reject bad arguments with ATTN_ERR_INVALID / _UNSUPPORTED
before any HIP call is made (all calls here use arguments that fail the
host checks, so nothing reaches a device).
"""

import ctypes
import os

import pytest

from bf16_causal_prefill_fwd_amd import build as build_mod
from bf16_causal_prefill_fwd_amd import ops

pytestmark = pytest.mark.skipif(not os.path.exists(build_mod.LIB_PATH), reason="library not built")

INVALID, UNSUPPORTED = -1, -2
FAKE = 0x10000  # a 16-byte-aligned non-null address; never dereferenced by host checks


def test_exports_every_header_function():
    names = ops.header_functions()
    assert set(names) == {"attn_prefill_fwd", "attn_prefill_fwd_ex", "attn_quantize_fp8", "attn_quantize_fp8_q",
                          "attn_quantize_fp8_hadamard", "attn_quantize_fp8_qkv", "attn_cast_bf16", "attn_strerror",
                          "attn_abi_version"}
    L = ctypes.CDLL(build_mod.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert set(names) <= set(ops._SIGNATURES)


def test_version_and_strerror():
    L = ops.lib()
    assert L.attn_abi_version() == 1
    assert ops.strerror(0) == "success"
    assert "invalid" in ops.strerror(INVALID)
    assert "gfx950" in ops.strerror(UNSUPPORTED)


def _fwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, qs=1.0, ks=1.0, vs=1.0, B=1, S=64, Hq=4, Hkv=2,
             dqk=128, dv=128, causal=1, dtype=0)
    a.update(kw)
    return ops.lib().attn_prefill_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["qs"], a["ks"], a["vs"],
                                      a["B"], a["S"], a["Hq"], a["Hkv"], a["dqk"], a["dv"], a["causal"],
                                      a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID),
    (dict(o=None), INVALID),
    (dict(B=0), INVALID),
    (dict(S=-1), INVALID),
    (dict(Hq=6, Hkv=4), INVALID),
    (dict(causal=2), INVALID),
    (dict(qs=0.0), INVALID),
    (dict(vs=float("nan")), INVALID),
    (dict(q=FAKE + 4), INVALID),
    (dict(S=(1 << 24) + 1), INVALID),
    (dict(Hq=1 << 17, Hkv=1 << 17), INVALID),  # a 64-row K tile would span >= 2^31 bytes
    (dict(dtype=7), UNSUPPORTED),
    (dict(dqk=64, dv=64), UNSUPPORTED),
    (dict(dqk=192, dv=192), UNSUPPORTED),
])
def test_fwd_rejects_bad_arguments(kw, code):
    assert _fwd(**kw) == code


def test_fwd_ex_rejects_bad_softmax_scale_and_scale_pointer():
    L = ops.lib()
    f = L.attn_prefill_fwd_ex
    args = [FAKE, FAKE, FAKE, FAKE, None, 1.0, 1.0, 1.0, None]
    assert f(*args, 0.0, 1, 64, 2, 2, 128, 128, 1, 0, None) == INVALID
    assert f(*args[:8], FAKE + 2, 0.1, 1, 64, 2, 2, 128, 128, 1, 0, None) == INVALID


def test_quantize_q_rejects_bad_arguments():
    L = ops.lib()
    f = L.attn_quantize_fp8_q
    assert f(FAKE, 0, 16, FAKE, FAKE + 64, None, 0.1, None) == INVALID        # no key scale
    assert f(FAKE, 0, 16, FAKE, FAKE + 64, FAKE + 128, 0.0, None) == INVALID  # softmax scale 0
    assert f(FAKE, 0, 16, FAKE, FAKE + 64, FAKE + 128, float("inf"), None) == INVALID
    assert f(FAKE, 0, 16, FAKE, FAKE + 64, FAKE + 66, 0.1, None) == INVALID   # misaligned key scale
    assert f(FAKE, 0, 16, FAKE, FAKE + 64, FAKE + 64, 0.1, None) == INVALID   # key scale aliases d_scale
    assert f(FAKE, 3, 16, FAKE, FAKE + 64, FAKE + 128, 0.1, None) == UNSUPPORTED


def test_quantize_and_cast_reject_bad_arguments():
    L = ops.lib()
    assert L.attn_quantize_fp8(None, 0, 16, FAKE, FAKE, None) == INVALID
    assert L.attn_quantize_fp8(FAKE, 0, 0, FAKE, FAKE, None) == INVALID
    assert L.attn_quantize_fp8(FAKE, 2, 16, FAKE, FAKE + 1024, None) == UNSUPPORTED
    assert L.attn_quantize_fp8(FAKE + 8, 0, 16, FAKE, FAKE + 1024, None) == INVALID
    assert L.attn_quantize_fp8(FAKE, 0, 16, FAKE + 1024, FAKE + 8, None) == INVALID  # scale aliases x
    assert L.attn_cast_bf16(None, 8, FAKE, None) == INVALID
    assert L.attn_cast_bf16(FAKE, -5, FAKE, None) == INVALID


def test_quantize_hadamard_rejects_bad_arguments():
    f = ops.lib().attn_quantize_fp8_hadamard
    # x: 256 fp32 at FAKE; codes at FAKE + 4096; scale at FAKE + 8192; key scale at FAKE + 8256
    x, x8, sc, ks = FAKE, FAKE + 4096, FAKE + 8192, FAKE + 8256
    assert f(x, 0, 288, 96, x8, sc, None, 0.0, None) == UNSUPPORTED     # 32-wide blocks
    assert f(x, 0, 256, 32, x8, sc, None, 0.0, None) == UNSUPPORTED
    assert f(x, 0, 256, 0, x8, sc, None, 0.0, None) == INVALID
    assert f(x, 0, 200, 128, x8, sc, None, 0.0, None) == INVALID        # n not a multiple of d
    assert f(x, 0, 0, 128, x8, sc, None, 0.0, None) == INVALID
    assert f(None, 0, 256, 128, x8, sc, None, 0.0, None) == INVALID
    assert f(x, 3, 256, 128, x8, sc, None, 0.0, None) == UNSUPPORTED
    assert f(x, 0, 256, 128, x8, x + 16, None, 0.0, None) == INVALID    # scale inside x
    assert f(x, 0, 384, 192, x8, sc, ks, 0.0, None) == INVALID          # query: softmax scale 0
    assert f(x, 0, 384, 192, x8, sc, sc, 0.1, None) == INVALID          # key scale aliases d_scale
    assert f(x, 0, 384, 192, x8, sc, ks + 2, 0.1, None) == INVALID      # misaligned key scale


def test_quantize_qkv_rejects_bad_arguments():
    f = ops.lib().attn_quantize_fp8_qkv
    # q, k, v: 256 fp32 each; codes after them; scales (3 floats) at sc
    q, k, v = FAKE, FAKE + 1024, FAKE + 2048
    q8, k8, v8, sc = FAKE + 4096, FAKE + 4352, FAKE + 4608, FAKE + 8192
    ok = (q, k, v, 0, 256, 256, 256, q8, k8, v8, sc, 0.1, None)

    def call(**kw):
        a = list(ok)
        names = ["q", "k", "v", "xdt", "nq", "nk", "nv", "q8", "k8", "v8", "sc", "sm", "st"]
        for key, val in kw.items():
            a[names.index(key)] = val
        return f(*a)
    assert call(q=None) == INVALID
    assert call(v8=None) == INVALID
    assert call(sc=None) == INVALID
    assert call(nk=0) == INVALID
    assert call(nv=1 << 40) == INVALID
    assert call(sm=0.0) == INVALID
    assert call(sm=float("nan")) == INVALID
    assert call(xdt=2) == UNSUPPORTED
    assert call(k=k + 8) == INVALID            # misaligned input
    assert call(q8=q8 + 4) == INVALID          # misaligned codes
    assert call(sc=sc + 2) == INVALID          # misaligned scales
    assert call(sc=v + 1020) == INVALID        # scales overlap the end of v
    assert call(sc=k8 + 16) == INVALID         # scales inside k's codes
