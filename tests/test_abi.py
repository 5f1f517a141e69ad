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
                          "attn_quantize_fp8_hadamard", "attn_quantize_fp8_qkv", "attn_quantize_fp8_qkv_hadamard",
                          "attn_cast_bf16", "attn_strerror", "attn_abi_version"}
    L = ctypes.CDLL(build_mod.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert set(names) <= set(ops._SIGNATURES)


def test_version_and_strerror():
    L = ops.lib()
    assert L.attn_abi_version() == 2
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
    assert f(*args, 0.0, 1, 64, 2, 2, 128, 128, 1, 0, 0, None) == INVALID
    assert f(*args[:8], FAKE + 2, 0.1, 1, 64, 2, 2, 128, 128, 1, 0, 0, None) == INVALID


def test_fwd_ex_flags():
    f = ops.lib().attn_prefill_fwd_ex
    args = [FAKE, FAKE, FAKE, FAKE, None, 1.0, 1.0, 1.0, None, 0.1, 1, 64, 2, 2, 128, 128, 1]
    assert f(*args, 0, 1 << 9, None) == INVALID                             # unknown flag
    assert f(*args, 1, ops.ATTN_FLAG_P_BLOCK_SCALE, None) == UNSUPPORTED    # BF16 has no scaled MFMA
    assert f(*args[:4], FAKE + 2, *args[5:], 0, ops.ATTN_FLAG_P_BLOCK_SCALE, None) == INVALID  # misaligned lse
    # Lean P: O only (an lse pointer is invalid), not with block scaling, and switched off
    assert f(*args[:4], FAKE, *args[5:], 0, ops.ATTN_FLAG_LEAN_P, None) == INVALID
    assert f(*args, 0, ops.ATTN_FLAG_LEAN_P | ops.ATTN_FLAG_P_BLOCK_SCALE, None) == INVALID
    assert f(*args, 0, ops.ATTN_FLAG_LEAN_P, None) == UNSUPPORTED
    # the rounded-sum normalizer: FP8 only, only with block-scaled P, not with
    # Lean P (which has it built in)
    RSPS = ops.ATTN_FLAG_P_ROUNDED_SUM | ops.ATTN_FLAG_P_BLOCK_SCALE
    assert f(*args, 1, RSPS, None) == UNSUPPORTED
    assert f(*args, 0, ops.ATTN_FLAG_P_ROUNDED_SUM, None) == INVALID
    assert f(*args, 0, ops.ATTN_FLAG_LEAN_P | ops.ATTN_FLAG_P_ROUNDED_SUM, None) == INVALID
    assert f(*args[:4], FAKE + 2, *args[5:], 0, RSPS, None) == INVALID  # misaligned lse


def test_quantize_q_rejects_bad_arguments():
    L = ops.lib()
    f = L.attn_quantize_fp8_q
    assert f(FAKE, 0, FAKE, FAKE + 64, 16, None, 0.1, None) == INVALID        # no key scale
    assert f(FAKE, 0, FAKE, FAKE + 64, 16, FAKE + 128, 0.0, None) == INVALID  # softmax scale 0
    assert f(FAKE, 0, FAKE, FAKE + 64, 16, FAKE + 128, float("inf"), None) == INVALID
    assert f(FAKE, 0, FAKE, FAKE + 64, 16, FAKE + 66, 0.1, None) == INVALID   # misaligned key scale
    assert f(FAKE, 0, FAKE, FAKE + 64, 16, FAKE + 64, 0.1, None) == INVALID   # key scale aliases d_scale
    assert f(FAKE, 3, FAKE, FAKE + 64, 16, FAKE + 128, 0.1, None) == UNSUPPORTED


def test_quantize_and_cast_reject_bad_arguments():
    L = ops.lib()
    assert L.attn_quantize_fp8(None, 0, FAKE, FAKE, 16, None) == INVALID
    assert L.attn_quantize_fp8(FAKE, 0, FAKE, FAKE, 0, None) == INVALID
    assert L.attn_quantize_fp8(FAKE, 2, FAKE, FAKE + 1024, 16, None) == UNSUPPORTED
    assert L.attn_quantize_fp8(FAKE + 8, 0, FAKE, FAKE + 1024, 16, None) == INVALID
    assert L.attn_quantize_fp8(FAKE, 0, FAKE + 1024, FAKE + 8, 16, None) == INVALID  # scale aliases x
    assert L.attn_cast_bf16(None, FAKE, 8, None) == INVALID
    assert L.attn_cast_bf16(FAKE, FAKE, -5, None) == INVALID


def test_quantize_hadamard_rejects_bad_arguments():
    f = ops.lib().attn_quantize_fp8_hadamard
    # x: 256 fp32 at FAKE; codes at FAKE + 4096; scale at FAKE + 8192; key scale at FAKE + 8256
    x, x8, sc, ks = FAKE, FAKE + 4096, FAKE + 8192, FAKE + 8256
    assert f(x, 0, x8, sc, 288, 96, None, 0.0, None) == UNSUPPORTED     # 32-wide blocks
    assert f(x, 0, x8, sc, 256, 32, None, 0.0, None) == UNSUPPORTED
    assert f(x, 0, x8, sc, 256, 0, None, 0.0, None) == INVALID
    assert f(x, 0, x8, sc, 200, 128, None, 0.0, None) == INVALID        # n not a multiple of d
    assert f(x, 0, x8, sc, 0, 128, None, 0.0, None) == INVALID
    assert f(None, 0, x8, sc, 256, 128, None, 0.0, None) == INVALID
    assert f(x, 3, x8, sc, 256, 128, None, 0.0, None) == UNSUPPORTED
    assert f(x, 0, x8, x + 16, 256, 128, None, 0.0, None) == INVALID    # scale inside x
    assert f(x, 0, x8, sc, 384, 192, ks, 0.0, None) == INVALID          # query: softmax scale 0
    assert f(x, 0, x8, sc, 384, 192, sc, 0.1, None) == INVALID          # key scale aliases d_scale
    assert f(x, 0, x8, sc, 384, 192, ks + 2, 0.1, None) == INVALID      # misaligned key scale


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


def test_quantize_qkv_hadamard_rejects_bad_arguments():
    f = ops.lib().attn_quantize_fp8_qkv_hadamard
    q, k, v = FAKE, FAKE + 1024, FAKE + 2048
    q8, k8, v8, sc = FAKE + 4096, FAKE + 4352, FAKE + 4608, FAKE + 8192
    names = ["q", "k", "v", "xdt", "nq", "nk", "nv", "d", "q8", "k8", "v8", "sc", "sm", "st"]
    ok = (q, k, v, 0, 256, 256, 256, 128, q8, k8, v8, sc, 0.1, None)

    def call(**kw):
        a = list(ok)
        for key, val in kw.items():
            a[names.index(key)] = val
        return f(*a)
    assert call(q=None) == INVALID
    assert call(sc=sc + 2) == INVALID
    assert call(sm=0.0) == INVALID
    assert call(d=0) == INVALID
    assert call(d=96) == INVALID                # 256 is not a multiple of 96
    assert call(d=32) == UNSUPPORTED            # 32-column blocks
    assert call(nk=200) == INVALID              # k not whole rows
    assert call(xdt=2) == UNSUPPORTED


# ---------------------------------------------------------------- binding-side checks (no GPU)
# The Python binding checks every shape, dtype and element count before it
# passes pointers to the library, since the kernels trust the sizes they are
# given: a short k or an undersized out would be read or written out of
# bounds. Structure is checked before placement, so CPU tensors reach each of
# these errors without a device.

import torch  # noqa: E402

F8, BF, F32 = torch.uint8, torch.bfloat16, torch.float32


def _t(shape, dt=F8):
    return torch.empty(shape, dtype=dt)


@pytest.mark.parametrize("kw,msg", [
    (dict(k=_t((1, 63, 2, 128))), "k must have shape"),             # shorter k
    (dict(k=_t((1, 64, 2, 64))), "k must have shape"),              # k narrower than q's d_qk
    (dict(v=_t((1, 64, 4, 128))), "v must have shape"),             # v head count differs from k's
    (dict(v=_t((2, 64, 2, 128))), "v must have shape"),             # v batch differs
    (dict(q=_t((1, 64, 4, 128, 1))), "must be 4-D"),
    (dict(q=_t((1, 64, 3, 128)), ), "multiple of Hkv"),
    (dict(q=_t((1, 0, 4, 128)), k=_t((1, 0, 2, 128)), v=_t((1, 0, 2, 128))), "empty"),
    (dict(v=_t((1, 64, 2, 128), BF)), "share one dtype"),
    (dict(q=_t((1, 64, 4, 128), F32)), "codes or bfloat16"),
    (dict(out=_t((1, 64, 4, 64), BF)), "out must have shape"),      # undersized out
    (dict(out=_t((1, 64, 4, 128), F32)), "out must be of dtype"),   # wrong out dtype
    (dict(lse=_t((1, 64, 4), F32)), "lse must have shape"),         # lse in the wrong layout
    (dict(lse=_t((1, 4, 64), BF)), "lse must be of dtype"),
    (dict(d_scales=_t((2,), F32)), "d_scales must hold 3"),
    (dict(d_scales=_t((3,), BF)), "d_scales must be of dtype"),
    (dict(), "must be a device tensor"),                            # well formed, but on the host
])
def test_binding_rejects_mismatched_attention_args(kw, msg):
    a = dict(q=_t((1, 64, 4, 128)), k=_t((1, 64, 2, 128)), v=_t((1, 64, 2, 128)), out=None, lse=None,
             d_scales=None)
    a.update(kw)
    with pytest.raises(ValueError, match=msg):
        ops.check_attention_args(a["q"], a["k"], a["v"], a["out"], a["lse"], a["d_scales"])


def test_binding_accepts_mla_shapes_up_to_placement():
    # MLA (d_qk 192, d_v 128) is well formed: only the host placement fails
    q, k, v = _t((1, 16, 4, 192)), _t((1, 16, 4, 192)), _t((1, 16, 4, 128))
    with pytest.raises(ValueError, match="device tensor"):
        ops.check_attention_args(q, k, v, _t((1, 16, 4, 128), BF), _t((1, 4, 16), F32), _t((3,), F32))


@pytest.mark.parametrize("kw,msg", [
    (dict(out=_t((99,))), "out must hold 100"),
    (dict(out=_t((100,), F32)), "out must be of dtype"),
    (dict(scale=_t((2,), F32)), "scale must hold 1"),
    (dict(scale=_t((1,), BF)), "scale must be of dtype"),
    (dict(k_scale=_t((3,), F32), softmax_scale=0.1), "k_scale must hold 1"),
    (dict(k_scale=_t((1,), F32)), "needs softmax_scale"),
    (dict(x=_t((100,), torch.float16)), "float32 or bfloat16"),
    (dict(x=_t((0,), F32)), "empty"),
    (dict(), "must be a device tensor"),
])
def test_binding_rejects_mismatched_quantize_args(kw, msg):
    a = dict(x=_t((100,), F32), out=None, scale=None, k_scale=None, softmax_scale=None)
    a.update(kw)
    with pytest.raises(ValueError, match=msg):
        ops.check_quantize_args(a["x"], a["out"], a["scale"], a["k_scale"], a["softmax_scale"])


@pytest.mark.parametrize("kw,msg", [
    (dict(out=(_t((10,)), _t((20,)))), "three code tensors"),
    (dict(out=(_t((10,)), _t((20,)), _t((29,)))), "v8 must hold 30"),
    (dict(out=(_t((10,), BF), _t((20,)), _t((30,)))), "q8 must be of dtype"),
    (dict(scales=_t((1,), F32)), "scales must hold 3"),
    (dict(v=_t((30,), BF)), "must all be float32"),
    (dict(k=_t((0,), F32)), "k is empty"),
    (dict(), "must be a device tensor"),
])
def test_binding_rejects_mismatched_quantize_qkv_args(kw, msg):
    a = dict(q=_t((10,), F32), k=_t((20,), F32), v=_t((30,), F32), out=None, scales=None)
    a.update(kw)
    with pytest.raises(ValueError, match=msg):
        ops.check_quantize_qkv_args(a["q"], a["k"], a["v"], a["out"], a["scales"])


def test_binding_rejects_mismatched_cast_args():
    with pytest.raises(ValueError, match="out must hold 9"):
        ops.attn_cast_bf16(_t((9,), F32), out=_t((8,), BF))
    with pytest.raises(ValueError, match="out must be of dtype"):
        ops.attn_cast_bf16(_t((9,), F32), out=_t((9,), F32))
    with pytest.raises(ValueError, match="x must be float32"):
        ops.attn_cast_bf16(_t((9,), BF))
