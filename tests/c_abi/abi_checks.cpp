// Host-side argument checks of every entry point of include/attn_prefill.h,
// from plain C++ with no GPU: each call carries an argument that the host
// checks reject, so it returns before any HIP call and nothing is enqueued.
// The CPU tests build the library and this program with AddressSanitizer on
// the host code and run it, so the validation code is exercised under the
// sanitizer. Exit status 0 and a line "abi checks: OK" on success.
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "attn_prefill.h"

static int failures = 0;

#define EXPECT(call, code)                                                                       \
  do {                                                                                           \
    const int r_ = (call);                                                                       \
    if (r_ != (code)) {                                                                          \
      fprintf(stderr, "%s:%d %s returned %d, expected %d\n", __FILE__, __LINE__, #call, r_, (code)); \
      ++failures;                                                                                \
    }                                                                                            \
  } while (0)

// 16-byte-aligned non-null addresses that the host checks never dereference
static void* fake(uintptr_t off = 0) { return (void*)(uintptr_t)(0x10000 + off); }
static float* fakef(uintptr_t off = 0) { return (float*)fake(off); }
static uint8_t* fake8(uintptr_t off = 0) { return (uint8_t*)fake(off); }

static int fwd(const void* q, void* o, float* lse, float qs, int B, int S, int Hq, int Hkv, int dqk, int dv,
               int causal, int dtype) {
  return attn_prefill_fwd(q, fake(), fake(), o, lse, qs, 1.f, 1.f, B, S, Hq, Hkv, dqk, dv, causal, dtype, 0);
}

static int fwd_ex(float* lse, const float* d_scales, float sm, int dtype, int flags) {
  return attn_prefill_fwd_ex(fake(), fake(), fake(), fake(), lse, 1.f, 1.f, 1.f, d_scales, sm, 1, 64, 2, 2, 128,
                             128, 1, dtype, flags, 0);
}

int main() {
  const int INVALID = ATTN_ERR_INVALID, UNSUPPORTED = ATTN_ERR_UNSUPPORTED;

  // attn_prefill_fwd
  EXPECT(fwd(nullptr, fake(), fakef(), 1.f, 1, 64, 4, 2, 128, 128, 1, 0), INVALID);
  EXPECT(fwd(fake(), nullptr, fakef(), 1.f, 1, 64, 4, 2, 128, 128, 1, 0), INVALID);
  EXPECT(fwd(fake(), fake(), fakef(), 1.f, 0, 64, 4, 2, 128, 128, 1, 0), INVALID);
  EXPECT(fwd(fake(), fake(), fakef(), 1.f, 1, -1, 4, 2, 128, 128, 1, 0), INVALID);
  EXPECT(fwd(fake(), fake(), fakef(), 1.f, 1, 64, 6, 4, 128, 128, 1, 0), INVALID);
  EXPECT(fwd(fake(), fake(), fakef(), 1.f, 1, 64, 4, 2, 128, 128, 2, 0), INVALID);
  EXPECT(fwd(fake(), fake(), fakef(), 0.f, 1, 64, 4, 2, 128, 128, 1, 0), INVALID);
  EXPECT(fwd(fake(), fake(), fakef(), NAN, 1, 64, 4, 2, 128, 128, 1, 0), INVALID);
  EXPECT(fwd(fake(), fake(), fakef(), INFINITY, 1, 64, 4, 2, 128, 128, 1, 0), INVALID);
  EXPECT(fwd(fake(4), fake(), fakef(), 1.f, 1, 64, 4, 2, 128, 128, 1, 0), INVALID);
  EXPECT(fwd(fake(), fake(), fakef(2), 1.f, 1, 64, 4, 2, 128, 128, 1, 0), INVALID);
  EXPECT(fwd(fake(), fake(), fakef(), 1.f, 1, (1 << 24) + 1, 4, 2, 128, 128, 1, 0), INVALID);
  EXPECT(fwd(fake(), fake(), fakef(), 1.f, 1, 64, 1 << 17, 1 << 17, 128, 128, 1, 0), INVALID);
  EXPECT(fwd(fake(), fake(), fakef(), 1.f, INT_MAX, INT_MAX, INT_MAX, 1, 128, 128, 1, 0), INVALID);
  EXPECT(fwd(fake(), fake(), fakef(), 1.f, 1, 64, 4, 2, 128, 128, 1, 7), UNSUPPORTED);
  EXPECT(fwd(fake(), fake(), fakef(), 1.f, 1, 64, 4, 2, 64, 64, 1, 0), UNSUPPORTED);
  EXPECT(fwd(fake(), fake(), fakef(), 1.f, 1, 64, 4, 2, 192, 192, 1, 0), UNSUPPORTED);

  // attn_prefill_fwd_ex: softmax scale, scale pointer, flags
  EXPECT(fwd_ex(nullptr, nullptr, 0.f, 0, 0), INVALID);
  EXPECT(fwd_ex(nullptr, nullptr, -INFINITY, 0, 0), INVALID);
  EXPECT(fwd_ex(nullptr, fakef(2), 0.1f, 0, 0), INVALID);
  EXPECT(fwd_ex(nullptr, nullptr, 0.1f, 0, 1 << 9), INVALID);
  EXPECT(fwd_ex(nullptr, nullptr, 0.1f, 1, ATTN_FLAG_P_BLOCK_SCALE), UNSUPPORTED);
  EXPECT(fwd_ex(fakef(2), nullptr, 0.1f, 0, ATTN_FLAG_P_BLOCK_SCALE), INVALID);
  EXPECT(fwd_ex(fakef(), nullptr, 0.1f, 0, ATTN_FLAG_LEAN_P), INVALID);
  EXPECT(fwd_ex(nullptr, nullptr, 0.1f, 0, ATTN_FLAG_LEAN_P | ATTN_FLAG_P_BLOCK_SCALE), INVALID);
  EXPECT(fwd_ex(nullptr, nullptr, 0.1f, 0, ATTN_FLAG_LEAN_P), UNSUPPORTED);
  EXPECT(fwd_ex(nullptr, nullptr, 0.1f, 0, ATTN_FLAG_P_ROUNDED_SUM), INVALID);
  EXPECT(fwd_ex(nullptr, nullptr, 0.1f, 0, ATTN_FLAG_LEAN_P | ATTN_FLAG_P_ROUNDED_SUM), INVALID);
  EXPECT(fwd_ex(nullptr, nullptr, 0.1f, 1, ATTN_FLAG_P_ROUNDED_SUM | ATTN_FLAG_P_BLOCK_SCALE), UNSUPPORTED);

  // quantizers and the cast: inputs of 256 fp32 at +0 / +1024 / +2048, codes
  // at +4096 / +4352 / +4608, scales at +8192, a key scale at +8256
  void *x = fake(), *k = fake(1024), *v = fake(2048);
  uint8_t *x8 = fake8(4096), *k8 = fake8(4352), *v8 = fake8(4608);
  float *sc = fakef(8192), *ks = fakef(8256);
  EXPECT(attn_quantize_fp8(nullptr, 0, x8, sc, 256, 0), INVALID);
  EXPECT(attn_quantize_fp8(x, 0, nullptr, sc, 256, 0), INVALID);
  EXPECT(attn_quantize_fp8(x, 0, x8, nullptr, 256, 0), INVALID);
  EXPECT(attn_quantize_fp8(x, 0, x8, sc, 0, 0), INVALID);
  EXPECT(attn_quantize_fp8(x, 0, x8, sc, (int64_t)1 << 40, 0), INVALID);
  EXPECT(attn_quantize_fp8(x, 2, x8, sc, 256, 0), UNSUPPORTED);
  EXPECT(attn_quantize_fp8(fake(8), 0, x8, sc, 256, 0), INVALID);         // misaligned input
  EXPECT(attn_quantize_fp8(x, 0, x8, (float*)fake(16), 256, 0), INVALID);  // scale inside x
  EXPECT(attn_quantize_fp8_q(x, 0, x8, sc, 256, nullptr, 0.1f, 0), INVALID);
  EXPECT(attn_quantize_fp8_q(x, 0, x8, sc, 256, ks, 0.f, 0), INVALID);
  EXPECT(attn_quantize_fp8_q(x, 0, x8, sc, 256, ks, INFINITY, 0), INVALID);
  EXPECT(attn_quantize_fp8_q(x, 0, x8, sc, 256, (float*)fake(8258), 0.1f, 0), INVALID);
  EXPECT(attn_quantize_fp8_q(x, 0, x8, sc, 256, sc, 0.1f, 0), INVALID);
  EXPECT(attn_quantize_fp8_q(x, 3, x8, sc, 256, ks, 0.1f, 0), UNSUPPORTED);
  EXPECT(attn_quantize_fp8_qkv(nullptr, k, v, 0, 256, 256, 256, x8, k8, v8, sc, 0.1f, 0), INVALID);
  EXPECT(attn_quantize_fp8_qkv(x, k, v, 0, 256, 0, 256, x8, k8, v8, sc, 0.1f, 0), INVALID);
  EXPECT(attn_quantize_fp8_qkv(x, k, v, 0, 256, 256, (int64_t)1 << 40, x8, k8, v8, sc, 0.1f, 0), INVALID);
  EXPECT(attn_quantize_fp8_qkv(x, k, v, 0, 256, 256, 256, x8, k8, v8, sc, NAN, 0), INVALID);
  EXPECT(attn_quantize_fp8_qkv(x, k, v, 0, 256, 256, 256, x8, k8, v8, (float*)fake(8194), 0.1f, 0), INVALID);
  EXPECT(attn_quantize_fp8_qkv(x, k, v, 0, 256, 256, 256, x8, k8, v8, (float*)fake(3068), 0.1f, 0), INVALID);
  EXPECT(attn_quantize_fp8_qkv(x, k, v, 2, 256, 256, 256, x8, k8, v8, sc, 0.1f, 0), UNSUPPORTED);
  EXPECT(attn_quantize_fp8_hadamard(x, 0, x8, sc, 256, 0, nullptr, 0.f, 0), INVALID);
  EXPECT(attn_quantize_fp8_hadamard(x, 0, x8, sc, 200, 128, nullptr, 0.f, 0), INVALID);
  EXPECT(attn_quantize_fp8_hadamard(x, 0, x8, sc, 288, 96, nullptr, 0.f, 0), UNSUPPORTED);
  EXPECT(attn_quantize_fp8_hadamard(x, 0, x8, sc, 384, 192, ks, 0.f, 0), INVALID);
  EXPECT(attn_quantize_fp8_hadamard(x, 0, x8, sc, 384, 192, sc, 0.1f, 0), INVALID);
  EXPECT(attn_quantize_fp8_qkv_hadamard(x, k, v, 0, 256, 256, 256, 96, x8, k8, v8, sc, 0.1f, 0), INVALID);
  EXPECT(attn_quantize_fp8_qkv_hadamard(x, k, v, 0, 256, 256, 256, 32, x8, k8, v8, sc, 0.1f, 0), UNSUPPORTED);
  EXPECT(attn_quantize_fp8_qkv_hadamard(x, k, v, 0, 256, 256, 256, 128, x8, k8, v8, sc, 0.f, 0), INVALID);
  EXPECT(attn_cast_bf16(nullptr, (uint16_t*)x8, 8, 0), INVALID);
  EXPECT(attn_cast_bf16((const float*)x, (uint16_t*)x8, -5, 0), INVALID);
  EXPECT(attn_cast_bf16((const float*)x, (uint16_t*)fake(4098), 8, 0), INVALID);

  // every code has a text, unknown codes included
  const int codes[] = {ATTN_OK, INVALID, UNSUPPORTED, ATTN_ERR_HIP, 7, -100, INT_MIN, INT_MAX};
  for (int c : codes) {
    const char* s = attn_strerror(c);
    if (!s || !s[0]) {
      fprintf(stderr, "attn_strerror(%d) is empty\n", c);
      ++failures;
    }
  }
  if (attn_abi_version() != 2) {
    fprintf(stderr, "attn_abi_version() = %d\n", attn_abi_version());
    ++failures;
  }
  if (failures) {
    fprintf(stderr, "abi checks: %d failures\n", failures);
    return 1;
  }
  printf("abi checks: OK\n");
  return 0;
}
