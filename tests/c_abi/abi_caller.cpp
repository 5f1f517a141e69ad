// A plain C++ caller of libattn_prefill.so: HIP runtime calls and the C ABI
// of include/attn_prefill.h only (no torch, no Python). It runs the FP8 and
// the BF16 path on a case whose answer has a closed form and checks it:
//
//   Q = 0 makes every logit 0, so row i of the causal softmax weighs keys
//   0..i equally: O[i, h] = mean_{j <= i} V[j, h / G] (dequantized) and
//   LSE[h, i] = ln(i + 1).
//
// It also checks that an invalid call returns ATTN_ERR_INVALID and enqueues
// nothing. Exit status 0 and a line "c-abi caller: OK" on success.
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "attn_prefill.h"

#define HIP_OK(x)                                                                  \
  do {                                                                             \
    hipError_t e_ = (x);                                                           \
    if (e_ != hipSuccess) {                                                        \
      fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
      return 2;                                                                    \
    }                                                                              \
  } while (0)

#define ATTN_OK_(x)                                                                \
  do {                                                                             \
    int r_ = (x);                                                                  \
    if (r_ != ATTN_OK) {                                                           \
      fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, attn_strerror(r_)); \
      return 3;                                                                    \
    }                                                                              \
  } while (0)

static const int B = 1, S = 300, HQ = 4, HKV = 2, D = 128, G = HQ / HKV;

// OCP e4m3fn value of a code (finite codes only): bias 7, 3 mantissa bits.
static double e4m3fn_value(uint8_t c) {
  const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  const double mag = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
  return s ? -mag : mag;
}

static double bf16_value(uint16_t u) {
  uint32_t w = (uint32_t)u << 16;
  float f;
  memcpy(&f, &w, 4);
  return f;
}

// Standard normal draws from a 64-bit LCG and Box-Muller (seeded, host only).
struct Lcg {
  uint64_t s;
  double uniform() {
    s = s * 6364136223846793005ULL + 1442695040888963407ULL;
    return ((s >> 11) + 0.5) * (1.0 / 9007199254740992.0);
  }
  float normal() { return (float)(sqrt(-2.0 * log(uniform())) * cos(6.283185307179586 * uniform())); }
};

// Checks O and LSE against the running-mean closed form; vdeq[j][g][c].
static int check(const char* what, const std::vector<uint16_t>& o, const std::vector<float>& lse,
                 const std::vector<double>& vdeq) {
  double vmax = 0;
  for (double x : vdeq) vmax = fmax(vmax, fabs(x));
  std::vector<double> sum((size_t)HKV * D, 0.0);
  for (int i = 0; i < S; ++i) {
    for (int g = 0; g < HKV; ++g)
      for (int c = 0; c < D; ++c) sum[(size_t)g * D + c] += vdeq[((size_t)i * HKV + g) * D + c];
    for (int h = 0; h < HQ; ++h) {
      for (int c = 0; c < D; ++c) {
        const double want = sum[(size_t)(h / G) * D + c] / (i + 1);
        const double got = bf16_value(o[(((size_t)i) * HQ + h) * D + c]);
        // bf16 output rounding (2^-9 relative) plus fp32 accumulation
        if (fabs(got - want) > ldexp(fabs(want), -8) + 1e-5 * vmax) {
          fprintf(stderr, "%s: O[%d, %d, %d] = %.6g, running mean %.6g\n", what, i, h, c, got, want);
          return 1;
        }
      }
      const double l = lse[(size_t)h * S + i];
      if (fabs(l - log((double)(i + 1))) > 1e-5) {
        fprintf(stderr, "%s: LSE[%d, %d] = %.8g, ln(i+1) = %.8g\n", what, h, i, l, log((double)(i + 1)));
        return 1;
      }
    }
  }
  return 0;
}

int main() {
  const size_t nq = (size_t)B * S * HQ * D, nkv = (size_t)B * S * HKV * D;
  std::vector<float> hq(nq, 0.0f), hk(nkv), hv(nkv);
  Lcg rng{12345};
  for (auto& x : hk) x = rng.normal();
  for (auto& x : hv) x = rng.normal();

  hipStream_t st;
  HIP_OK(hipStreamCreate(&st));
  float *dq, *dk, *dv, *dscales, *dlse;
  uint8_t *q8, *k8, *v8;
  uint16_t *qb, *kb, *vb, *dout;
  HIP_OK(hipMalloc(&dq, nq * 4));
  HIP_OK(hipMalloc(&dk, nkv * 4));
  HIP_OK(hipMalloc(&dv, nkv * 4));
  HIP_OK(hipMalloc(&q8, nq));
  HIP_OK(hipMalloc(&k8, nkv));
  HIP_OK(hipMalloc(&v8, nkv));
  HIP_OK(hipMalloc(&qb, nq * 2));
  HIP_OK(hipMalloc(&kb, nkv * 2));
  HIP_OK(hipMalloc(&vb, nkv * 2));
  HIP_OK(hipMalloc(&dscales, 3 * 4));
  HIP_OK(hipMalloc(&dout, nq * 2));
  HIP_OK(hipMalloc(&dlse, (size_t)B * HQ * S * 4));
  HIP_OK(hipMemcpyAsync(dq, hq.data(), nq * 4, hipMemcpyHostToDevice, st));
  HIP_OK(hipMemcpyAsync(dk, hk.data(), nkv * 4, hipMemcpyHostToDevice, st));
  HIP_OK(hipMemcpyAsync(dv, hv.data(), nkv * 4, hipMemcpyHostToDevice, st));

  // an invalid call (Hq not a multiple of Hkv) is rejected on the host
  if (attn_prefill_fwd(q8, k8, v8, dout, dlse, 1.f, 1.f, 1.f, B, S, 3, 2, D, D, 1, ATTN_DTYPE_FP8_E4M3, st) !=
      ATTN_ERR_INVALID) {
    fprintf(stderr, "invalid head counts were not rejected\n");
    return 1;
  }

  std::vector<uint16_t> o(nq);
  std::vector<float> lse((size_t)B * HQ * S);
  std::vector<double> vdeq(nkv);
  const float sm = 1.0f / sqrtf((float)D);

  // ---- FP8: K and V quantized, then Q with the folded scale; scales stay on the device
  ATTN_OK_(attn_quantize_fp8(dk, 0, k8, dscales + 1, (int64_t)nkv, st));
  ATTN_OK_(attn_quantize_fp8(dv, 0, v8, dscales + 2, (int64_t)nkv, st));
  ATTN_OK_(attn_quantize_fp8_q(dq, 0, q8, dscales, (int64_t)nq, dscales + 1, sm, st));
  // (a flag outside the ABI, or a flag on the BF16 path, is rejected on the host)
  if (attn_prefill_fwd_ex(q8, k8, v8, dout, dlse, 1.f, 1.f, 1.f, dscales, sm, B, S, HQ, HKV, D, D, 1,
                          ATTN_DTYPE_FP8_E4M3, 1 << 20, st) != ATTN_ERR_INVALID ||
      attn_prefill_fwd_ex(qb, kb, vb, dout, dlse, 1.f, 1.f, 1.f, nullptr, sm, B, S, HQ, HKV, D, D, 1,
                          ATTN_DTYPE_BF16, ATTN_FLAG_P_BLOCK_SCALE, st) != ATTN_ERR_UNSUPPORTED) {
    fprintf(stderr, "bad flags were not rejected\n");
    return 1;
  }
  std::vector<uint8_t> hv8(nkv);
  float hs[3];
  // exact probabilities, the block-scaled form, and that with the rounded-sum
  // normalizer (for Q = 0 every p is 1, exact under any power-of-two
  // scaling, and the rounded row sum is exact)
  for (int flags : {0, (int)ATTN_FLAG_P_BLOCK_SCALE, (int)(ATTN_FLAG_P_ROUNDED_SUM | ATTN_FLAG_P_BLOCK_SCALE)}) {
    ATTN_OK_(attn_prefill_fwd_ex(q8, k8, v8, dout, dlse, 1.f, 1.f, 1.f, dscales, sm, B, S, HQ, HKV, D, D, 1,
                                 ATTN_DTYPE_FP8_E4M3, flags, st));
    HIP_OK(hipMemcpyAsync(hv8.data(), v8, nkv, hipMemcpyDeviceToHost, st));
    HIP_OK(hipMemcpyAsync(hs, dscales, 12, hipMemcpyDeviceToHost, st));
    HIP_OK(hipMemcpyAsync(o.data(), dout, nq * 2, hipMemcpyDeviceToHost, st));
    HIP_OK(hipMemcpyAsync(lse.data(), dlse, lse.size() * 4, hipMemcpyDeviceToHost, st));
    HIP_OK(hipStreamSynchronize(st));
    for (size_t i = 0; i < nkv; ++i) vdeq[i] = e4m3fn_value(hv8[i]) * hs[2];
    const char* what = flags == 0                              ? "fp8"
                       : flags == (int)ATTN_FLAG_P_BLOCK_SCALE ? "fp8 block-scaled P"
                                                               : "fp8 block-scaled P, rounded-sum normalizer";
    if (check(what, o, lse, vdeq)) return 1;
  }

  // ---- BF16: RNE casts, then the same closed form
  ATTN_OK_(attn_cast_bf16(dq, qb, (int64_t)nq, st));
  ATTN_OK_(attn_cast_bf16(dk, kb, (int64_t)nkv, st));
  ATTN_OK_(attn_cast_bf16(dv, vb, (int64_t)nkv, st));
  ATTN_OK_(attn_prefill_fwd(qb, kb, vb, dout, dlse, 1.f, 1.f, 1.f, B, S, HQ, HKV, D, D, 1, ATTN_DTYPE_BF16, st));
  std::vector<uint16_t> hvb(nkv);
  HIP_OK(hipMemcpyAsync(hvb.data(), vb, nkv * 2, hipMemcpyDeviceToHost, st));
  HIP_OK(hipMemcpyAsync(o.data(), dout, nq * 2, hipMemcpyDeviceToHost, st));
  HIP_OK(hipMemcpyAsync(lse.data(), dlse, lse.size() * 4, hipMemcpyDeviceToHost, st));
  HIP_OK(hipStreamSynchronize(st));
  for (size_t i = 0; i < nkv; ++i) vdeq[i] = bf16_value(hvb[i]);
  if (check("bf16", o, lse, vdeq)) return 1;

  for (void* p : {(void*)dq, (void*)dk, (void*)dv, (void*)q8, (void*)k8, (void*)v8, (void*)qb, (void*)kb,
                  (void*)vb, (void*)dscales, (void*)dout, (void*)dlse})
    HIP_OK(hipFree(p));
  HIP_OK(hipStreamDestroy(st));
  printf("c-abi caller: OK (FP8 and BF16, B=%d S=%d Hq=%d Hkv=%d d=%d, q_scale %.6g k_scale %.6g v_scale %.6g)\n",
         B, S, HQ, HKV, D, hs[0], hs[1], hs[2]);
  return 0;
}
