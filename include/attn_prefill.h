/*
 * attn_prefill.h -- C ABI of libattn_prefill.so: causal prefill attention
 * forward for AMD Instinct MI355X (gfx950), FP8 e4m3 and BF16.
 *
 * What is computed: the causal forward (prefill) attention pass the ZYFA
 * pages describe -- tiled Q.K^T, a row softmax with running max and row sum,
 * then P.V -- in FP8 e4m3 and BF16, for head dim 128 with grouped-query heads
 * and for the MLA shape (Q.K dim 192, V dim 128). Sources: Le Fil IA (ZYFA:
 * FlashAttention en FP8 pour l'AMD MI355X), summary paragraph; aicronaca.it,
 * section "Che cosa ha annunciato Zyphra"; ai4bro.com, section "TL;DR".
 *
 *   s[i,j]   = softmax_scale * q_scale * k_scale * dot(q[b,i,h,:], k[b,j,g,:]),
 *              g = h / (Hq/Hkv), visible iff j <= i (causal) or always;
 *   o[b,i,h] = v_scale * sum_j softmax_j(s[i,:]) * v[b,j,g,:]       (bf16)
 *   lse[b,h,i] = ln sum_j exp(s[i,j])                                (fp32)
 *
 * with softmax_scale = 1/sqrt(d_qk) in attn_prefill_fwd.
 *
 * Conventions shared by every entry point:
 *  - Layouts are those of flash_attn_func (the pages present the library as
 *    a drop-in for it), contiguous, row-major:
 *      q [B, S, Hq,  d_qk]   k [B, S, Hkv, d_qk]   v [B, S, Hkv, d_v]
 *      o [B, S, Hq,  d_v]  bfloat16          lse [B, Hq, S]  float32
 *  - FP8 is OCP e4m3fn (1 byte, bias 7, max 448, no infinities). A value is
 *    code * scale with one float scale per tensor.
 *  - Every pointer argument except `stream` is DEVICE memory owned by the
 *    caller. The library allocates nothing, keeps no pointer after return,
 *    and does not synchronise: work is enqueued on `stream` (0 = the null
 *    stream) and the call returns.
 *  - Return value: 0 on success, or a negative ATTN_ERR_* code. Argument
 *    checks run on the host before anything is enqueued; a failed check
 *    enqueues nothing. ATTN_ERR_HIP reports a launch failure
 *    (hipGetLastError after the launch).
 *  - Runs are deterministic: each output element has one fixed reduction
 *    order, and the only atomics are the quantizers' integer maxima of
 *    absmax bits, whose result does not depend on their order, so repeated
 *    launches are bit-identical.
 */
#ifndef ATTN_PREFILL_H
#define ATTN_PREFILL_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID = -1,      /* null pointer, non-positive size, Hq % Hkv != 0, causal not 0/1 */
  ATTN_ERR_UNSUPPORTED = -2,  /* dtype or (d_qk, d_v) not built, device is not gfx950 */
  ATTN_ERR_HIP = -3,          /* a HIP call or kernel launch failed */
};

enum {
  ATTN_DTYPE_FP8_E4M3 = 0,    /* q, k, v are uint8 e4m3fn codes */
  ATTN_DTYPE_BF16 = 1,        /* q, k, v are bfloat16 */
};

/*
 * Causal (or full) prefill attention forward.
 *   q, k, v     device inputs in the layouts above, element type per `dtype`.
 *   o           device output, bfloat16 [B, S, Hq, d_v].
 *   lse         device output float32 [B, Hq, S], natural log, including the
 *               softmax and dequantization scales; NULL skips it.
 *   q_scale, k_scale, v_scale
 *               per-tensor dequantization scales (value = code * scale);
 *               pass 1.0 for BF16. Must be finite and > 0.
 *   B, S, Hq, Hkv  batch, sequence length (queries = keys), query heads,
 *               key/value heads; Hq must be a multiple of Hkv (grouped-query
 *               attention, query head h reads kv head h / (Hq/Hkv)).
 *   d_qk, d_v   head dims; supported: (128, 128) and (192, 128).
 *   causal      1: key j visible to query i iff j <= i; 0: all keys visible.
 *   dtype       ATTN_DTYPE_FP8_E4M3 or ATTN_DTYPE_BF16.
 * Limits: B*S*Hq*max(d_qk,d_v) < 2^40 elements; S <= 2^24;
 *         Hkv*max(d_qk,d_v) < 2^24.
 */
int attn_prefill_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     float q_scale, float k_scale, float v_scale,
                     int B, int S, int Hq, int Hkv, int d_qk, int d_v,
                     int causal, int dtype, hipStream_t stream);

enum {
  /*
   * FP8 only: per (query row, 64-key block) power-of-two scaling of P. Each
   * block's probabilities are rounded to e4m3 as p * 2^k (k >= 0, one k per
   * row and block) and the P.V MFMA multiplies its products by 2^-k again
   * through the power-of-two (E8M0) scale of its P operand, so small
   * probabilities keep normal e4m3 precision (aicronaca.it, "Perché l'FP8
   * non basta da solo"; ai4bro.com, "How does ZYFA work?"). O is still
   * divided by the fp32 sum of the exact exponentials and LSE is unchanged.
   */
  ATTN_FLAG_P_BLOCK_SCALE = 1,
  /*
   * FP8 only, O only (lse must be NULL; not with ATTN_FLAG_P_BLOCK_SCALE):
   * Lean P (Le Fil IA, context paragraph; aicronaca.it, "Perché l'FP8 non
   * basta da solo"; ai4bro.com, "How does ZYFA work?"). No exponential is
   * evaluated: an e4m3 code read as an integer grows by 8 per doubling, so
   * the code of p = 2^x is taken as round(8x + 56) (exact at powers of two,
   * linear in between, up to 6.2% high), with a power-of-two shift per
   * (query row, 64-key block) taken back by the P operand's E8M0 scale, and
   * O is divided by the sum of these rounded probabilities (one more MFMA).
   * An approximation: its O error is about 1.5 times that of the exact path.
   * SWITCHED OFF: it misses the FP8 O bar of 3e-2 on part of the workloads
   * and runs no faster than the exact path on this hardware, so every call
   * with this flag (and no other argument error) returns
   * ATTN_ERR_UNSUPPORTED.
   */
  ATTN_FLAG_LEAN_P = 2,
  /*
   * FP8 only, together with ATTN_FLAG_P_BLOCK_SCALE (alone, or with
   * ATTN_FLAG_LEAN_P: ATTN_ERR_INVALID): O is divided by the row sum of the
   * rounded, block-scaled probabilities that the P.V products take,
   * accumulated by one more MFMA per 64-key step (P times an operand of
   * e4m3 ones, under P's power-of-two scale), instead of by the fp32 sum of
   * the exact exponentials (aicronaca.it, "Perché l'FP8 non basta da solo";
   * ai4bro.com, "How does ZYFA work?": the row sum from one extra MFMA). The
   * rounding of each row's largest probabilities then cancels between O and
   * its normalizer, which lowers the O error on heavy-tailed inputs. The
   * block scaling is required: without it, probabilities far below a row's
   * running maximum underflow in e4m3 and drop out of the rounded sum. LSE
   * still comes from the fp32 exact sum. This mode applies the score factor
   * with one fma per score whatever the query scale.
   */
  ATTN_FLAG_P_ROUNDED_SUM = 4,
};

/*
 * As attn_prefill_fwd, with an explicit softmax scale (> 0, finite), the
 * three dequantization scales read from DEVICE memory (each a pointer to one
 * float, e.g. the output of attn_quantize_fp8), so a quantize -> attention
 * sequence needs no host synchronisation, and option flags. Passing
 * d_scales == NULL uses q_scale, k_scale, v_scale from the host arguments
 * instead.
 *   d_scales    NULL, or device float[3] = {q_scale, k_scale, v_scale}.
 *   flags       0 or ATTN_FLAG_* bits: an unknown bit is ATTN_ERR_INVALID, a
 *               flag with dtype BF16 ATTN_ERR_UNSUPPORTED.
 */
int attn_prefill_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                        float q_scale, float k_scale, float v_scale, const float* d_scales,
                        float softmax_scale,
                        int B, int S, int Hq, int Hkv, int d_qk, int d_v,
                        int causal, int dtype, int flags, hipStream_t stream);

/*
 * Per-tensor FP8 quantize-and-layout step (the input side of the FP8 path).
 * The attention inputs are FP8 e4m3 (ai4bro.com, "TL;DR"; Le Fil IA, context
 * paragraph: an e4m3 code read as an integer grows by 8 per doubling); the
 * pages give no scale granularity, so this is one absmax scale per tensor.
 *   x        device input, n elements, float32 (x_dtype 0) or bfloat16 (1),
 *            16-byte aligned.
 *   x8       device output, n uint8 e4m3fn codes, same layout as x, 16-byte
 *            aligned.
 *   d_scale  device output, one float: absmax(|x|)/448 in fp32 (1.0 when x
 *            is all zeros). Also used as the absmax accumulator while the
 *            call's kernels run, so it must not overlap x or x8.
 *   n        element count, 0 < n < 2^40.
 * code = e4m3fn(x / scale), division in fp32 correctly rounded, rounding to
 * nearest with ties to even. Inputs must be finite. Deterministic.
 * Errors: ATTN_ERR_INVALID for a null or misaligned pointer, a bad n or an
 * overlap of d_scale with x or x8; ATTN_ERR_UNSUPPORTED for another x_dtype.
 */
int attn_quantize_fp8(const void* x, int x_dtype, uint8_t* x8, float* d_scale, int64_t n,
                      hipStream_t stream);

/*
 * The same step for a QUERY tensor (same e4m3 format and sources), with the
 * scale folded for the kernel; x, x_dtype, x8, d_scale, n as above:
 *   d_k_scale      device pointer to the key tensor's scale (one float,
 *                  e.g. the d_scale of attn_quantize_fp8 on k), read on
 *                  the device after the work queued before this call.
 *   softmax_scale  the softmax scale the attention call will use (> 0,
 *                  finite; 1/sqrt(d_qk) for attn_prefill_fwd).
 * d_scale receives the smallest scale 2^j / (k_scale * softmax_scale *
 * log2(e)), j an integer, that is >= absmax(|x|)/448 (so at most twice it),
 * evaluated in fp64 with correctly rounded steps and rounded once to fp32;
 * 1.0 when x is all zeros. Codes are e4m3fn(x / scale) as above. The product
 * q_scale * k_scale * softmax_scale * log2(e) is then a power of two, which
 * lets the attention kernel apply it through the FP8 MFMA's power-of-two
 * operand scales instead of one vector multiply per score (the kernel
 * detects this by itself; any other scale takes the general path). d_k_scale
 * must not overlap d_scale.
 */
int attn_quantize_fp8_q(const void* x, int x_dtype, uint8_t* x8, float* d_scale, int64_t n,
                        const float* d_k_scale, float softmax_scale, hipStream_t stream);

/*
 * The whole FP8 input step for one attention call: K and V as
 * attn_quantize_fp8, then Q as attn_quantize_fp8_q with K's scale, in one
 * absmax launch and one encode launch over the three tensors (fewer, larger
 * launches than three separate calls; the codes and scales are identical).
 *   q, k, v      device inputs of nq, nk, nv elements (float32 if x_dtype 0,
 *                bfloat16 if 1), each 16-byte aligned; 0 < n < 2^40.
 *   q8, k8, v8   device outputs, e4m3fn codes in the layouts of the inputs.
 *   d_scales     device float[3] receiving {q_scale (folded), k_scale,
 *                v_scale}: the d_scales argument of attn_prefill_fwd_ex. Also
 *                the absmax accumulators while the call's kernels run, so it
 *                must not overlap any input or output.
 *   softmax_scale  the attention call's softmax scale (> 0, finite).
 */
int attn_quantize_fp8_qkv(const void* q, const void* k, const void* v, int x_dtype, int64_t nq, int64_t nk,
                          int64_t nv, uint8_t* q8, uint8_t* k8, uint8_t* v8, float* d_scales, float softmax_scale,
                          hipStream_t stream);

/*
 * The FP8 input step with a Hadamard rotation of the head vectors, for Q and
 * K (aicronaca.it, section "Perché l'FP8 non basta da solo": rotating Q and K
 * before the FP8 cast about halves the input quantization error). V is not
 * rotated.
 *   x, x_dtype, x8, d_scale, n   as attn_quantize_fp8; x is rows of d elements.
 *   d          head dim, the length of the last axis (n % d == 0). Rotation
 *              blocks of b = largest power of two dividing d, at most 128,
 *              must be 64 or 128 (d = 128: one block; d = 192: three of 64),
 *              else ATTN_ERR_UNSUPPORTED.
 *   d_k_scale  NULL: key tensor. Else query tensor, with d_k_scale and
 *              softmax_scale as in attn_quantize_fp8_q.
 * Each b-element block of a row becomes y = x H_b, H_b the unnormalized
 * Sylvester Hadamard matrix (entry (i,j) = (-1)^popcount(i & j)), formed in
 * fp64. Then (q H)(k H)^T = b q.k^T. The absmax is the max of fp32(|y|).
 * The code scale follows the rule of attn_quantize_fp8 (key) or
 * attn_quantize_fp8_q (query) on that absmax, and
 * code = e4m3fn(fp32(y * fp64(1/scale))), ties to even. d_scale receives the
 * code scale for a key and the code scale / b for a query. The dequantized
 * products are then the unrotated q.k, and the query keeps the folded
 * property, so the attention call needs no change. Deterministic.
 */
int attn_quantize_fp8_hadamard(const void* x, int x_dtype, uint8_t* x8, float* d_scale, int64_t n, int d,
                               const float* d_k_scale, float softmax_scale, hipStream_t stream);

/*
 * The rotated FP8 input step of one attention call: Q and K rotated by
 * Hadamard blocks as in attn_quantize_fp8_hadamard (Q with the folded scale
 * for the rotated K's scale, its stored scale divided by the block size), V
 * plain, in one absmax launch and one encode launch over the three tensors
 * (aicronaca.it, "Perché l'FP8 non basta da solo": the rotation costs a
 * small fraction of the attention time). Use it on heavy-tailed
 * activations: the FP8 matrix core sums a Q.K dot product only to about
 * 2^-12 of its sum of |products|, so where large Q and K channels meet (logits
 * of 50-80) the unrotated codes can move a row's LSE by up to ~2e-2; the
 * rotation spreads those channels over every column (under 6e-4 on the same
 * rows). Arguments as attn_quantize_fp8_qkv,
 * plus d, the head dim of Q and K (nq and nk multiples of it; blocks of
 * 64 or 128 columns as attn_quantize_fp8_hadamard, else
 * ATTN_ERR_UNSUPPORTED). The codes and scales equal those of the three
 * separate calls.
 */
int attn_quantize_fp8_qkv_hadamard(const void* q, const void* k, const void* v, int x_dtype, int64_t nq,
                                   int64_t nk, int64_t nv, int d, uint8_t* q8, uint8_t* k8, uint8_t* v8,
                                   float* d_scales, float softmax_scale, hipStream_t stream);

/*
 * BF16 input step: float32 -> bfloat16, round to nearest, ties to even (the
 * BF16 path takes its inputs unquantized: Le Fil IA, summary paragraph).
 *   x  device float32[n];  y  device bfloat16[n] (as uint16 bits), both
 *   16-byte aligned;  0 < n < 2^40.  Errors: ATTN_ERR_INVALID.
 */
int attn_cast_bf16(const float* x, uint16_t* y, int64_t n, hipStream_t stream);

/* Human-readable text of a return code (static storage). */
const char* attn_strerror(int code);

/* ABI version of this header: 2 (2: quantizers take (x, x_dtype, x8, d_scale, n, ...),
 * the cast (x, y, n, ...), attn_prefill_fwd_ex takes flags). */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_PREFILL_H */
