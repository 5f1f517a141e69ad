// Shared device-side types and small helpers for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

#define ATTN_LDS __attribute__((address_space(3)))

// 32x32x64 FP8 (e4m3 x e4m3) MFMA, fp32 accumulate. Operand lane layout on
// gfx950 (established on hardware): A lane l holds row l%32, B lane l holds
// column l%32; the 32 bytes of lanes 0..31 and of lanes 32..63 are two
// disjoint halves of the 64-deep contraction, paired byte for byte between A
// and B. C/D lane l holds column l%32, register r holds row
// 8*(r/4) + 4*(l/32) + r%4. Scale operands 0 select the unscaled form.
__device__ __forceinline__ f32x16 mfma_f8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// The same MFMA with the product scaled by 2^(sa-127) * 2^(sb-127) (E8M0
// operand scales, one value for every lane here); the accumulator input is
// not scaled.
__device__ __forceinline__ f32x16 mfma_f8_scaled(const i32x8& a, const i32x8& b, const f32x16& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// 32x32x16 BF16 MFMA, fp32 accumulate; same row/column/accumulator layout,
// 8 contraction elements per lane per half.
__device__ __forceinline__ f32x16 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ds_read_b64_tr_b8: within each 16-lane group, lane k supplies the address
// of 8 bytes forming half k%2 of row k/2 of an 8 x 16 byte tile; lane i
// receives column i (byte j from row j).
__device__ __forceinline__ i32x2 lds_read_tr8(const ATTN_LDS char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((ATTN_LDS i32x2*)p);
}

// ds_read_b64_tr_b16: within each 16-lane group, lane k supplies the address
// of 4 16-bit elements forming quarter k%4 of row k/4 of a 4 x 16 element
// tile; lane i receives column i (element j from row j).
__device__ __forceinline__ i16x4 lds_read_tr16(const ATTN_LDS char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4*)p);
}

__device__ __forceinline__ i32x4 lds_read_b128(const ATTN_LDS char* p) {
  return *(const ATTN_LDS i32x4*)p;
}

__device__ __forceinline__ void lds_write_b128(ATTN_LDS char* p, const i32x4& v) {
  *(ATTN_LDS i32x4*)p = v;
}

// Largest of 16 accumulator values and m (IEEE 754-2019 maximum: a NaN
// would propagate; the values here are finite or -inf). This form compiles
// to three-input v_maximum3_f32; fmaxf's NaN rules keep the compiler from
// merging pairs of maxima of MFMA results.
__device__ __forceinline__ float max16(const f32x16& x, float m) {
#pragma unroll
  for (int r = 0; r < 16; r += 2) m = __builtin_elementwise_maximum(m, __builtin_elementwise_maximum(x[r], x[r + 1]));
  return m;
}

// Value of the other half-wave's lane (l ^ 32).
__device__ __forceinline__ float swap_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  // lane < 32: r[1] holds lane l+32; lane >= 32: r[0] holds lane l-32
  return __int_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// Two fp32 values -> two e4m3fn bytes (round to nearest even), placed in
// bytes 0,1 (hi = false) or 2,3 (hi = true) of `old`.
__device__ __forceinline__ int cvt_fp8x2(float a, float b, int old, bool hi) {
  return hi ? __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, true)
            : __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, false);
}

// As cvt_fp8x2, of a / div and b / div (one rounding, to nearest even; div
// a power of two here, so this scales by an exact power of two first).
// Values past the e4m3 range give NaN codes: callers keep them in range.
typedef short i16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ int cvt_fp8x2_div(float a, float b, float div, int old, bool hi) {
  const i16x2 o = __builtin_bit_cast(i16x2, old);
  return __builtin_bit_cast(int, hi ? __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, a, b, div, true)
                                    : __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, a, b, div, false));
}

// fp32 2^e for an integer e in [-126, 127] (built from the exponent field).
__device__ __forceinline__ float pow2i(int e) { return __int_as_float((e + 127) << 23); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// LDS pointer from a byte address.
__device__ __forceinline__ const ATTN_LDS char* lds_at(uint32_t a) { return (const ATTN_LDS char*)(uintptr_t)a; }

// Byte address of an LDS object (what M0 and ds_* address operands hold).
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const ATTN_LDS void*)p;
}

// 16 bytes per lane from global memory straight into LDS: lane l reads
// base + voff (base wave-uniform, in scalar registers; voff per lane) and its
// bytes land at lds_addr + 16*l (lds_addr is wave-uniform; the instruction
// takes it from M0). Issued as inline assembly so that the compiler does not
// treat later LDS reads of other ring stages as dependent on it: the caller
// tracks completion itself with wait_vmcnt() before the barrier that
// publishes the stage. M0 is set immediately before the load, with one
// wait state, and this file uses no other construct that needs M0.
__device__ __forceinline__ void global_to_lds_16_async(const void* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "s"(lds_addr)
               : "memory", "m0");
}

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left at their maxima): at most N
// of this wave's vector memory loads, the youngest, are still in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // vmcnt bits [3:0] and [15:14]; expcnt (bits 6:4) and lgkmcnt (11:8) at max
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Compiler scheduling fence: no instruction is moved across it.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Scheduling groups: the next `n` instructions of the class (in the current
// scheduling region) are placed here, in the order of these calls.
constexpr int kSchedValu = 0x002;
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
// (n is a constant after unrolling; the builtin wants it literal.)
template <int MASK>
__device__ __forceinline__ void sched_group(int n) {
  switch (n) {
    case 1: __builtin_amdgcn_sched_group_barrier(MASK, 1, 0); break;
    case 2: __builtin_amdgcn_sched_group_barrier(MASK, 2, 0); break;
    case 3: __builtin_amdgcn_sched_group_barrier(MASK, 3, 0); break;
    case 4: __builtin_amdgcn_sched_group_barrier(MASK, 4, 0); break;
    case 5: __builtin_amdgcn_sched_group_barrier(MASK, 5, 0); break;
    case 6: __builtin_amdgcn_sched_group_barrier(MASK, 6, 0); break;
    case 7: __builtin_amdgcn_sched_group_barrier(MASK, 7, 0); break;
    case 8: __builtin_amdgcn_sched_group_barrier(MASK, 8, 0); break;
    case 12: __builtin_amdgcn_sched_group_barrier(MASK, 12, 0); break;
    case 14: __builtin_amdgcn_sched_group_barrier(MASK, 14, 0); break;
    case 16: __builtin_amdgcn_sched_group_barrier(MASK, 16, 0); break;
    case 28: __builtin_amdgcn_sched_group_barrier(MASK, 28, 0); break;
    case 32: __builtin_amdgcn_sched_group_barrier(MASK, 32, 0); break;
    default: break;
  }
}

// Materialises x at this point of the program (an empty asm that reads and
// writes it): keeps the compiler from sinking its computation into a later
// conditional block.
__device__ __forceinline__ int pin(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Wave priority for instruction issue (0 = default).
template <int P>
__device__ __forceinline__ void set_priority() {
  __builtin_amdgcn_s_setprio(P);
}

// Wave-uniform value in a scalar register.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// True if any lane of the wave has `pred` set.
__device__ __forceinline__ bool wave_any(bool pred) { return __builtin_amdgcn_ballot_w64(pred) != 0; }

}  // namespace attn
