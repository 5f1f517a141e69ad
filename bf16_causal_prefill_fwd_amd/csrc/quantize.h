// Host-side launchers of the input-step kernels (quantize.hip).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace attn {

// d_k_scale == nullptr: plain per-tensor scale; else the folded query scale
// for that key scale and softmax scale.
hipError_t launch_quantize_fp8(const void* x, int x_dtype, int64_t n, uint8_t* x8, float* d_scale,
                               const float* d_k_scale, float sm_scale, hipStream_t stream);
// Hadamard-rotated variant: block = 64 or 128 columns, n a multiple of it.
// d_k_scale == nullptr: key (plain scale); else query (folded scale / block).
hipError_t launch_quantize_fp8_hadamard(const void* x, int x_dtype, int64_t n, int block, uint8_t* x8,
                                        float* d_scale, const float* d_k_scale, float sm_scale,
                                        hipStream_t stream);
// Q, K and V in one absmax launch and one encode launch; d_scales = device
// float[3] receiving {folded q_scale, k_scale, v_scale}.
hipError_t launch_quantize_fp8_qkv(const void* const x[3], int x_dtype, const int64_t n[3], uint8_t* const x8[3],
                                   float* d_scales, float sm_scale, hipStream_t stream);
// The same with Q and K rotated by Hadamard blocks of `block` columns (V
// plain); the stored query scale is the folded code scale / block.
hipError_t launch_quantize_fp8_qkv_hadamard(const void* const x[3], int x_dtype, const int64_t n[3], int block,
                                            uint8_t* const x8[3], float* d_scales, float sm_scale,
                                            hipStream_t stream);
hipError_t launch_cast_bf16(const float* x, int64_t n, uint16_t* y, hipStream_t stream);

}  // namespace attn
