// Host-side launchers of the input-step kernels (quantize.hip).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace attn {

hipError_t launch_quantize_fp8(const void* x, int x_dtype, int64_t n, uint8_t* x8, float* d_scale,
                               hipStream_t stream);
hipError_t launch_cast_bf16(const float* x, int64_t n, uint16_t* y, hipStream_t stream);

}  // namespace attn
