// Input step of the attention path: per-tensor FP8 e4m3fn quantization and
// the fp32 -> bf16 cast.
//
// The pages fix the FP8 format (e4m3: ai4bro.com "TL;DR"; Le Fil IA, context
// paragraph) but not the scale granularity; this library uses one fp32 scale
// per tensor: scale = absmax / 448 (448 = largest e4m3fn value), code =
// e4m3fn(x / scale) rounded to nearest even. A query tensor may instead take
// the folded scale (folded_scale_from_amax), at most twice absmax / 448,
// which turns the attention kernel's score factor into a power of two.
//
// Two HBM passes: a grid-wide absmax (each workgroup folds its maximum in
// with one integer atomic max on the IEEE bits, which orders non-negative
// floats like their values, so the result is independent of timing), then the
// cast. Both passes stream 16-byte vectors and are bound by HBM bandwidth.
#include "common.h"
#include "quantize.h"

namespace attn {

constexpr int QTHREADS = 256;

__global__ void amax_reset_kernel(uint32_t* amax_bits) { *amax_bits = 0u; }

__device__ __forceinline__ float bf16_bits_to_float(uint32_t u16) { return __uint_as_float(u16 << 16); }

// Inputs are streamed as 16-byte vectors (4 fp32 or 8 bf16 elements); each
// thread loads kVecsInFlight consecutive vectors per trip (all issued before
// any is used), so a wave's trip covers one contiguous span of
// 64 * kVecsInFlight * 16 bytes.
constexpr int kVecsInFlight = 4;

template <int XDT>
struct In16 {
  static constexpr int N = XDT == 0 ? 4 : 8;  // elements per 16-byte vector
  __device__ static void unpack(const uint4& w, float* v) {
    if constexpr (XDT == 0) {
      v[0] = __uint_as_float(w.x); v[1] = __uint_as_float(w.y);
      v[2] = __uint_as_float(w.z); v[3] = __uint_as_float(w.w);
    } else {
      const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = bf16_bits_to_float(u[j] & 0xFFFFu);
        v[2 * j + 1] = bf16_bits_to_float(u[j] >> 16);
      }
    }
  }
  __device__ static float load1(const void* x, int64_t i) {
    return XDT == 0 ? ((const float*)x)[i] : bf16_bits_to_float(((const uint16_t*)x)[i]);
  }
};

template <int XDT>
__device__ __forceinline__ float absmax16(const uint4& w) {
  float v[In16<XDT>::N];
  In16<XDT>::unpack(w, v);
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < In16<XDT>::N; ++j) m = fmaxf(m, fabsf(v[j]));
  return m;
}

template <int XDT>
__global__ __launch_bounds__(QTHREADS) void amax_kernel(const void* __restrict__ x, int64_t n,
                                                         uint32_t* amax_bits) {
  constexpr int N = In16<XDT>::N, U = kVecsInFlight;
  float m = 0.f;
  const int64_t nthreads = (int64_t)gridDim.x * QTHREADS;
  const int64_t gtid = (int64_t)blockIdx.x * QTHREADS + threadIdx.x;
  const int64_t nv = n / N;
  const uint4* xv = (const uint4*)x;
  const int64_t ntrips = nv / U;
  for (int64_t t = gtid; t < ntrips; t += nthreads) {
    uint4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = xv[t * U + u];
#pragma unroll
    for (int u = 0; u < U; ++u) m = fmaxf(m, absmax16<XDT>(w[u]));
  }
  for (int64_t i = ntrips * U + gtid; i < nv; i += nthreads) m = fmaxf(m, absmax16<XDT>(xv[i]));
  for (int64_t e = nv * N + gtid; e < n; e += nthreads) m = fmaxf(m, fabsf(In16<XDT>::load1(x, e)));
  // wave reduction, then across the workgroup's 4 waves
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  __shared__ float red[QTHREADS / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = red[0];
#pragma unroll
    for (int w = 1; w < QTHREADS / 64; ++w) r = fmaxf(r, red[w]);
    atomicMax(amax_bits, __float_as_uint(r));
  }
}

__device__ __forceinline__ float scale_from_amax(uint32_t bits) {
  const float a = __uint_as_float(bits);
  return a == 0.f ? 1.f : __fdiv_rn(a, 448.f);
}

// Folded scale of a query tensor: the smallest scale of the form
// 2^j / (k_scale * softmax_scale * log2 e) that is >= absmax / 448, so that
// the attention kernel's score factor q_scale * k_scale * softmax_scale *
// log2 e is the power of two 2^j (up to the fp32 rounding of the stored
// scale) and goes into the MFMA's operand scales. Computed in fp64 (each
// step correctly rounded), rounded once to fp32; 1.0 for an all-zero tensor.
__device__ __forceinline__ float folded_scale_from_amax(uint32_t bits, float k_scale, float sm_scale) {
  const float a = __uint_as_float(bits);
  if (a == 0.f) return 1.f;
  const double g = (double)k_scale * (double)sm_scale * 1.4426950408889634;
  const double t = ((double)a / 448.0) * g;
  int e;
  const double f = frexp(t, &e);  // t = f * 2^e, f in [0.5, 1)
  const int j = f == 0.5 ? e - 1 : e;
  return (float)(ldexp(1.0, j) / g);
}

// The scale the cast uses: plain (d_k_scale == nullptr) or folded.
__device__ __forceinline__ float quant_scale(uint32_t bits, const float* d_k_scale, float sm_scale) {
  return d_k_scale ? folded_scale_from_amax(bits, *d_k_scale, sm_scale) : scale_from_amax(bits);
}

template <int XDT>
__global__ __launch_bounds__(QTHREADS) void quant_kernel(const void* __restrict__ x, int64_t n,
                                                          const uint32_t* __restrict__ amax_bits,
                                                          const float* __restrict__ d_k_scale, float sm_scale,
                                                          uint8_t* __restrict__ out) {
  const float scale = quant_scale(*amax_bits, d_k_scale, sm_scale);
  constexpr int N = In16<XDT>::N, U = kVecsInFlight;
  const int64_t nthreads = (int64_t)gridDim.x * QTHREADS;
  const int64_t gtid = (int64_t)blockIdx.x * QTHREADS + threadIdx.x;
  const int64_t nv = n / N;
  const uint4* xv = (const uint4*)x;
  // N codes of one vector: 4 bytes (fp32 input) or 8 bytes (bf16 input)
  auto encode = [&](const uint4& w, int64_t vi) {
    float v[N];
    In16<XDT>::unpack(w, v);
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] = __fdiv_rn(v[j], scale);
    int c[N / 4];
#pragma unroll
    for (int q = 0; q < N / 4; ++q) {
      const int lo = cvt_fp8x2(v[4 * q], v[4 * q + 1], 0, false);
      c[q] = cvt_fp8x2(v[4 * q + 2], v[4 * q + 3], lo, true);
    }
    if constexpr (N == 4) ((uint32_t*)out)[vi] = (uint32_t)c[0];
    else ((uint2*)out)[vi] = make_uint2((uint32_t)c[0], (uint32_t)c[1]);
  };
  const int64_t ntrips = nv / U;
  for (int64_t t = gtid; t < ntrips; t += nthreads) {
    uint4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = xv[t * U + u];
#pragma unroll
    for (int u = 0; u < U; ++u) encode(w[u], t * U + u);
  }
  for (int64_t i = ntrips * U + gtid; i < nv; i += nthreads) encode(xv[i], i);
  for (int64_t e = nv * N + gtid; e < n; e += nthreads)
    out[e] = (uint8_t)(cvt_fp8x2(__fdiv_rn(In16<XDT>::load1(x, e), scale), 0.f, 0, false) & 0xFF);
}

__global__ void scale_finalize_kernel(uint32_t* amax_bits, const float* d_k_scale, float sm_scale) {
  *amax_bits = __float_as_uint(quant_scale(*amax_bits, d_k_scale, sm_scale));
}

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__global__ __launch_bounds__(QTHREADS) void cast_bf16_kernel(const float* __restrict__ x, int64_t n,
                                                              uint16_t* __restrict__ y) {
  constexpr int U = kVecsInFlight;
  const int64_t nthreads = (int64_t)gridDim.x * QTHREADS;
  const int64_t gtid = (int64_t)blockIdx.x * QTHREADS + threadIdx.x;
  const int64_t nv = n / 4;
  const uint4* xv = (const uint4*)x;
  auto cast4 = [&](const uint4& w, int64_t vi) {
    ((uint2*)y)[vi] = make_uint2(f32_to_bf16_rne(__uint_as_float(w.x)) | (f32_to_bf16_rne(__uint_as_float(w.y)) << 16),
                                 f32_to_bf16_rne(__uint_as_float(w.z)) | (f32_to_bf16_rne(__uint_as_float(w.w)) << 16));
  };
  const int64_t ntrips = nv / U;
  for (int64_t t = gtid; t < ntrips; t += nthreads) {
    uint4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = xv[t * U + u];
#pragma unroll
    for (int u = 0; u < U; ++u) cast4(w[u], t * U + u);
  }
  for (int64_t i = ntrips * U + gtid; i < nv; i += nthreads) cast4(xv[i], i);
  for (int64_t e = nv * 4 + gtid; e < n; e += nthreads) y[e] = (uint16_t)f32_to_bf16_rne(x[e]);
}

static int stream_grid(int64_t n) {
  // up to 16 workgroups per CU, each running several trips
  const int64_t per_block = (int64_t)QTHREADS * kVecsInFlight * 4;  // elements (fp32 vectors)
  int64_t g = (n + per_block - 1) / per_block;
  if (g > 256 * 16) g = 256 * 16;
  if (g < 1) g = 1;
  return (int)g;
}

hipError_t launch_quantize_fp8(const void* x, int x_dtype, int64_t n, uint8_t* x8, float* d_scale,
                               const float* d_k_scale, float sm_scale, hipStream_t stream) {
  uint32_t* bits = (uint32_t*)d_scale;
  const int grid = stream_grid(n);
  hipLaunchKernelGGL(amax_reset_kernel, dim3(1), dim3(1), 0, stream, bits);
  if (x_dtype == 0) {
    hipLaunchKernelGGL(amax_kernel<0>, dim3(grid), dim3(QTHREADS), 0, stream, x, n, bits);
    hipLaunchKernelGGL(quant_kernel<0>, dim3(grid), dim3(QTHREADS), 0, stream, x, n, bits, d_k_scale, sm_scale, x8);
  } else {
    hipLaunchKernelGGL(amax_kernel<1>, dim3(grid), dim3(QTHREADS), 0, stream, x, n, bits);
    hipLaunchKernelGGL(quant_kernel<1>, dim3(grid), dim3(QTHREADS), 0, stream, x, n, bits, d_k_scale, sm_scale, x8);
  }
  hipLaunchKernelGGL(scale_finalize_kernel, dim3(1), dim3(1), 0, stream, bits, d_k_scale, sm_scale);
  return hipGetLastError();
}

hipError_t launch_cast_bf16(const float* x, int64_t n, uint16_t* y, hipStream_t stream) {
  hipLaunchKernelGGL(cast_bf16_kernel, dim3(stream_grid(n)), dim3(QTHREADS), 0, stream, x, n, y);
  return hipGetLastError();
}

}  // namespace attn
