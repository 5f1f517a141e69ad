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

// Absmax of x over the workgroups blk = 0 .. nblk-1 assigned to it; folded
// into *amax_bits.
template <int XDT>
__device__ __forceinline__ void amax_body(const void* __restrict__ x, int64_t n, uint32_t* amax_bits, int blk,
                                          int nblk) {
  constexpr int N = In16<XDT>::N, U = kVecsInFlight;
  float m = 0.f;
  const int64_t nthreads = (int64_t)nblk * QTHREADS;
  const int64_t gtid = (int64_t)blk * QTHREADS + threadIdx.x;
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

template <int XDT>
__global__ __launch_bounds__(QTHREADS) void amax_kernel(const void* __restrict__ x, int64_t n,
                                                         uint32_t* amax_bits) {
  amax_body<XDT>(x, n, amax_bits, blockIdx.x, gridDim.x);
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

// Codes of x with `scale` over the workgroups blk = 0 .. nblk-1 assigned to it.
template <int XDT>
__device__ __forceinline__ void quant_body(const void* __restrict__ x, int64_t n, float scale,
                                           uint8_t* __restrict__ out, int blk, int nblk) {
  constexpr int N = In16<XDT>::N, U = kVecsInFlight;
  const int64_t nthreads = (int64_t)nblk * QTHREADS;
  const int64_t gtid = (int64_t)blk * QTHREADS + threadIdx.x;
  const int64_t nv = n / N;
  const uint4* xv = (const uint4*)x;
  // N codes of one vector (4 bytes for fp32 input, 8 for bf16) into c[0 .. N/4)
  auto encode = [&](const uint4& w, uint32_t* c) {
    float v[N];
    In16<XDT>::unpack(w, v);
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] = __fdiv_rn(v[j], scale);
#pragma unroll
    for (int q = 0; q < N / 4; ++q) {
      const int lo = cvt_fp8x2(v[4 * q], v[4 * q + 1], 0, false);
      c[q] = (uint32_t)cvt_fp8x2(v[4 * q + 2], v[4 * q + 3], lo, true);
    }
  };
  const int64_t ntrips = nv / U;
  // trips in reverse order: the absmax pass ends on the tensor's tail, part
  // of which the memory-side cache still holds when this pass starts
  for (int64_t t0 = gtid; t0 < ntrips; t0 += nthreads) {
    const int64_t t = ntrips - 1 - t0;
    uint4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = xv[t * U + u];
    // the trip's U * N codes are contiguous: written with 16-byte stores
    uint32_t c[U * N / 4];
#pragma unroll
    for (int u = 0; u < U; ++u) encode(w[u], c + u * (N / 4));
    uint4* o4 = (uint4*)(out + t * (U * N));
#pragma unroll
    for (int i = 0; i < U * N / 16; ++i) o4[i] = make_uint4(c[4 * i], c[4 * i + 1], c[4 * i + 2], c[4 * i + 3]);
  }
  for (int64_t i = ntrips * U + gtid; i < nv; i += nthreads) {
    uint32_t c[N / 4];
    encode(xv[i], c);
    if constexpr (N == 4) ((uint32_t*)out)[i] = c[0];
    else ((uint2*)out)[i] = make_uint2(c[0], c[1]);
  }
  for (int64_t e = nv * N + gtid; e < n; e += nthreads)
    out[e] = (uint8_t)(cvt_fp8x2(__fdiv_rn(In16<XDT>::load1(x, e), scale), 0.f, 0, false) & 0xFF);
}

template <int XDT>
__global__ __launch_bounds__(QTHREADS) void quant_kernel(const void* __restrict__ x, int64_t n,
                                                          const uint32_t* __restrict__ amax_bits,
                                                          const float* __restrict__ d_k_scale, float sm_scale,
                                                          uint8_t* __restrict__ out) {
  quant_body<XDT>(x, n, quant_scale(*amax_bits, d_k_scale, sm_scale), out, blockIdx.x, gridDim.x);
}

// ---- Q, K and V in one pass each: the workgroups of one launch are split
// into three ranges, one per tensor (0 = Q, 1 = K, 2 = V). The absmax of Q
// does not depend on K, and Q's folded scale needs only K's absmax, so one
// absmax launch and one encode launch serve all three tensors; the codes and
// scales are those of three separate calls (K, V plain, Q folded).
struct Qkv3 {
  const void* x[3];
  int64_t n[3];
  uint8_t* out[3];
  int first[3];  // first workgroup of each range
  int nblk[3];
  uint32_t* bits;  // device float[3]: absmax bits, then the scales {q, k, v}
  float sm_scale;
};

__device__ __forceinline__ int qkv_range(const Qkv3& a, int bid) {
  return bid >= a.first[2] ? 2 : (bid >= a.first[1] ? 1 : 0);
}

__global__ void amax3_reset_kernel(uint32_t* bits) {
  if (threadIdx.x < 3) bits[threadIdx.x] = 0u;
}

template <int XDT>
__global__ __launch_bounds__(QTHREADS) void amax3_kernel(Qkv3 a) {
  const int i = qkv_range(a, blockIdx.x);
  amax_body<XDT>(a.x[i], a.n[i], a.bits + i, blockIdx.x - a.first[i], a.nblk[i]);
}

template <int XDT>
__global__ __launch_bounds__(QTHREADS) void quant3_kernel(Qkv3 a) {
  const int i = qkv_range(a, blockIdx.x);
  const float scale = i == 0 ? folded_scale_from_amax(a.bits[0], scale_from_amax(a.bits[1]), a.sm_scale)
                             : scale_from_amax(a.bits[i]);
  quant_body<XDT>(a.x[i], a.n[i], scale, a.out[i], blockIdx.x - a.first[i], a.nblk[i]);
}

// (q_post: 1, or 1/b for a rotated query: exact, b is a power of two)
__global__ void scale3_finalize_kernel(uint32_t* bits, float sm_scale, float q_post) {
  const float ks = scale_from_amax(bits[1]), vs = scale_from_amax(bits[2]);
  const float qs = folded_scale_from_amax(bits[0], ks, sm_scale) * q_post;
  bits[0] = __float_as_uint(qs);
  bits[1] = __float_as_uint(ks);
  bits[2] = __float_as_uint(vs);
}

// Replaces the absmax bits by the stored scale: the scale the codes were
// taken with, times `post` (1, or 1/b for a rotated query: exact, b is a
// power of two).
__global__ void scale_finalize_kernel(uint32_t* amax_bits, const float* d_k_scale, float sm_scale, float post) {
  *amax_bits = __float_as_uint(quant_scale(*amax_bits, d_k_scale, sm_scale) * post);
}

// ---- Hadamard rotation ahead of the FP8 cast (aicronaca.it, section "Perché
// l'FP8 non basta da solo": rotating Q and K before the cast about halves the
// input error). Each b-column block of a row (b = 128 for d = 128, 64 for
// d = 192) becomes y = x H_b, H_b the unnormalized Sylvester matrix with
// entry (i, j) = (-1)^popcount(i & j), so (q H)(k H)^T = b q.k^T. The sums
// are formed in fp64, so the code decision is taken on (nearly) exact values:
// code = e4m3(fp32(y * fp64(1 / scale))). The absmax is taken over fp32(|y|)
// and the scale follows the unrotated rules; a query's stored scale is then
// divided by b.
//
// Lane layout: one block row per quad of lanes. Lane j of a quad holds the
// row's 16-byte input vectors j, j+4, j+8, ..., so one load instruction of a
// quad reads 64 contiguous bytes. Element e of the row sits in lane
// j = (e / R) % 4, register (e % R) + R * (e / 4R), R elements per vector.
// The two lane bits of e are exchanged with quad-permute DPP moves; the
// other bits are butterflies over the lane's own registers.
template <int XDT, int BLK>
struct HadShape {
  static constexpr int R = XDT == 0 ? 4 : 8;   // elements per 16-byte vector
  static constexpr int NV = BLK / (4 * R);     // vectors per lane
  static constexpr int NE = NV * R;            // elements per lane
  static_assert(NV >= 1 && BLK % (4 * R) == 0, "block layout");
};

// Value of `v` in lane (lane ^ M) of the same quad (M = 1 or 2).
template <int M>
__device__ __forceinline__ double quad_xor(double v) {
  constexpr int ctrl = M == 1 ? 0xB1 : 0x4E;  // quad_perm [1,0,3,2] / [2,3,0,1]
  const uint64_t u = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, ctrl, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), ctrl, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}

// Rotated values of this lane's elements of block row `br` (all zero when
// br >= nbr, which holds for a whole quad at once). Every lane of the wave
// must call it (the DPP moves read the quad's other lanes).
template <int XDT, int BLK>
__device__ __forceinline__ void had_rotate(const void* __restrict__ x, int64_t br, int64_t nbr, int j, double* y) {
  using H = HadShape<XDT, BLK>;
  uint4 w[H::NV];
  if (br < nbr) {
    const uint4* row = (const uint4*)((const char*)x + br * (int64_t)(BLK * (XDT == 0 ? 4 : 2)));
#pragma unroll
    for (int u = 0; u < H::NV; ++u) w[u] = row[j + 4 * u];
  } else {
#pragma unroll
    for (int u = 0; u < H::NV; ++u) w[u] = make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int u = 0; u < H::NV; ++u) {
    float f[H::R];
    In16<XDT>::unpack(w[u], f);
#pragma unroll
    for (int r = 0; r < H::R; ++r) y[u * H::R + r] = (double)f[r];
  }
  // index bits held within the lane: (a, b) -> (a + b, a - b), a at the
  // position with the bit clear
#pragma unroll
  for (int h = 1; h < H::NE; h <<= 1) {
#pragma unroll
    for (int t = 0; t < H::NE; ++t) {
      if (!(t & h)) {
        const double a = y[t], b = y[t + h];
        y[t] = a + b;
        y[t + h] = a - b;
      }
    }
  }
  // the two lane bits
#pragma unroll
  for (int t = 0; t < H::NE; ++t) {
    const double o = quad_xor<1>(y[t]);
    y[t] = (j & 1) ? o - y[t] : y[t] + o;
  }
#pragma unroll
  for (int t = 0; t < H::NE; ++t) {
    const double o = quad_xor<2>(y[t]);
    y[t] = (j & 2) ? o - y[t] : y[t] + o;
  }
}

// Each wave takes 16 block rows per trip; the trip count is uniform per wave.
// The bodies serve the workgroups blk = 0 .. nblk-1 assigned to the tensor.
template <int XDT, int BLK>
__device__ __forceinline__ void had_amax_body(const void* __restrict__ x, int64_t nbr, uint32_t* amax_bits, int blk,
                                              int nblk) {
  using H = HadShape<XDT, BLK>;
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blk * (QTHREADS / 64) + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)nblk * (QTHREADS / 64);
  float m = 0.f;
  for (int64_t br0 = wave * 16; br0 < nbr; br0 += nwaves * 16) {
    double y[H::NE];
    had_rotate<XDT, BLK>(x, br0 + (lane >> 2), nbr, lane & 3, y);
#pragma unroll
    for (int t = 0; t < H::NE; ++t) m = fmaxf(m, (float)fabs(y[t]));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  __shared__ float red[QTHREADS / 64];
  if (lane == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = red[0];
#pragma unroll
    for (int w = 1; w < QTHREADS / 64; ++w) r = fmaxf(r, red[w]);
    atomicMax(amax_bits, __float_as_uint(r));
  }
}

template <int XDT, int BLK>
__global__ __launch_bounds__(QTHREADS) void had_amax_kernel(const void* __restrict__ x, int64_t nbr,
                                                             uint32_t* amax_bits) {
  had_amax_body<XDT, BLK>(x, nbr, amax_bits, blockIdx.x, gridDim.x);
}

template <int XDT, int BLK>
__device__ __forceinline__ void had_quant_body(const void* __restrict__ x, int64_t nbr, float scale,
                                               uint8_t* __restrict__ out, int blk, int nblk) {
  using H = HadShape<XDT, BLK>;
  const double rcp = 1.0 / (double)scale;
  const int lane = threadIdx.x & 63, j = lane & 3;
  const int64_t wave = (int64_t)blk * (QTHREADS / 64) + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)nblk * (QTHREADS / 64);
  for (int64_t br0 = wave * 16; br0 < nbr; br0 += nwaves * 16) {
    const int64_t br = br0 + (lane >> 2);
    double y[H::NE];
    had_rotate<XDT, BLK>(x, br, nbr, j, y);
    if (br < nbr) {
      uint8_t* orow = out + br * BLK;
#pragma unroll
      for (int u = 0; u < H::NV; ++u) {
        int c[H::R / 4];
#pragma unroll
        for (int q = 0; q < H::R / 4; ++q) {
          const double* yy = y + u * H::R + 4 * q;
          const int lo = cvt_fp8x2((float)(yy[0] * rcp), (float)(yy[1] * rcp), 0, false);
          c[q] = cvt_fp8x2((float)(yy[2] * rcp), (float)(yy[3] * rcp), lo, true);
        }
        uint8_t* dst = orow + H::R * (j + 4 * u);
        if constexpr (H::R == 4) *(uint32_t*)dst = (uint32_t)c[0];
        else *(uint2*)dst = make_uint2((uint32_t)c[0], (uint32_t)c[1]);
      }
    }
  }
}

template <int XDT, int BLK>
__global__ __launch_bounds__(QTHREADS) void had_quant_kernel(const void* __restrict__ x, int64_t nbr,
                                                              const uint32_t* __restrict__ amax_bits,
                                                              const float* __restrict__ d_k_scale, float sm_scale,
                                                              uint8_t* __restrict__ out) {
  had_quant_body<XDT, BLK>(x, nbr, quant_scale(*amax_bits, d_k_scale, sm_scale), out, blockIdx.x, gridDim.x);
}

// ---- the rotated input step of one attention call: Q and K rotated, V
// plain, split over the workgroups of one absmax launch and one encode
// launch as in Qkv3 (Q folded with the rotated K's scale; its stored scale
// is then divided by the block size). The codes and scales are those of the
// three separate calls.
template <int XDT, int BLK>
__global__ __launch_bounds__(QTHREADS) void had_amax3_kernel(Qkv3 a) {
  const int i = qkv_range(a, blockIdx.x);
  if (i < 2) had_amax_body<XDT, BLK>(a.x[i], a.n[i] / BLK, a.bits + i, blockIdx.x - a.first[i], a.nblk[i]);
  else amax_body<XDT>(a.x[2], a.n[2], a.bits + 2, blockIdx.x - a.first[2], a.nblk[2]);
}

template <int XDT, int BLK>
__global__ __launch_bounds__(QTHREADS) void had_quant3_kernel(Qkv3 a) {
  const int i = qkv_range(a, blockIdx.x);
  const float ks = scale_from_amax(a.bits[1]);
  if (i == 0)
    had_quant_body<XDT, BLK>(a.x[0], a.n[0] / BLK, folded_scale_from_amax(a.bits[0], ks, a.sm_scale), a.out[0],
                             blockIdx.x - a.first[0], a.nblk[0]);
  else if (i == 1)
    had_quant_body<XDT, BLK>(a.x[1], a.n[1] / BLK, ks, a.out[1], blockIdx.x - a.first[1], a.nblk[1]);
  else
    quant_body<XDT>(a.x[2], a.n[2], scale_from_amax(a.bits[2]), a.out[2], blockIdx.x - a.first[2], a.nblk[2]);
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
  hipLaunchKernelGGL(scale_finalize_kernel, dim3(1), dim3(1), 0, stream, bits, d_k_scale, sm_scale, 1.0f);
  return hipGetLastError();
}

static int had_grid(int64_t nbr);

template <int XDT, int BLK>
static void launch_had(const void* x, int64_t nbr, uint32_t* bits, const float* d_k_scale, float sm_scale,
                       uint8_t* x8, hipStream_t stream) {
  const int g = had_grid(nbr);
  hipLaunchKernelGGL((had_amax_kernel<XDT, BLK>), dim3(g), dim3(QTHREADS), 0, stream, x, nbr, bits);
  hipLaunchKernelGGL((had_quant_kernel<XDT, BLK>), dim3(g), dim3(QTHREADS), 0, stream, x, nbr, bits, d_k_scale,
                     sm_scale, x8);
}

hipError_t launch_quantize_fp8_hadamard(const void* x, int x_dtype, int64_t n, int block, uint8_t* x8,
                                        float* d_scale, const float* d_k_scale, float sm_scale,
                                        hipStream_t stream) {
  uint32_t* bits = (uint32_t*)d_scale;
  const int64_t nbr = n / block;
  hipLaunchKernelGGL(amax_reset_kernel, dim3(1), dim3(1), 0, stream, bits);
  if (block == 128) {
    if (x_dtype == 0) launch_had<0, 128>(x, nbr, bits, d_k_scale, sm_scale, x8, stream);
    else launch_had<1, 128>(x, nbr, bits, d_k_scale, sm_scale, x8, stream);
  } else {
    if (x_dtype == 0) launch_had<0, 64>(x, nbr, bits, d_k_scale, sm_scale, x8, stream);
    else launch_had<1, 64>(x, nbr, bits, d_k_scale, sm_scale, x8, stream);
  }
  const float post = d_k_scale ? 1.0f / (float)block : 1.0f;
  hipLaunchKernelGGL(scale_finalize_kernel, dim3(1), dim3(1), 0, stream, bits, d_k_scale, sm_scale, post);
  return hipGetLastError();
}

hipError_t launch_quantize_fp8_qkv(const void* const x[3], int x_dtype, const int64_t n[3], uint8_t* const x8[3],
                                   float* d_scales, float sm_scale, hipStream_t stream) {
  Qkv3 a{};
  int total = 0;
  for (int i = 0; i < 3; ++i) {
    a.x[i] = x[i];
    a.n[i] = n[i];
    a.out[i] = x8[i];
    a.first[i] = total;
    a.nblk[i] = stream_grid(n[i]);
    total += a.nblk[i];
  }
  a.bits = (uint32_t*)d_scales;
  a.sm_scale = sm_scale;
  hipLaunchKernelGGL(amax3_reset_kernel, dim3(1), dim3(64), 0, stream, a.bits);
  if (x_dtype == 0) {
    hipLaunchKernelGGL(amax3_kernel<0>, dim3(total), dim3(QTHREADS), 0, stream, a);
    hipLaunchKernelGGL(quant3_kernel<0>, dim3(total), dim3(QTHREADS), 0, stream, a);
  } else {
    hipLaunchKernelGGL(amax3_kernel<1>, dim3(total), dim3(QTHREADS), 0, stream, a);
    hipLaunchKernelGGL(quant3_kernel<1>, dim3(total), dim3(QTHREADS), 0, stream, a);
  }
  hipLaunchKernelGGL(scale3_finalize_kernel, dim3(1), dim3(1), 0, stream, a.bits, sm_scale, 1.0f);
  return hipGetLastError();
}

static int had_grid(int64_t nbr) {
  // 64 block rows per workgroup trip (16 per wave), up to 16 workgroups per CU
  int64_t g = (nbr + 63) / 64;
  if (g > 256 * 16) g = 256 * 16;
  if (g < 1) g = 1;
  return (int)g;
}

template <int XDT, int BLK>
static void launch_had3(const Qkv3& a, int total, hipStream_t stream) {
  hipLaunchKernelGGL((had_amax3_kernel<XDT, BLK>), dim3(total), dim3(QTHREADS), 0, stream, a);
  hipLaunchKernelGGL((had_quant3_kernel<XDT, BLK>), dim3(total), dim3(QTHREADS), 0, stream, a);
}

hipError_t launch_quantize_fp8_qkv_hadamard(const void* const x[3], int x_dtype, const int64_t n[3], int block,
                                            uint8_t* const x8[3], float* d_scales, float sm_scale,
                                            hipStream_t stream) {
  Qkv3 a{};
  int total = 0;
  for (int i = 0; i < 3; ++i) {
    a.x[i] = x[i];
    a.n[i] = n[i];
    a.out[i] = x8[i];
    a.first[i] = total;
    a.nblk[i] = i < 2 ? had_grid(n[i] / block) : stream_grid(n[i]);
    total += a.nblk[i];
  }
  a.bits = (uint32_t*)d_scales;
  a.sm_scale = sm_scale;
  hipLaunchKernelGGL(amax3_reset_kernel, dim3(1), dim3(64), 0, stream, a.bits);
  if (block == 128) {
    if (x_dtype == 0) launch_had3<0, 128>(a, total, stream);
    else launch_had3<1, 128>(a, total, stream);
  } else {
    if (x_dtype == 0) launch_had3<0, 64>(a, total, stream);
    else launch_had3<1, 64>(a, total, stream);
  }
  hipLaunchKernelGGL(scale3_finalize_kernel, dim3(1), dim3(1), 0, stream, a.bits, sm_scale, 1.0f / (float)block);
  return hipGetLastError();
}

hipError_t launch_cast_bf16(const float* x, int64_t n, uint16_t* y, hipStream_t stream) {
  hipLaunchKernelGGL(cast_bf16_kernel, dim3(stream_grid(n)), dim3(QTHREADS), 0, stream, x, n, y);
  return hipGetLastError();
}

}  // namespace attn
