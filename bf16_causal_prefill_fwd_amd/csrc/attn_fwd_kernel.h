// Causal prefill attention forward kernel for gfx950 (MI355X), FP8 e4m3 and BF16.
//
// The method (Le Fil IA, context paragraph; aicronaca.it, "Perché l'FP8 non
// basta da solo"; ai4bro.com, "Why is FP8 attention slow on MI355X?"): the
// two products Q.K^T and P.V run on the matrix cores, the row softmax between
// them runs on the vector ALU, tile by tile over the keys with a running row
// maximum and row sum. This file is its MI355X design:
//
//  * One workgroup owns BM = 32 * NWAVES query rows of one (batch, head);
//    each wave owns 32 rows and keeps its Q fragment in registers.
//  * Key/value tiles of BN rows are staged HBM -> registers -> LDS with
//    coalesced 16-byte loads, double buffered (one barrier per tile).
//  * S^T = K.Q^T is computed (K is the MFMA A operand), so each lane holds
//    scores of a single query: the row max needs one half-wave swap and the
//    row sum stays lane-local until the epilogue.
//  * O^T = V^T.P^T: P goes from the S^T accumulator straight into the B
//    operand (no shuffles); the key order inside the contraction is permuted
//    to match, and V is read in that order with LDS transpose reads, so V
//    stays row-major in LDS.
//  * Causal tile skip: a workgroup walks only key tiles up to its diagonal;
//    only tiles that straddle the diagonal (or the sequence end) are masked.
#pragma once

#include "common.h"

namespace attn {

struct FwdParams {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  uint16_t* o;
  float* lse;
  const float* d_scales;  // nullable: device {q_scale, k_scale, v_scale}
  float q_scale, k_scale, v_scale;
  float sm_scale;
  int B, S, Hq, Hkv;
  int causal;
  int n_mtiles;
  int xcd_remap;
};

template <bool FP8_, int DQK_, int DV_, int BM_, int BN_>
struct FwdCfg {
  static constexpr bool FP8 = FP8_;
  static constexpr int DQK = DQK_, DV = DV_, BM = BM_, BN = BN_;
  static constexpr int EB = FP8 ? 1 : 2;             // bytes per element
  static constexpr int NWAVES = BM / 32;
  static constexpr int NTHREADS = NWAVES * 64;
  static constexpr int KROW = DQK * EB;              // bytes per K row
  static constexpr int VROW = DV * EB;               // bytes per V row
  static constexpr int KCH = KROW / 16;              // 16-byte chunks per K row
  static constexpr int VCH = VROW / 16;
  static constexpr int KTILE = BN * KROW;
  static constexpr int VTILE = BN * VROW;
  static constexpr int STAGE = KTILE + VTILE;
  static constexpr int LDS_BYTES = 2 * STAGE;
  static constexpr int NST = BN / 32;                // 32-key score tiles
  static constexpr int NOT = DV / 32;                // 32-wide output tiles
  static constexpr int QK_STEPS = FP8 ? DQK / 64 : DQK / 16;
  static constexpr int KLOADS = KTILE / 16 / NTHREADS;
  static constexpr int VLOADS = VTILE / 16 / NTHREADS;
  static_assert(BM % 32 == 0 && BN % 64 == 0, "tile sizes");
  static_assert(DV % 32 == 0 && DQK % 64 == 0, "head dims");
  static_assert(KTILE % (16 * NTHREADS) == 0 && VTILE % (16 * NTHREADS) == 0, "staging split");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// Physical 16-byte chunk of logical chunk c in LDS row `row` (rows hold nch
// chunks). XOR-swizzling by the row spreads the column reads of consecutive
// rows over different banks. Rows of 12 chunks (FP8 d=192) swizzle chunks
// 0..7 and 8..11 separately so every chunk stays inside its row.
template <int NCH>
__device__ __forceinline__ int swz(int c, int row) {
  if constexpr (NCH % 8 == 0) {
    return c ^ (row & 7);
  } else {
    static_assert(NCH == 12, "row width");
    return c < 8 ? (c ^ (row & 7)) : (8 + ((c - 8) ^ (row & 3)));
  }
}

template <class C>
__device__ __forceinline__ void decode_work(const FwdParams& p, int& b, int& h, int& mt) {
  const int bid = blockIdx.x;
  const int G = p.Hq / p.Hkv;
  if (p.xcd_remap) {
    // Workgroups are dispatched round-robin over the 8 XCDs (bid % 8). Give
    // each XCD whole (batch, kv-head) units so the G query heads and all
    // query tiles that re-read one head's K/V share that XCD's L2; within
    // an XCD run the longest (latest) query tiles first.
    const int xcd = bid & 7, j = bid >> 3;
    const int upx = (p.B * p.Hkv) >> 3;
    const int per_tile = upx * G;
    const int tt = j / per_tile, rem = j - tt * per_tile;
    mt = p.n_mtiles - 1 - tt;
    const int ul = rem / G, gq = rem - ul * G;
    const int unit = xcd + 8 * ul;
    b = unit / p.Hkv;
    const int kvh = unit - b * p.Hkv;
    h = kvh * G + gq;
  } else {
    const int per_tile = p.B * p.Hq;
    const int tt = bid / per_tile, rem = bid - tt * per_tile;
    mt = p.n_mtiles - 1 - tt;
    b = rem / p.Hq;
    h = rem - b * p.Hq;
  }
}

template <class C>
__global__ __launch_bounds__(C::NTHREADS, 2) void attn_fwd_kernel(FwdParams p) {
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  ATTN_LDS char* smem = (ATTN_LDS char*)smem_raw;

  constexpr int BM = C::BM, BN = C::BN, DQK = C::DQK, DV = C::DV;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;   // query column / operand row of this lane
  const int g = lane >> 5;     // contraction half

  int b, h, mt;
  decode_work<C>(p, b, h, mt);
  const int G = p.Hq / p.Hkv;
  const int kvh = h / G;
  const int S = p.S;
  const int m0 = mt * BM;

  float qs = p.q_scale, ks = p.k_scale, vs = p.v_scale;
  if (p.d_scales) {
    qs = p.d_scales[0];
    ks = p.d_scales[1];
    vs = p.d_scales[2];
  }
  // scores in log2 units: t = c * (q8 . k8)
  const float c_log2 = qs * ks * p.sm_scale * 1.4426950408889634f;

  const int64_t q_row_stride = (int64_t)p.Hq * C::KROW;
  const int64_t kv_row_stride_k = (int64_t)p.Hkv * C::KROW;
  const int64_t kv_row_stride_v = (int64_t)p.Hkv * C::VROW;
  const uint8_t* kbase = p.k + ((int64_t)b * S * p.Hkv + kvh) * C::KROW;
  const uint8_t* vbase = p.v + ((int64_t)b * S * p.Hkv + kvh) * C::VROW;

  // ---- Q fragment (B operand of S^T = K.Q^T), loaded once per wave
  const int qrow = m0 + wave * 32 + l32;
  constexpr int QREGS = C::FP8 ? 8 : 4;  // ints per k-step
  i32x4 qf[C::QK_STEPS * QREGS / 4];
  {
    const uint8_t* qp = p.q + ((int64_t)b * S + qrow) * q_row_stride + (int64_t)h * C::KROW;
#pragma unroll
    for (int u = 0; u < C::QK_STEPS; ++u) {
      if constexpr (C::FP8) {
        // bytes [64u + 32g, +32): chunks 4u + 2g, 4u + 2g + 1
        const int off = 64 * u + 32 * g;
        i32x4 a = {0, 0, 0, 0}, c = {0, 0, 0, 0};
        if (qrow < S) {
          a = *(const i32x4*)(qp + off);
          c = *(const i32x4*)(qp + off + 16);
        }
        qf[2 * u] = a;
        qf[2 * u + 1] = c;
      } else {
        // elements [16u + 8g, +8) = bytes [32u + 16g, +16)
        const int off = 32 * u + 16 * g;
        i32x4 a = {0, 0, 0, 0};
        if (qrow < S) a = *(const i32x4*)(qp + off);
        qf[u] = a;
      }
    }
  }

  // ---- key range
  const int n_kv = p.causal ? min(S, m0 + BM) : S;
  const int nblk = (n_kv + BN - 1) / BN;

  // ---- staging of one K/V tile: global -> registers -> LDS
  i32x4 kst[C::KLOADS], vst[C::VLOADS];
  auto stage_load = [&](int n0) {
#pragma unroll
    for (int i = 0; i < C::KLOADS; ++i) {
      const int cid = tid + i * C::NTHREADS;
      const int row = cid / C::KCH, ch = cid % C::KCH;
      const int key = n0 + row;
      i32x4 x = {0, 0, 0, 0};
      if (key < S) x = *(const i32x4*)(kbase + (int64_t)key * kv_row_stride_k + 16 * ch);
      kst[i] = x;
    }
#pragma unroll
    for (int i = 0; i < C::VLOADS; ++i) {
      const int cid = tid + i * C::NTHREADS;
      const int row = cid / C::VCH, ch = cid % C::VCH;
      const int key = n0 + row;
      i32x4 x = {0, 0, 0, 0};
      if (key < S) x = *(const i32x4*)(vbase + (int64_t)key * kv_row_stride_v + 16 * ch);
      vst[i] = x;
    }
  };
  auto stage_store = [&](int buf) {
    ATTN_LDS char* kl = smem + buf * C::STAGE;
    ATTN_LDS char* vl = kl + C::KTILE;
#pragma unroll
    for (int i = 0; i < C::KLOADS; ++i) {
      const int cid = tid + i * C::NTHREADS;
      const int row = cid / C::KCH, ch = cid % C::KCH;
      lds_write_b128(kl + row * C::KROW + 16 * swz<C::KCH>(ch, row), kst[i]);
    }
#pragma unroll
    for (int i = 0; i < C::VLOADS; ++i) {
      const int cid = tid + i * C::NTHREADS;
      const int row = cid / C::VCH, ch = cid % C::VCH;
      lds_write_b128(vl + row * C::VROW + 16 * swz<C::VCH>(ch, row), vst[i]);
    }
  };

  // ---- running state
  f32x16 oacc[C::NOT];
#pragma unroll
  for (int t = 0; t < C::NOT; ++t) oacc[t] = f32x16{};
  float m_run = -INFINITY;  // running max of t (log2 units)
  float l_run = 0.f;        // this lane's share of the running row sum

  stage_load(0);
  stage_store(0);
  __syncthreads();

  for (int n = 0; n < nblk; ++n) {
    const int n0 = n * BN;
    const bool more = n + 1 < nblk;
    if (more) stage_load(n0 + BN);

    const ATTN_LDS char* kl = smem + (n & 1) * C::STAGE;
    const ATTN_LDS char* vl = kl + C::KTILE;

    // ---- S^T = K . Q^T
    f32x16 s[C::NST];
#pragma unroll
    for (int t = 0; t < C::NST; ++t) {
      s[t] = f32x16{};
      const int row = 32 * t + l32;
      const ATTN_LDS char* kr = kl + row * C::KROW;
#pragma unroll
      for (int u = 0; u < C::QK_STEPS; ++u) {
        if constexpr (C::FP8) {
          const int c0 = 4 * u + 2 * g;
          i32x4 a0 = lds_read_b128(kr + 16 * swz<C::KCH>(c0, row));
          i32x4 a1 = lds_read_b128(kr + 16 * swz<C::KCH>(c0 + 1, row));
          i32x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
          i32x8 bq = {qf[2 * u][0], qf[2 * u][1], qf[2 * u][2], qf[2 * u][3],
                      qf[2 * u + 1][0], qf[2 * u + 1][1], qf[2 * u + 1][2], qf[2 * u + 1][3]};
          s[t] = mfma_f8(a, bq, s[t]);
        } else {
          const int c0 = 2 * u + g;
          i32x4 a = lds_read_b128(kr + 16 * swz<C::KCH>(c0, row));
          s[t] = mfma_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, qf[u]), s[t]);
        }
      }
    }

    // ---- mask (only tiles that cross the diagonal or the sequence end)
    const bool need_mask = p.causal ? (n0 + BN - 1 > m0 + wave * 32) : (n0 + BN > S);
    if (need_mask) {
#pragma unroll
      for (int t = 0; t < C::NST; ++t) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = n0 + 32 * t + 8 * (r >> 2) + 4 * g + (r & 3);
          const bool hidden = p.causal ? (key > qrow) : (key >= S);
          if (hidden) s[t][r] = -INFINITY;
        }
      }
    }

    // ---- online softmax (exact exp2), log2 domain
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < C::NST; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
    mx = fmaxf(mx, swap_halves(mx));
    const float m_new = fmaxf(m_run, mx * c_log2);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    float lsum = 0.f;
#pragma unroll
    for (int t = 0; t < C::NST; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = fast_exp2(__builtin_fmaf(s[t][r], c_log2, -m_new));
        s[t][r] = pv;
        lsum += pv;
      }
    l_run = l_run * alpha + lsum;
#pragma unroll
    for (int t = 0; t < C::NOT; ++t) oacc[t] *= alpha;

    // ---- O^T += V^T . P^T
    if constexpr (C::FP8) {
#pragma unroll
      for (int u = 0; u < BN / 64; ++u) {
        // B operand byte j <- score tile 2u + j/16, register j%16
        i32x8 pf;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          const int t = 2 * u + (w >> 2), r = 4 * (w & 3);
          int x = cvt_fp8x2(s[t][r], s[t][r + 1], 0, false);
          pf[w] = cvt_fp8x2(s[t][r + 2], s[t][r + 3], x, true);
        }
        // V^T operand: lane (dv row l32, half g) byte j must hold the key that
        // byte j of the P operand holds: key 64u + 32(j/16) + 8((j%16)/4) + 4g + j%4.
        const int hh = lane >> 4, kk = lane & 15;
        const int krow_lane = 4 * (hh >> 1) + 8 * ((kk >> 1) >> 2) + ((kk >> 1) & 3);
#pragma unroll
        for (int tv = 0; tv < C::NOT; ++tv) {
          const int ch = 2 * tv + (hh & 1);
          i32x8 va;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int key = 64 * u + 32 * (rr >> 1) + 16 * (rr & 1) + krow_lane;
            const ATTN_LDS char* ap = vl + key * C::VROW + 16 * swz<C::VCH>(ch, key) + 8 * (kk & 1);
            i32x2 x = lds_read_tr8(ap);
            va[2 * rr] = x[0];
            va[2 * rr + 1] = x[1];
          }
          oacc[tv] = mfma_f8(va, pf, oacc[tv]);
        }
      }
    } else {
      const int hh = lane >> 4, kk = lane & 15;
#pragma unroll
      for (int t = 0; t < C::NST; ++t) {
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          // B operand element e <- score tile t, register 8cc + e
          bf16x8 pb;
#pragma unroll
          for (int e = 0; e < 8; ++e) pb[e] = (__bf16)s[t][8 * cc + e];
#pragma unroll
          for (int tv = 0; tv < C::NOT; ++tv) {
            // element e of lane (dv row, half g) <- key 32t + 16cc + 8(e/4) + 4g + e%4
            const int dv0 = 32 * tv + 16 * (hh & 1);
            const int chunk = dv0 / 8 + ((kk & 3) >> 1);
            i16x4 x[2];
#pragma unroll
            for (int hp = 0; hp < 2; ++hp) {
              const int key = 32 * t + 16 * cc + 8 * hp + 4 * (hh >> 1) + (kk >> 2);
              const ATTN_LDS char* ap = vl + key * C::VROW + 16 * swz<C::VCH>(chunk, key) + 8 * (kk & 1);
              x[hp] = lds_read_tr16(ap);
            }
            i32x4 vi = {0, 0, 0, 0};
            vi[0] = (int)(uint16_t)x[0][0] | ((int)(uint16_t)x[0][1] << 16);
            vi[1] = (int)(uint16_t)x[0][2] | ((int)(uint16_t)x[0][3] << 16);
            vi[2] = (int)(uint16_t)x[1][0] | ((int)(uint16_t)x[1][1] << 16);
            vi[3] = (int)(uint16_t)x[1][2] | ((int)(uint16_t)x[1][3] << 16);
            oacc[tv] = mfma_bf16(__builtin_bit_cast(bf16x8, vi), pb, oacc[tv]);
          }
        }
      }
    }

    if (more) stage_store((n + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: O = O_acc * v_scale / l, LSE = ln2 * (m + log2 l)
  const float l_tot = l_run + swap_halves(l_run);
  const float inv = vs / l_tot;
  if (qrow < S) {
    uint16_t* op = p.o + (((int64_t)b * S + qrow) * p.Hq + h) * DV;
#pragma unroll
    for (int tv = 0; tv < C::NOT; ++tv) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int dv = 32 * tv + 8 * a + 4 * g;
        uint32_t w0, w1;
        {
          __bf16 e0 = (__bf16)(oacc[tv][4 * a + 0] * inv), e1 = (__bf16)(oacc[tv][4 * a + 1] * inv);
          __bf16 e2 = (__bf16)(oacc[tv][4 * a + 2] * inv), e3 = (__bf16)(oacc[tv][4 * a + 3] * inv);
          w0 = (uint32_t)__builtin_bit_cast(uint16_t, e0) | ((uint32_t)__builtin_bit_cast(uint16_t, e1) << 16);
          w1 = (uint32_t)__builtin_bit_cast(uint16_t, e2) | ((uint32_t)__builtin_bit_cast(uint16_t, e3) << 16);
        }
        *(uint2*)(op + dv) = make_uint2(w0, w1);
      }
    }
    if (p.lse && g == 0) {
      p.lse[((int64_t)b * p.Hq + h) * S + qrow] = (m_run + log2f(l_tot)) * 0.6931471805599453f;
    }
  }
}

}  // namespace attn
