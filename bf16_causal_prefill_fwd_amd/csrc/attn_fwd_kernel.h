// Causal prefill attention forward kernel for gfx950 (MI355X), FP8 e4m3 and BF16.
//
// The method (Le Fil IA, context paragraph; aicronaca.it, "Perché l'FP8 non
// basta da solo"; ai4bro.com, "Why is FP8 attention slow on MI355X?"): the
// two products Q.K^T and P.V run on the matrix cores, the row softmax between
// them runs on the vector ALU, tile by tile over the keys with a running row
// maximum and row sum; the vector work per tile is close to the matrix work,
// so the two have to overlap. This file is its MI355X design:
//
//  * One workgroup = 4 waves = 128 query rows of one (batch, head); each
//    wave owns 32 rows and keeps its Q fragment in registers. Two workgroups
//    share a CU, so each SIMD runs two independent waves. (BF16, and FP8 at
//    d_qk = 192, on long sequences: one workgroup of 8 waves = 256 rows per
//    CU, which halves the staging traffic per FLOP; the two waves of a SIMD
//    then share a barrier.)
//  * Software pipeline inside each wave, one key tile of BN keys per step
//    (64 for FP8 and for 8-wave BF16 at d = 128, 32 for the other BF16
//    forms): while the softmax of tile n runs on the vector ALU, the same wave
//    issues the MFMAs of S^T = K.Q^T for tile n+1 and of O^T += V^T.P^T for
//    tile n-1, interleaved with it in a fixed order, so both pipes stay busy
//    without relying on another wave's phase (the pages overlap the two
//    with a two-wave ping-pong: ai4bro.com, "How does ZYFA work?";
//    aicronaca.it, "Perché l'FP8 non basta da solo"). The LDS reads of the
//    MFMA operands run two MFMAs ahead. The step loop is unrolled by the
//    ring depth, so every LDS stage address is a constant offset.
//  * Key/value tiles go from HBM straight into LDS with coalesced 16-byte
//    global-to-LDS loads, into K and V rings of NSTAGE stages, issued
//    NSTAGE-1 steps before use; every wave waits only for its own loads
//    (vmcnt) before the barrier that publishes them, once per step.
//  * LDS rows are XOR-swizzled per tile kind so that every K read
//    (ds_read_b128, 16 lanes per LDS cycle) and every transposed V read
//    (ds_read_b64_tr_b8/_b16, 32 lanes per cycle) touches each bank once.
//  * S^T = K.Q^T is computed (K is the MFMA A operand), so each lane holds
//    scores of a single query: the row max needs one half-wave swap and the
//    row sum stays lane-local until the epilogue.
//  * O^T = V^T.P^T: P goes from the S^T accumulator straight into the B
//    operand (no shuffles); the key order inside the contraction is permuted
//    to match, and V is read in that order with LDS transpose reads, so V
//    stays row-major in LDS.
//  * Causal tile skip: a workgroup walks only key tiles up to its diagonal;
//    tiles that straddle a wave's diagonal or the sequence end are masked
//    (a tile wholly past a wave's rows is simply fully masked).
#pragma once

#include <type_traits>

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

template <bool FP8_, int DQK_, int DV_, int BN_, int NSTAGE_, bool STAGE_UNROLL_ = true, int LOOKAHEAD_ = 2,
          int NWAVES_ = 4>
struct FwdCfg {
  static constexpr bool FP8 = FP8_;
  static constexpr int DQK = DQK_, DV = DV_, BN = BN_;
  // two waves per SIMD: 4-wave workgroups two per CU, or 8-wave workgroups
  // one per CU (twice the query rows per K/V tile staged, but the two waves
  // of a SIMD meet at every barrier); each wave interleaves its MFMAs with
  // its own softmax
  static constexpr int NWAVES = NWAVES_;
  static constexpr int WG_PER_CU = 8 / NWAVES;
  static constexpr int BM = 32 * NWAVES;             // query rows per workgroup
  static constexpr int NTHREADS = NWAVES * 64;
  static constexpr int EB = FP8 ? 1 : 2;             // bytes per element
  static constexpr int KROW = DQK * EB;              // bytes per K row
  static constexpr int VROW = DV * EB;               // bytes per V row
  static constexpr int KCH = KROW / 16;              // 16-byte chunks per K row
  static constexpr int VCH = VROW / 16;
  static constexpr int KTILE = BN * KROW;
  static constexpr int VTILE = BN * VROW;
  static constexpr int NSTAGE = NSTAGE_;             // K ring and V ring depth
  // main loop unrolled by NSTAGE (every ring stage a constant LDS offset, no
  // per-step address arithmetic) rather than by 2 (the score parity only);
  // the longer loop body needs more registers (every configuration built
  // here takes the long one; the FP8 d_qk = 192 one with a look-ahead of 1)
  static constexpr bool STAGE_UNROLL = STAGE_UNROLL_;
  static constexpr int LOOKAHEAD = LOOKAHEAD_;      // MFMA jobs whose LDS operand reads are in flight
  // softmax chunks software-pipelined (exponentials one chunk ahead of their
  // use); measured 0.3% slower on a two-step loop
  static constexpr bool CHUNK_PIPE = STAGE_UNROLL;
  // folded score form available (the scaled MFMA exists for FP8 only)
  static constexpr bool FOLDABLE = FP8;
  static constexpr int LDS_BYTES = NSTAGE * (KTILE + VTILE);
  // the V ring (after the K ring) ends past the 16-bit ds_read offset
  static constexpr bool V_ABS = LDS_BYTES > 65536;
  static constexpr int NST = BN / 32;                // 32-key score tiles
  static constexpr int NOT = DV / 32;                // 32-wide output tiles
  static constexpr int QK_STEPS = FP8 ? DQK / 64 : DQK / 16;
  static constexpr int PV_STEPS = FP8 ? BN / 64 : BN / 16;   // key steps of one P.V output tile
  static constexpr int NPV = NOT * PV_STEPS;                 // P.V MFMAs per step
  static constexpr int NQK = NST * QK_STEPS;                 // Q.K^T MFMAs per step
  // 16-byte loads per lane per tile; a K tile that does not split evenly
  // over the workgroup (FP8 d_qk = 192 in 8 waves: 12 KiB over 8 KiB per
  // instruction) has a last instruction that only the first waves need: the
  // others load one line into a pad of their own, so every wave issues the
  // same loads and the vmcnt bookkeeping stays one constant
  static constexpr int KLOADS = (KTILE + 16 * NTHREADS - 1) / (16 * NTHREADS);
  static constexpr bool KPART = KTILE % (16 * NTHREADS) != 0;
  static constexpr int PAD_BYTES = KPART ? NWAVES * 1024 : 0;
  static constexpr int VLOADS = VTILE / 16 / NTHREADS;
  // loads a wave may leave in flight at the end of a step
  static constexpr int INFLIGHT = (NSTAGE - 2) * (KLOADS + VLOADS);
  static_assert((FP8 ? BN == 64 : (BN == 32 || BN == 64)), "FP8: 64 keys per step (one P operand); BF16: 32 or 64");
  static_assert(DV % 32 == 0 && DQK % 64 == 0, "head dims");
  static_assert(KTILE % 1024 == 0 && VTILE % (16 * NTHREADS) == 0, "staging split");
  static_assert(NSTAGE >= 2 && INFLIGHT < 64, "ring depth / vmcnt range");
  static_assert(!STAGE_UNROLL || NSTAGE % 2 == 0, "the stage index must carry the score parity");
  static_assert(NWAVES == 4 || NWAVES == 8, "two waves per SIMD");
  static_assert(WG_PER_CU * (LDS_BYTES + PAD_BYTES) <= 160 * 1024, "LDS of the workgroups of one CU");
};

// LDS swizzles: physical 16-byte chunk of logical chunk c in tile row r.
// Each is a bijection on a row's chunks and its own inverse (the staging
// loads use it to find which logical chunk lands in a physical slot), and it
// depends on r mod 16 only (every K read starts at a row that is a multiple
// of 32, every V read at a multiple of 16 (FP8) or 8 (BF16, whose V swizzle
// depends on r mod 4), so a lane's swizzle term is the same for every tile).
// The LDS serves 256 bytes per cycle: 16 lanes of a ds_read_b128, 32 lanes
// of an 8-byte read. The forms below make those lane groups hit distinct
// banks for the access patterns of this kernel (measured on MI355X: an
// earlier c ^ (r & 7) form made K reads 1.8x and V reads 1.6x slower).
//
// K tile (ds_read_b128 by rows 32t + lane%32): with a 128-byte row pitch
// rows r and r+1 share a 256-byte bank line, so the term must differ within
// every run of 16 rows.
template <int NCH>
__host__ __device__ constexpr int k_swz(int c, int r) {
  if constexpr (NCH == 8) {          // FP8 d=128: 128-byte rows
    return c ^ ((r >> 1) & 7);
  } else if constexpr (NCH == 12) {  // FP8 d=192: 192-byte rows, chunk quads
    return 4 * (c >> 2) + ((c & 3) ^ ((r >> 2) & 3));
  } else if constexpr (NCH == 16) {  // BF16 d=128: 256-byte rows
    return c ^ (r & 15);
  } else {                           // BF16 d=192: 384-byte rows, chunk octets
    static_assert(NCH == 24, "K row width");
    return 8 * (c >> 3) + ((c & 7) ^ ((r >> 1) & 7));
  }
}

// V tile (transposed reads: 8 keys x 16 bytes (FP8) or 4 keys x 32 bytes
// (BF16) per 16-lane group, two groups per LDS cycle reading adjacent
// chunks of the same keys).
template <int NCH>
__host__ __device__ constexpr int v_swz(int c, int r) {
  if constexpr (NCH == 8) {          // FP8 d_v=128: keys {0-3, 8-11} (+4) per group
    return c ^ (2 * ((r >> 1) & 1) + 4 * ((r >> 3) & 1));
  } else {                           // BF16 d_v=128: 4 consecutive keys per group
    static_assert(NCH == 16, "V row width");
    return c ^ (4 * (r & 3));
  }
}

template <class F>
constexpr bool swizzle_ok(F f, int nch) {
  for (int r = 0; r < 32; ++r) {
    bool seen[32] = {};
    for (int c = 0; c < nch; ++c) {
      const int ph = f(c, r);
      if (ph < 0 || ph >= nch || seen[ph]) return false;
      seen[ph] = true;
      if (f(ph, r) != c) return false;        // involution
      if (f(c, r + 16) != ph) return false;   // period 16 in the row
    }
  }
  return true;
}
static_assert(swizzle_ok([](int c, int r) { return k_swz<8>(c, r); }, 8) &&
              swizzle_ok([](int c, int r) { return k_swz<12>(c, r); }, 12) &&
              swizzle_ok([](int c, int r) { return k_swz<16>(c, r); }, 16) &&
              swizzle_ok([](int c, int r) { return k_swz<24>(c, r); }, 24),
              "K swizzles");
static_assert(swizzle_ok([](int c, int r) { return v_swz<8>(c, r); }, 8) &&
              swizzle_ok([](int c, int r) { return v_swz<16>(c, r); }, 16),
              "V swizzles");

// Workgroup -> (batch, query head, query tile).
__device__ __forceinline__ void decode_work(const FwdParams& p, int& b, int& h, int& mt) {
  const int bid = blockIdx.x;
  const int G = p.Hq / p.Hkv;
  if (p.xcd_remap) {
    // Workgroups are dispatched round-robin over the 8 XCDs (bid % 8). Give
    // each XCD whole (batch, kv-head) units so the G query heads and all
    // query tiles that re-read one head's K/V share that XCD's L2, and run
    // an XCD's units one after the other (longest, latest query tiles
    // first within a unit): the workgroups in flight on an XCD then stream
    // one head's K/V at a time, which its L2 can hold a good part of
    // (measured on the 32K MHA layer: 3x less L2-miss traffic than
    // interleaving the XCD's heads).
    const int xcd = bid & 7, j = bid >> 3;
    const int per_unit = p.n_mtiles * G;
    const int ul = j / per_unit, rem = j - ul * per_unit;
    const int tt = rem / G, gq = rem - tt * G;
    mt = p.n_mtiles - 1 - tt;
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

// Per-lane partial row sums above this trigger the exact-maximum path (see
// the softmax comment in the kernel). It keeps every probability <= 256,
// inside the e4m3 range (448), and far from fp32 overflow.
constexpr float kLazyMaxThreshold = 256.f;

// Scores as the MFMA hands them to the softmax. In both forms the softmax
// works on t = c * (q . k) - m in log2 units, with c = q_scale * k_scale *
// softmax_scale * log2(e) and m the running row maximum.
//  * kScaleFma: the MFMA gives q . k; one fma per score forms t.
//  * kScaleFolded (FP8, when c is a power of two 2^kc): the MFMA applies 2^kc
//    through its E8M0 operand scales and starts its accumulation from -m, so
//    it hands over t itself and the fma disappears from the softmax. The
//    input step can pick Q's per-tensor scale so that c is a power of two.
// f(integral_constant<int, I>) for I = B .. E-1, in order, while it returns true
template <int B, int E, class F>
__device__ __forceinline__ bool static_for_steps(F&& f) {
  if constexpr (B == E) {
    return true;
  } else {
    if (!f(std::integral_constant<int, B>{})) return false;
    return static_for_steps<B + 1, E>(f);
  }
}

enum ScoreForm { kScaleFma = 0, kScaleFolded = 1 };

// How probabilities reach the P.V MFMA.
//  * kPExact: P = e4m3 (FP8) or bf16 rounding of p, the exact exp2.
//  * kPBlockScaled (FP8): per (query row, 64-key block), P = e4m3(p * 2^kb)
//    with an integer kb >= 0, and the P.V MFMA multiplies its products by
//    2^-kb through the E8M0 operand scale of P, so O is unchanged up to the
//    rounding; small probabilities keep normal e4m3 precision instead of
//    falling into the subnormal range (aicronaca.it, "Perché l'FP8 non basta
//    da solo"; ai4bro.com, "How does ZYFA work?": power-of-two scaling of
//    each 64-key block of P, absorbed by the scaled MFMA).
//  * kPLean (FP8, O only: no LSE): Lean P (Le Fil IA, context paragraph;
//    aicronaca.it, "Perché l'FP8 non basta da solo"; ai4bro.com, "How does
//    ZYFA work?"). An e4m3 code read as an integer grows by 8 per doubling
//    of its value, so the code of p = 2^x is about 8x + 56 (1.0 is code 56,
//    linear within each binade): the scores come out of the Q.K^T MFMA
//    already as y = 8x + 56 + 8kb (the folded scale times 8, and a preset
//    accumulator), and one conversion per score rounds y to an integer and
//    clamps it to a byte, which is the e4m3 code fed to the P.V MFMA. No
//    exp2 runs. kb is an integer shift per (query row, 64-key block), taken
//    back by the P operand's E8M0 scale, that keeps every block's largest
//    code in (96, 104]; O is divided by the sum of the same rounded
//    probabilities, taken by one more MFMA (P times a block of ones).
enum PMode { kPExact = 0, kPBlockScaled = 1, kPLean = 2, kPBlockScaledRoundedSum = 3 };

// Lean P: a block's largest code is re-aimed into (kLeanTarget - 8,
// kLeanTarget] when it leaves [kLeanLow, kLeanHigh] (code 127 is a NaN, 128
// and up are negative); the shift stays within [-kMaxShift, kMaxShift]
// after rebasing the O reference by 2^64 when it goes below -kLeanRebase.
constexpr float kLeanTarget = 104.f, kLeanLow = 56.f, kLeanHigh = 126.f;
constexpr int kLeanRebase = 60;

// Largest block shift: 2^-kMaxShift stays a normal fp32 and 127 - kMaxShift
// a valid E8M0 scale.
constexpr int kMaxShift = 100;

template <class C, int FORM, int PM>
__device__ __forceinline__ void attn_fwd_body(const FwdParams& p, char* k_ring, char* v_ring, float vs,
                                              float c_log2, int kc) {
  const ATTN_LDS char* k_lds = (const ATTN_LDS char*)k_ring;
  const ATTN_LDS char* v_lds = (const ATTN_LDS char*)v_ring;
  const uint32_t k_lds_addr = lds_address(k_ring);
  const uint32_t v_lds_addr = lds_address(v_ring);
  constexpr bool FOLD = FORM == kScaleFolded;
  static_assert(!FOLD || C::FP8, "scale folding needs the scaled FP8 MFMA");
  constexpr bool PS = PM == kPBlockScaled || PM == kPBlockScaledRoundedSum;
  constexpr bool LEAN = PM == kPLean;
  // O divided by the sum of the rounded probabilities the P.V MFMAs take
  // (one more MFMA per step: P times a ones operand); Lean P always
  constexpr bool RSUM = LEAN || PM == kPBlockScaledRoundedSum;
  static_assert(!(LEAN && FOLD), "Lean P forms its codes with one fma per score: the fma form");
  static_assert(!(PS || RSUM) || C::FP8, "block-scaled P, Lean P and the rounded row sum need the FP8 MFMA");
  // scaled MFMAs (and the extra row-sum MFMA) are not matched by scheduling
  // groups: fences order the jobs
  constexpr bool FENCED = FOLD || PS || RSUM;

  constexpr int BN = C::BN, DV = C::DV, NS = C::NSTAGE;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int l32 = lane & 31;   // query column / operand row of this lane
  const int g = lane >> 5;     // contraction half
  const int hh = lane >> 4, kk = lane & 15;

  int b, h, mt;
  decode_work(p, b, h, mt);
  const int G = p.Hq / p.Hkv;
  const int kvh = h / G;
  const int S = p.S;
  const int m0 = mt * C::BM;
  const int r0 = m0 + 32 * wave;   // first row of this wave
  const int qrow = r0 + l32;

  // E8M0 operand scales of the folded form: 2^kc split over A and B
  // (each covers 2^-127 .. 2^127)
  const int kca = kc < -127 ? -127 : (kc > 127 ? 127 : kc);
  const int sc_a = 127 + kca, sc_b = 127 + (kc - kca);

  const int64_t q_row_stride = (int64_t)p.Hq * C::KROW;
  const int64_t k_row_stride = (int64_t)p.Hkv * C::KROW;
  const int64_t v_row_stride = (int64_t)p.Hkv * C::VROW;
  const uint8_t* kbase = p.k + ((int64_t)b * S * p.Hkv + kvh) * C::KROW;
  const uint8_t* vbase = p.v + ((int64_t)b * S * p.Hkv + kvh) * C::VROW;

  // ---- key tiles of the workgroup (every wave runs every step)
  const int n_kv = p.causal ? min(S, m0 + C::BM) : S;
  const int T = (n_kv + BN - 1) / BN;
  // a tile starting at key n0 needs the mask for this wave when n0 >
  // mask_after: causal, when it reaches past row r0 (n0 + BN - 1 > r0);
  // otherwise when it reaches past the sequence end (n0 + BN > S). Under the
  // causal mask a tile that crosses the sequence end always lies at or past
  // the first one that reaches past r0 (r0 < S, or the wave's rows are not
  // written at all).
  const int mask_after = p.causal ? r0 - BN + 1 : S - BN;

  // ---- Q fragment (B operand of S^T = K.Q^T), loaded once per wave
  constexpr int QREGS = C::FP8 ? 8 : 4;  // ints per k-step
  i32x4 qf[C::QK_STEPS * QREGS / 4];
  {
    const uint8_t* qp = p.q + ((int64_t)b * S + min(qrow, S - 1)) * q_row_stride + (int64_t)h * C::KROW;
#pragma unroll
    for (int u = 0; u < C::QK_STEPS; ++u) {
      if constexpr (C::FP8) {
        // bytes [64u + 32g, +32): chunks 4u + 2g, 4u + 2g + 1
        const int off = 64 * u + 32 * g;
        qf[2 * u] = *(const i32x4*)(qp + off);
        qf[2 * u + 1] = *(const i32x4*)(qp + off + 16);
      } else {
        // elements [16u + 8g, +8) = bytes [32u + 16g, +16)
        qf[u] = *(const i32x4*)(qp + 32 * u + 16 * g);
      }
    }
  }

  // ---- HBM -> LDS staging of tile `n` into ring stage n % NSTAGE:
  // instruction i of wave w fills stage bytes [(i*NWAVES + w)*1024, +1024);
  // lane l's 16 bytes are physical chunk (o % ROW)/16 of row o / ROW, so it
  // loads the logical chunk that the swizzle maps there. Keys past the end
  // are clamped to the last row (they are masked before use), and a tile
  // index past the workgroup's last tile loads that last tile again (into a
  // stage no step reads any more), so every step issues the same number of
  // loads and the vmcnt bookkeeping is a constant.
  // A lane's row within its 1 KB block and its swizzled chunk depend only on
  // the instruction, not on the tile, so each instruction's byte offset
  // within a tile is precomputed per lane (32-bit); the tile's base address
  // is wave-uniform and goes in a scalar register pair, so a load costs no
  // vector instruction. Only a tile that crosses the sequence end clamps
  // rows per lane.
  int k_loff[C::KLOADS], v_loff[C::VLOADS];
  const int k_stride32 = (int)k_row_stride, v_stride32 = (int)v_row_stride;
#pragma unroll
  for (int i = 0; i < C::KLOADS; ++i) {
    const int o = (i * C::NWAVES + wave) * 1024 + 16 * lane;
    const int row = o / C::KROW;
    k_loff[i] = o < C::KTILE ? row * k_stride32 + 16 * k_swz<C::KCH>((o % C::KROW) / 16, row) : 0;
  }
  // this wave's last K instruction past the tile: row 0 into its pad (after the K ring)
  const bool k_pad = C::KPART && ((C::KLOADS - 1) * C::NWAVES + wave) * 1024 >= C::KTILE;
  const uint32_t k_pad_addr = k_lds_addr + C::NSTAGE * C::KTILE + wave * 1024;
#pragma unroll
  for (int i = 0; i < C::VLOADS; ++i) {
    const int o = (i * C::NWAVES + wave) * 1024 + 16 * lane;
    const int row = o / C::VROW;
    v_loff[i] = row * v_stride32 + 16 * v_swz<C::VCH>((o % C::VROW) / 16, row);
  }
  // Only tiles from T_full on reach past the sequence end and clamp rows.
  // The scalar work per tile is kept small (it competes with the vector and
  // matrix instructions for the wave's issue slots): the tile's byte offset
  // is one 32 x 32 -> 64-bit product (BN * row stride fits 31 bits, checked
  // on the host), and the ring stage is a compile-time constant in the
  // unrolled loop, so each load's LDS address is this wave's ring base plus
  // a constant.
  const int T_full = S / BN;
  const int k_tile_bytes = BN * k_stride32, v_tile_bytes = BN * v_stride32;
  const uint32_t k_lds_w = k_lds_addr + wave * 1024, v_lds_w = v_lds_addr + wave * 1024;
  // Unchecked loads (CHECKc false) run in the loop's unchecked part, whose
  // tiles are all full and inside the sequence, one after the other: they
  // take the tile from a running pointer (`next`, advanced by one tile per
  // call) rather than from n.
  // (pad_last: this wave's last instruction goes to its pad)
  auto issue_tile = [&](const uint8_t* base, int tile_bytes, int stride, const int* loff, int nloads, int rowbytes,
                        uint32_t dst, int n, auto CHECKc, const uint8_t*& next, bool pad_last) {
    auto dst_of = [&](int i) -> uint32_t {
      return (i == nloads - 1 && pad_last) ? k_pad_addr : dst + i * C::NWAVES * 1024;
    };
    if constexpr (!decltype(CHECKc)::value) {
      const uint8_t* tb = next;
      next += tile_bytes;
#pragma unroll
      for (int i = 0; i < nloads; ++i) global_to_lds_16_async(tb, loff[i], dst_of(i));
      return;
    }
    const int nn = min(n, T - 1);
    const uint8_t* tb = base + (int64_t)nn * tile_bytes;
    if (nn < T_full) {
#pragma unroll
      for (int i = 0; i < nloads; ++i) global_to_lds_16_async(tb, loff[i], dst_of(i));
    } else {
#pragma unroll
      for (int i = 0; i < nloads; ++i) {
        if (i == nloads - 1 && pad_last) {
          global_to_lds_16_async(tb, 0, k_pad_addr);  // row 0 of the tile: inside the sequence
        } else {
          const int row = ((i * C::NWAVES + wave) * 1024 + 16 * lane) / rowbytes;
          const int key = min(nn * BN + row, S - 1);
          global_to_lds_16_async(tb, loff[i] + (key - nn * BN - row) * stride, dst + i * C::NWAVES * 1024);
        }
      }
    }
  };
  // tile n into ring stage `stage` (= n % NS)
  const uint8_t* k_next = kbase;  // next unchecked K / V tile
  const uint8_t* v_next = vbase;
  auto issue_k = [&](int n, int stage, auto CHECKc) {
    issue_tile(kbase, k_tile_bytes, k_stride32, k_loff, C::KLOADS, C::KROW, k_lds_w + stage * C::KTILE, n, CHECKc,
               k_next, k_pad);
  };
  auto issue_v = [&](int n, int stage, auto CHECKc) {
    issue_tile(vbase, v_tile_bytes, v_stride32, v_loff, C::VLOADS, C::VROW, v_lds_w + stage * C::VTILE, n, CHECKc,
               v_next, false);
  };

  // ---- per-lane LDS read offsets within a stage (the swizzle term depends
  // on row mod 16 only, which is fixed per lane for every tile below)
  // K (A operand): row 32t + l32, chunk pair of contraction step u
  int k_off[C::QK_STEPS][C::FP8 ? 2 : 1];
#pragma unroll
  for (int u = 0; u < C::QK_STEPS; ++u) {
    if constexpr (C::FP8) {
      k_off[u][0] = l32 * C::KROW + 16 * k_swz<C::KCH>(4 * u + 2 * g, l32);
      k_off[u][1] = l32 * C::KROW + 16 * k_swz<C::KCH>(4 * u + 2 * g + 1, l32);
    } else {
      k_off[u][0] = l32 * C::KROW + 16 * k_swz<C::KCH>(2 * u + g, l32);
    }
  }
  // V (A operand of O^T = V^T.P^T) through transpose reads. FP8: lane (dv row,
  // half g) byte j holds key 64u + 32(j/16) + 8((j%16)/4) + 4g + j%4, the key
  // that byte j of the P operand holds; the 16-lane group's 8 rows per read
  // are keys base + {0..3, 8..11}. BF16: element e holds key
  // 16u + 8(e/4) + 4g + e%4, rows base + {0..3}.
  int v_off[C::NOT];
  {
    const int krow_lane = C::FP8 ? (4 * (hh >> 1) + 8 * ((kk >> 1) >> 2) + ((kk >> 1) & 3))
                                 : (4 * (hh >> 1) + (kk >> 2));
#pragma unroll
    for (int tv = 0; tv < C::NOT; ++tv) {
      const int dv0 = 32 * tv + 16 * (hh & 1);
      const int ch = C::FP8 ? dv0 / 16 : dv0 / 8 + ((kk & 3) >> 1);
      v_off[tv] = krow_lane * C::VROW + 16 * v_swz<C::VCH>(ch, krow_lane) + 8 * (kk & 1);
      // V ring ending past 64 KiB: the lane's base holds the ring's address,
      // so each read's immediate carries only the stage and key offsets
      if constexpr (C::V_ABS) v_off[tv] = pin((int)v_lds_addr + v_off[tv]);
    }
  }

  // ---- running state
  f32x16 oacc[C::NOT];
#pragma unroll
  for (int t = 0; t < C::NOT; ++t) oacc[t] = f32x16{};
  // Running max of t (log2 units). Fma form: starting from a huge finite
  // negative (not -inf) keeps fma(s, c, -m) free of inf - inf, and the first
  // tile always takes the exact path because its sums overflow the
  // threshold. Folded form: the MFMA starts each score tile from cblk =
  // -m_run (16 copies, the shape of an accumulator), m_run starts at 0 and
  // the first tile is sent to the exact path explicitly.
  float m_run = FOLD ? 0.f : -1e30f;
  float l_run = 0.f;  // this lane's share of the running row sum
  f32x16 cblk = f32x16{};
  // Block-scaled P: kb_div = 2^-kb for the shift kb of the tile being
  // converted (the same for the two lanes of a query, which hold the two
  // halves of its 64-key block; kb_div is the divisor of the scaled
  // conversion), and by tile parity the E8M0 scale 127 - kb that the tile's
  // P.V MFMA applies, which is kb_div's exponent field. Each block's shift
  // comes from its own largest probability 2^lg (taken from its scores
  // before any of them is converted): kb = 7 - floor(lg), at least 0, maps
  // it into [128, 256), below the e4m3 maximum 448; a larger probability
  // (lg >= 8) takes kb = 0, and its block the exact path. fmed3 keeps
  // lg = -inf (every key of the block hidden from the lane's query) at the
  // largest shift, where its zeros stay zeros.
  float kb_div = 1.f;
  int e8[2] = {127, 127};
  // Lean P: the shift kb of the tile being converted and the code bias of
  // the scores (56 + 8 (kb - m_ref), m_ref the integer reference of O, so
  // the code of a score s is 8 c s + bias). Lean P and the rounded-sum
  // modes: the row sum of the rounded probabilities (every register of lacc
  // holds it).
  int kb = 0;
  float cbias = 0.f;
  f32x16 lacc = f32x16{};
  // e4m3 1.0 in every byte: the ones operand of the row-sum MFMA
  const i32x8 ones8 = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                       0x38383838, 0x38383838, 0x38383838, 0x38383838};
  auto set_shift = [&](float lg) {
    if constexpr (PS) kb_div = pow2i((int)__builtin_amdgcn_fmed3f(floorf(lg) - 7.f, (float)-kMaxShift, 0.f));
  };

  // Scores and P operands are double-buffered by tile parity: step n reads
  // the scores of tile n from sbuf[n&1] and writes tile n+1's into
  // sbuf[~n&1]; it reads the P operand of tile n-1 from pbuf[~n&1] and
  // writes tile n's into pbuf[n&1]. The loop is unrolled (by the ring depth,
  // or by two) so every index is a constant (no register copies between
  // steps).
  f32x16 sbuf[2][C::NST];
  constexpr int PREGS = C::FP8 ? 2 : C::PV_STEPS;   // FP8: 2 x i32x4 per 64 keys; BF16: one bf16x8 per 16 keys
  typedef typename std::conditional<C::FP8, i32x4, bf16x8>::type PVec;
  PVec pbuf[2][PREGS];
#pragma unroll
  for (int i = 0; i < PREGS; ++i) pbuf[1][i] = PVec{};

  // ---- matrix work of one step, as a list of MFMA jobs: P.V jobs (tile n-1)
  // then Q.K^T jobs (tile n+1), contraction step outermost so that two
  // consecutive MFMAs never accumulate into the same score tile.
  typedef typename std::conditional<C::FP8, i32x8, i32x4>::type Frag;
  auto frag_reads = [](int j) constexpr -> int {
    return j < C::NPV ? (C::FP8 ? 4 : 2) : (C::FP8 ? 2 : 1);
  };
  // A operand of job j (tile bases: vl for P.V, kl for Q.K^T)
  auto load_frag = [&](int j, const ATTN_LDS char* vl, const ATTN_LDS char* kl) -> Frag {
    Frag a;
    if (j < C::NPV) {
      const int tv = j % C::NOT, u = j / C::NOT;
      if constexpr (C::FP8) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int key0 = 64 * u + 32 * (rr >> 1) + 16 * (rr & 1);
          i32x2 x = C::V_ABS ? lds_read_tr8(lds_at((uint32_t)(v_off[tv] + (int)(vl - v_lds) + key0 * C::VROW)))
                             : lds_read_tr8(vl + key0 * C::VROW + v_off[tv]);
          a[2 * rr] = x[0];
          a[2 * rr + 1] = x[1];
        }
      } else {
        // two transposed reads of 4 elements each, concatenated (element e
        // of the operand is 16-bit lane e of the pair)
        const int so = (int)(vl - v_lds);
        const i32x2 x0 = __builtin_bit_cast(
            i32x2, C::V_ABS ? lds_read_tr16(lds_at((uint32_t)(v_off[tv] + so + (16 * u) * C::VROW)))
                            : lds_read_tr16(vl + (16 * u) * C::VROW + v_off[tv]));
        const i32x2 x1 = __builtin_bit_cast(
            i32x2, C::V_ABS ? lds_read_tr16(lds_at((uint32_t)(v_off[tv] + so + (16 * u + 8) * C::VROW)))
                            : lds_read_tr16(vl + (16 * u + 8) * C::VROW + v_off[tv]));
        a = i32x4{x0[0], x0[1], x1[0], x1[1]};
      }
    } else {
      const int jq = j - C::NPV, t = jq % C::NST, u = jq / C::NST;
      const ATTN_LDS char* kr = kl + 32 * t * C::KROW;
      if constexpr (C::FP8) {
        i32x4 a0 = lds_read_b128(kr + k_off[u][0]);
        i32x4 a1 = lds_read_b128(kr + k_off[u][1]);
        a = i32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      } else {
        a = lds_read_b128(kr + k_off[u][0]);
      }
    }
    return a;
  };
  // job j: P.V jobs accumulate into oacc with operand P = pbuf[PP]; Q.K^T
  // jobs write the score tiles sbuf[SQ]
  auto run_job = [&](int j, const Frag& a, auto PPc, auto SQc) {
    constexpr int PP = decltype(PPc)::value, SQ = decltype(SQc)::value;
    const PVec* pv = pbuf[PP];
    f32x16* sq = sbuf[SQ];
    if (j < C::NPV) {
      const int tv = j % C::NOT, u = j / C::NOT;
      if constexpr (C::FP8) {
        i32x8 pop = {pv[0][0], pv[0][1], pv[0][2], pv[0][3], pv[1][0], pv[1][1], pv[1][2], pv[1][3]};
        oacc[tv] = (PS || LEAN) ? mfma_f8_scaled(a, pop, oacc[tv], 127, e8[PP]) : mfma_f8(a, pop, oacc[tv]);
        if constexpr (RSUM) {
          if (j == 0) lacc = mfma_f8_scaled(ones8, pop, lacc, 127, e8[PP]);
        }
      } else {
        oacc[tv] = mfma_bf16(__builtin_bit_cast(bf16x8, a), pv[u], oacc[tv]);
      }
    } else {
      const int jq = j - C::NPV, t = jq % C::NST, u = jq / C::NST;
      const f32x16 acc = u == 0 ? (FOLD ? cblk : f32x16{}) : sq[t];
      if constexpr (C::FP8) {
        i32x8 bq = {qf[2 * u][0], qf[2 * u][1], qf[2 * u][2], qf[2 * u][3],
                    qf[2 * u + 1][0], qf[2 * u + 1][1], qf[2 * u + 1][2], qf[2 * u + 1][3]};
        sq[t] = FOLD ? mfma_f8_scaled(a, bq, acc, sc_a, sc_b) : mfma_f8(a, bq, acc);
      } else {
        sq[t] = mfma_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, qf[u]), acc);
      }
    }
  };

  // ---- softmax of one tile, in NCHUNK chunks (interleaved with the MFMA
  // jobs). Log2 domain, exact exp2, P rounded to the operand type.
  // Probabilities are taken against the running max m_run as it stands
  // (p = 2^(c*s - m_run)); the row max is only recomputed when some lane's
  // partial sum of a tile exceeds the threshold, i.e. when the scores have
  // grown well past m_run (always on the first tile). Every p then stays
  // <= 256, and the result is the same softmax: m only shifts the common
  // factor that O and l share.
  // Fma form: t = fma(s, c, -m). Folded form: the score is t already, less
  // `m` on the exact path (m = the increase of the running max).
  constexpr int NCHUNK = C::NST * 4;              // 4 fp32 scores per lane each
  auto log2_prob = [&](float s, float m, auto SHIFTc) -> float {
    if constexpr (!FOLD) return __builtin_fmaf(s, c_log2, -m);
    else if constexpr (decltype(SHIFTc)::value) return s - m;
    else return s;
  };
  // A chunk in two parts: its four exponentials, then their use (the row
  // sum and the operand pack).
  auto chunk_exp = [&](int c, auto Pc, float m, auto SHIFTc, float* pe) {
    constexpr int P = decltype(Pc)::value;
    const f32x16* sc = sbuf[P];
    // chunk c: score tile t = c / 4, registers r .. r+3
    const int t = c >> 2, r = 4 * (c & 3);
#pragma unroll
    for (int i = 0; i < 4; ++i) pe[i] = fast_exp2(log2_prob(sc[t][r + i], m, SHIFTc));
  };
  auto chunk_use = [&](int c, auto Pc, const float* pe, float& lsum) {
    constexpr int P = decltype(Pc)::value;
    PVec* pout = pbuf[P];
    const int t = c >> 2, r = 4 * (c & 3);
    const float p0 = pe[0], p1 = pe[1], p2 = pe[2], p3 = pe[3];
    // (the first chunk starts the sum: adding it to 0 would cost an add)
    const float s4 = (p0 + p1) + (p2 + p3);
    lsum = c == 0 ? s4 : lsum + s4;
    if constexpr (C::FP8) {
      // FP8 operand byte j <- score tile j/16, register j%16: chunk c fills
      // dword (c & 3) of pout[t]
      // (both halves are written: the register's old contents only save an
      // instruction that would clear it)
      if constexpr (PS) {
        const int x = cvt_fp8x2_div(p0, p1, kb_div, pout[t][c & 3], false);
        pout[t][c & 3] = pin(cvt_fp8x2_div(p2, p3, kb_div, x, true));
      } else {
        const int x = cvt_fp8x2(p0, p1, pout[t][c & 3], false);
        pout[t][c & 3] = pin(cvt_fp8x2(p2, p3, x, true));
      }
    } else {
      // BF16 operand u = 2t + (r / 8) holds registers 8(u%2) .. +7 of tile t
      const int u = 2 * t + (r >> 3), e = r & 7;
      pout[u][e] = (__bf16)p0;
      pout[u][e + 1] = (__bf16)p1;
      pout[u][e + 2] = (__bf16)p2;
      pout[u][e + 3] = (__bf16)p3;
    }
  };
  // Lean P chunk c: four scores to four codes (the code-unit score by one
  // fma, then round to nearest even and clamp to [0, 255]; -inf, a hidden
  // key, gives 0), packed into dword c & 3 of the score tile's P operand
  const float c8 = 8.f * c_log2;
  auto lean_chunk = [&](int c, auto Pc) {
    constexpr int P = decltype(Pc)::value;
    const f32x16* sc = sbuf[P];
    PVec* pout = pbuf[P];
    const int t = c >> 2, r = 4 * (c & 3);
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) w = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(sc[t][r + i], c8, cbias), i, w);
    pout[t][c & 3] = pin((int)w);
  };
  auto probs_chunk = [&](int c, auto Pc, float m, float& lsum, auto SHIFTc) {
    float pe[4];
    chunk_exp(c, Pc, m, SHIFTc, pe);
    chunk_use(c, Pc, pe, lsum);
  };

  // exact-maximum path for a tile whose partial sums overflowed (or, folded
  // form, the first tile): new row max, rescale of l and O (O holds every
  // P.V issued so far), P again. Q is the parity of the next tile's scores,
  // which the folded form computed against the old max.
  using False_ = std::integral_constant<bool, false>;
  using True_ = std::integral_constant<bool, true>;
  auto exact_path = [&](auto Pc, float& lsum, bool first) {
    constexpr int P = decltype(Pc)::value, Q = 1 - P;
    const f32x16* sc = sbuf[P];
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < C::NST; ++t) mx = max16(sc[t], mx);
    mx = fmaxf(mx, swap_halves(mx));
    // (block-scaled P: the block's largest probability after the update is
    // 2^lg, lg <= 0)
    if constexpr (!FOLD) {
      const float m_new = fmaxf(m_run, mx * c_log2);
      const float alpha = fast_exp2(m_run - m_new);
      set_shift(mx * c_log2 - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < C::NOT; ++t) oacc[t] *= alpha;
      if constexpr (RSUM) lacc *= alpha;
#pragma unroll
      for (int c = 0; c < NCHUNK; ++c) probs_chunk(c, Pc, m_run, lsum, False_{});
    } else {
      // scores are t = c*s - m_run: the max grows by d = max(mx, 0) (on the
      // first tile, where nothing is accumulated yet, it is set to mx; a row
      // always sees key 0 there, so mx is finite)
      const float d = first ? mx : fmaxf(mx, 0.f);
      const float alpha = first ? 0.f : fast_exp2(-d);
      set_shift(mx - d);
      m_run += d;
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < C::NOT; ++t) oacc[t] *= alpha;
      if constexpr (RSUM) lacc *= alpha;
#pragma unroll
      for (int i = 0; i < 16; ++i) cblk[i] = -m_run;
#pragma unroll
      for (int t = 0; t < C::NST; ++t) sbuf[Q][t] -= d;
#pragma unroll
      for (int c = 0; c < NCHUNK; ++c) probs_chunk(c, Pc, d, lsum, True_{});
    }
  };

  constexpr int NJOB = C::NPV + C::NQK;
  // Issue order of the step's jobs (job numbers: P.V 0..NPV-1, Q.K^T
  // NPV..NJOB-1). With one score tile per step (BF16) every Q.K^T job
  // accumulates into the same tile, so P.V and Q.K^T jobs alternate to keep
  // two dependent MFMAs apart; otherwise P.V jobs come first.
  constexpr bool ALTERNATE = C::NST == 1 && C::NPV == C::NQK;
  auto job_at = [](int pos) constexpr -> int {
    return ALTERNATE ? ((pos & 1) ? C::NPV + (pos >> 1) : (pos >> 1)) : pos;
  };
  // ---- one pipeline step n. M: n % NS when the loop is unrolled by NS
  // (then every LDS stage address is a constant offset), else n % 2 (M = -1,
  // stage addresses computed). The parity P = n & 1 says where tile n's
  // scores are (sbuf[P]). FIRST: n == 0.
  auto step = [&](int n, auto Mc, auto FIRSTc, auto CHECKc) {
    constexpr int M = decltype(Mc)::value;
    constexpr bool FIRST = decltype(FIRSTc)::value;
    constexpr bool CONST_STAGE = C::STAGE_UNROLL;
    constexpr int P = M & 1, Q = 1 - P;
    using Pc = std::integral_constant<int, P>;
    const int n0 = n * BN;
    // mask (wave-uniform branch: tiles that straddle this wave's diagonal,
    // lie wholly past its rows, or cross the sequence end)
    if (n0 > mask_after) {
#pragma unroll
      for (int t = 0; t < C::NST; ++t) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = n0 + 32 * t + 8 * (r >> 2) + 4 * g + (r & 3);
          const bool hidden = p.causal ? (key > qrow || key >= S) : (key >= S);
          sbuf[P][t][r] = hidden ? -INFINITY : sbuf[P][t][r];
        }
      }
    }
    // Lean P: the block's largest code, from its largest score; the lanes
    // whose block left the band (all on the first tile) re-aim it by a
    // whole number of binades, which moves the code bias of this tile and
    // the ones after it, and kb (on the first tile the shift instead sets
    // the reference of O). Branch-free: the bias enters every code through
    // the fma that forms it.
    if constexpr (LEAN) {
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < C::NST; ++t) mx = max16(sbuf[P][t], mx);
      mx = fmaxf(mx, swap_halves(mx));
      const float ymax = __builtin_fmaf(mx, c8, cbias);
      const bool off = ymax > -1e30f && (FIRST || !(ymax >= kLeanLow && ymax <= kLeanHigh));
      int dlt = (int)floorf((kLeanTarget - (off ? ymax : kLeanTarget)) * 0.125f);
      if (!FIRST) dlt = min(dlt, kMaxShift - kb);
      cbias += 8.f * (float)dlt;
      if (!FIRST) kb += dlt;
      // scores far above the reference: rebase O by 2^-64 (exact)
      if (wave_any(kb < -kLeanRebase)) {
        const float f = kb < -kLeanRebase ? 0x1p-64f : 1.f;
#pragma unroll
        for (int t = 0; t < C::NOT; ++t) oacc[t] *= f;
        lacc *= f;
        kb += kb < -kLeanRebase ? 64 : 0;
      }
    }
    // block-scaled P: the shift of tile n from its largest score
    if constexpr (PS) {
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < C::NST; ++t) mx = max16(sbuf[P][t], mx);
      mx = fmaxf(mx, swap_halves(mx));
      set_shift(FOLD ? mx : mx * c_log2 - m_run);
    }
    // V(n-1) sits in stage (n-1) % NS; at n = 0 P is zero and stage 0 (V(0)) is read
    const int vst = FIRST ? 0 : (CONST_STAGE ? (M + NS - 1) % NS : (n - 1) % NS);
    const int kst = CONST_STAGE ? (M + 1) % NS : (n + 1) % NS;
    const ATTN_LDS char* vl = v_lds + vst * C::VTILE;
    const ATTN_LDS char* kl = k_lds + kst * C::KTILE;
    // MFMA jobs interleaved with the softmax chunks of tile n; job j's LDS
    // reads go out LOOKAHEAD jobs ahead (a ring of LOOKAHEAD + 1 operands)
    float lsum = 0.f;
    constexpr int LA = C::LOOKAHEAD;
    Frag fr[LA + 1];
    int reads0 = 0;
#pragma unroll
    for (int j = 0; j < LA; ++j) {
      fr[j] = load_frag(job_at(j), vl, kl);
      reads0 += frag_reads(job_at(j));
    }
    sched_group<kSchedDsRead>(reads0);
    int c = 0;
    // CHUNK_PIPE: the exponentials of chunk c + 1 go out with the use of
    // chunk c, so no pack or add waits on a just-issued exp2
    float pe[2][4];
    if (C::CHUNK_PIPE && !LEAN) chunk_exp(0, Pc{}, m_run, False_{}, pe[0]);
#pragma unroll
    for (int j = 0; j < NJOB; ++j) {
      if (j + LA < NJOB) fr[(j + LA) % (LA + 1)] = load_frag(job_at(j + LA), vl, kl);
      // chunks are spread evenly over the jobs, each ahead of its job's
      // MFMA: the first one covers the latency of the step's first operand
      // reads, and the last MFMA runs on while the wave waits at the barrier
      const int c_end = (j + 1) * NCHUNK / NJOB;
      for (; c < c_end; ++c) {
        if constexpr (LEAN) {
          lean_chunk(c, Pc{});
        } else if (C::CHUNK_PIPE) {
          if (c + 1 < NCHUNK) chunk_exp(c + 1, Pc{}, m_run, False_{}, pe[(c + 1) & 1]);
          chunk_use(c, Pc{}, pe[c & 1], lsum);
        } else {
          probs_chunk(c, Pc{}, m_run, lsum, False_{});
        }
      }
      if constexpr (FENCED) sched_fence();
      run_job(job_at(j), fr[j % (LA + 1)], std::integral_constant<int, Q>{}, std::integral_constant<int, Q>{});
      // this step's loads (K(n+NS), V(n+NS-2)) go out behind the first MFMA,
      // so their address arithmetic overlaps the softmax
      if (j == 0) {
        issue_k(n + NS, CONST_STAGE ? M : n % NS, CHECKc);
        issue_v(n + NS - 2, CONST_STAGE ? (M + NS - 2) % NS : (n + NS - 2) % NS, CHECKc);
      }
      // issue order: this job's look-ahead reads, then its MFMA. Fma form:
      // the softmax instructions are left to the scheduler (pinning them
      // measured slower). Folded form: the scaled MFMA is not matched by
      // scheduling groups, so fences keep each job's chunk ahead of its MFMA
      if constexpr (FENCED) {
        sched_fence();
      } else {
        if (j + LA < NJOB) sched_group<kSchedDsRead>(frag_reads(job_at(j + LA)));
        sched_group<kSchedMfma>(1);
      }
    }
    wait_vmcnt<C::INFLIGHT>();
    __syncthreads();
    // lazy-max check of tile n after the barrier, by when its row sums are
    // complete (the exact path touches registers only)
    if constexpr (LEAN) {
      e8[P] = 127 - kb;  // for tile n's P.V in step n + 1
    } else {
      const bool first = FOLD && FIRST;
      if (wave_any(first | !(lsum <= kLazyMaxThreshold))) exact_path(Pc{}, lsum, first);
      l_run += lsum;
      if constexpr (PS) e8[P] = __float_as_int(kb_div) >> 23;  // 127 - kb, for tile n's P.V in step n + 1
    }
  };

  // ---- prologue: stages of K(0..NS-1) and V(0..NS-3) in flight, then all
  // published; S^T of tile 0 into sbuf[0].
#pragma unroll
  for (int n = 0; n < NS; ++n) issue_k(n, n, True_{});
#pragma unroll
  for (int n = 0; n < NS - 2; ++n) issue_v(n, n, True_{});
  wait_vmcnt<0>();
  __syncthreads();
#pragma unroll
  for (int j = C::NPV; j < NJOB; ++j)
    run_job(j, load_frag(j, v_lds, k_lds), std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{});
  // step 0 loads K(NS) into stage 0, which every wave has just read
  __syncthreads();

  // ---- main loop. Step n: S^T of tile n+1 and O += P.V of tile n-1 on the
  // matrix cores while the softmax of tile n runs; K(n+NS) and V(n+NS-2) are
  // loaded meanwhile (their stages were last read in step n-1). At the end
  // each wave waits for all but the last NS-2 steps' loads, so K(n+2) and
  // V(n) are complete at the barrier.
  step(0, std::integral_constant<int, 0>{}, True_{}, True_{});
  if constexpr (C::STAGE_UNROLL) {
    int n = 1;
    // iterations whose NS steps all exist (n + NS - 1 < T; under the causal
    // mask T can be far below T_full) and that load only tiles ending inside
    // the sequence (K up to n + 2NS - 1, V up to n + 2NS - 3, all < T_full):
    // their loads need no clamping and no test for it. A loaded tile past
    // the workgroup's last one (index T or more) goes to a stage no step
    // reads, as the clamped reloads of the checked path do.
    k_next = kbase + (int64_t)(n + NS) * k_tile_bytes;
    v_next = vbase + (int64_t)(n + NS - 2) * v_tile_bytes;
    for (; n + NS <= T && n + 2 * NS - 1 < T_full; n += NS) {
      static_for_steps<0, NS>([&](auto Ic) {
        constexpr int i = decltype(Ic)::value;
        step(n + i, std::integral_constant<int, (1 + i) % NS>{}, False_{}, False_{});
        return true;
      });
    }
    for (; n < T; n += NS) {
      const bool more = static_for_steps<0, NS>([&](auto Ic) {
        constexpr int i = decltype(Ic)::value;
        if (n + i >= T) return false;
        step(n + i, std::integral_constant<int, (1 + i) % NS>{}, False_{}, True_{});
        return true;
      });
      if (!more) break;
    }
  } else {
    int n = 1;
    // unchecked part as above, two steps per iteration (K up to n + 1 + NS)
    k_next = kbase + (int64_t)(n + NS) * k_tile_bytes;
    v_next = vbase + (int64_t)(n + NS - 2) * v_tile_bytes;
    for (; n + 2 <= T && n + 1 + NS < T_full; n += 2) {
      step(n, std::integral_constant<int, 1>{}, False_{}, False_{});
      step(n + 1, std::integral_constant<int, 0>{}, False_{}, False_{});
    }
    for (; n < T; n += 2) {
      step(n, std::integral_constant<int, 1>{}, False_{}, True_{});
      if (n + 1 >= T) break;
      step(n + 1, std::integral_constant<int, 0>{}, False_{}, True_{});
    }
  }
  // last tile T-1: its lazy-max check, then its P.V (V stage complete: waited
  // at the end of step T-2)
  {
    const ATTN_LDS char* vl = v_lds + ((T - 1) % NS) * C::VTILE;
    auto finish = [&](auto Pc) {
      constexpr int P = decltype(Pc)::value;
#pragma unroll
      for (int j = 0; j < C::NPV; ++j)
        run_job(j, load_frag(j, vl, k_lds), Pc, std::integral_constant<int, 1 - P>{});
    };
    if ((T - 1) & 1) finish(std::integral_constant<int, 1>{});
    else finish(std::integral_constant<int, 0>{});
  }
  wait_vmcnt<0>();  // drain the loads of the last steps before the workgroup ends

  // ---- epilogue: O = O_acc * v_scale / l, LSE = ln2 * (m + log2 l), with
  // l the fp32 sum of the exact exponentials over both key halves; O is
  // divided instead by the rounded probabilities' row sum where that is kept
  // (Lean P has no other)
  const float l_tot = LEAN ? lacc[0] : l_run + swap_halves(l_run);
  const float inv = vs / (RSUM ? lacc[0] : l_tot);
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
    if (!LEAN && p.lse && g == 0) {
      p.lse[((int64_t)b * p.Hq + h) * S + qrow] = (m_run + log2f(l_tot)) * 0.6931471805599453f;
    }
  }
}

template <class C, int PM>
__global__ __launch_bounds__(C::NTHREADS, C::WG_PER_CU) void attn_fwd_kernel(FwdParams p) {
  __shared__ __attribute__((aligned(1024))) char k_ring[C::NSTAGE * C::KTILE + C::PAD_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_ring[C::NSTAGE * C::VTILE];
  float qs = p.q_scale, ks = p.k_scale, vs = p.v_scale;
  if (p.d_scales) {
    qs = p.d_scales[0];
    ks = p.d_scales[1];
    vs = p.d_scales[2];
  }
  // scores in log2 units: t = c * (q . k)
  const float c_log2 = qs * ks * p.sm_scale * 1.4426950408889634f;
  // (Lean P and the rounded-sum modes take the fma form only: with the
  // folded form's -m block their extra registers do not fit)
  if constexpr (C::FOLDABLE && PM != kPLean && PM != kPBlockScaledRoundedSum) {
    // c = f * 2^e, f in [0.5, 1): a power of two up to fp32 rounding of the
    // scale product (a relative 2^-18 covers it many times over)
    int e;
    const float f = frexpf(c_log2, &e);
    const bool pow2 = fabsf(f - 0.5f) <= 0x1p-19f || fabsf(f - 1.0f) <= 0x1p-18f;
    if (uniform(pow2 ? 1 : 0)) {
      attn_fwd_body<C, kScaleFolded, PM>(p, k_ring, v_ring, vs, c_log2, uniform(f < 0.75f ? e - 1 : e));
      return;
    }
  }
  attn_fwd_body<C, kScaleFma, PM>(p, k_ring, v_ring, vs, c_log2, 0);
}

}  // namespace attn
