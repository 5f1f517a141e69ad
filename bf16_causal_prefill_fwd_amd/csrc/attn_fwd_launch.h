// Attention kernel variants and their launch: (dtype, d_qk, d_v) -> tile
// configuration, grid size and the XCD work-order switch.
#pragma once

#include "attn_fwd_kernel.h"

namespace attn {

using CfgF8D128 = FwdCfg<true, 128, 128, 64, 4>;
// (FP8 d_qk = 192: the loop unrolled by the ring depth fits the 256
// registers of two waves per SIMD only with one MFMA job's operand reads in
// flight instead of two)
using CfgF8D192 = FwdCfg<true, 192, 128, 64, 4, true, 1>;
// FP8 d_qk = 192 with exact P in 8-wave workgroups, under the same switch as
// BF16 below: 1.0-1.5% faster on the 16K MLA layer on two boxes, outputs
// bitwise identical (its 12 KiB K tile takes one and a half load
// instructions per lane; FP8 d = 128 loses in 8 waves, 0.2-1.8%)
using CfgF8D192W8 = FwdCfg<true, 192, 128, 64, 4, true, 1, 8>;
using CfgBFD128 = FwdCfg<false, 128, 128, 32, 4>;
// BF16 d_qk = 128 in 8-wave workgroups (256 query rows, one per CU): half
// the K/V staging per FLOP. Measured 1.5-1.9% faster than two 4-wave ones on
// the 16K GQA layer and up to 4% from 16K to 64K tokens (FP8: 0.2-1.8%
// slower). It loses on short rows, where the taller tile's causal diagonal
// (every wave runs every step of its workgroup) outweighs the staging (+4%
// at 4K, +18% at 1K and 512 tokens, however many sequences), and on small
// grids (+39% at 1K tokens and 32 heads, B = 1). So it runs from 8K tokens,
// when its grid has at least 4 workgroups per CU of the 256. Its key step is
// 64 keys (the 4-wave form spills with 64 and keeps 32): another 1.2-3.2%
// from 8K to 64K tokens.
using CfgBFD128W8 = FwdCfg<false, 128, 128, 64, 4, true, 2, 8>;
constexpr int kWave8MinSeq = 8192;
constexpr int64_t kWave8MinWorkgroups = 1024;
using CfgBFD192 = FwdCfg<false, 192, 128, 32, 4>;
// BF16 d_qk = 192 in 8-wave workgroups under the same switch: 2.0% faster at
// 16K and 32K tokens (16 heads), 4.3% at 8K (32 heads), outputs bitwise
// identical (64-key steps spill here)
using CfgBFD192W8 = FwdCfg<false, 192, 128, 32, 4, true, 2, 8>;

enum LaunchStatus { kLaunched = 0, kTooManyWorkgroups = 1, kLaunchFailed = 2 };

// One workgroup per (batch, query head, query tile); the XCD-aware order
// needs the (batch, kv head) units to split evenly over the 8 XCDs.
template <class C, int PM>
inline LaunchStatus launch_fwd(FwdParams prm, hipStream_t stream) {
  prm.n_mtiles = (prm.S + C::BM - 1) / C::BM;
  const int64_t units = (int64_t)prm.B * prm.Hkv;
  const int64_t items = (int64_t)prm.B * prm.Hq * prm.n_mtiles;
  if (items > 0x7FFFFFFF) return kTooManyWorkgroups;
  prm.xcd_remap = (units % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL((attn_fwd_kernel<C, PM>), dim3((unsigned)items), dim3(C::NTHREADS), 0, stream, prm);
  return hipGetLastError() == hipSuccess ? kLaunched : kLaunchFailed;
}

// d_qk is 128 or 192 (d_v 128), pmode kPExact for BF16 and lse null for
// kPLean, checked by the caller.
inline LaunchStatus launch_attn_fwd(FwdParams prm, bool fp8, int d_qk, int pmode, hipStream_t stream) {
  if (fp8 && pmode == kPBlockScaled)
    return d_qk == 128 ? launch_fwd<CfgF8D128, kPBlockScaled>(prm, stream)
                       : launch_fwd<CfgF8D192, kPBlockScaled>(prm, stream);
  if (fp8 && pmode == kPBlockScaledRoundedSum)
    return d_qk == 128 ? launch_fwd<CfgF8D128, kPBlockScaledRoundedSum>(prm, stream)
                       : launch_fwd<CfgF8D192, kPBlockScaledRoundedSum>(prm, stream);
  if (fp8 && pmode == kPLean)
    return d_qk == 128 ? launch_fwd<CfgF8D128, kPLean>(prm, stream) : launch_fwd<CfgF8D192, kPLean>(prm, stream);
  // 8-wave workgroups (256 query rows) from kWave8MinSeq tokens when that
  // grid has at least kWave8MinWorkgroups of them
  const int64_t wg8 = (int64_t)prm.B * prm.Hq * ((prm.S + 255) / 256);
  const bool wave8 = prm.S >= kWave8MinSeq && wg8 >= kWave8MinWorkgroups;
  if (fp8 && d_qk == 128) return launch_fwd<CfgF8D128, kPExact>(prm, stream);
  if (fp8) return wave8 ? launch_fwd<CfgF8D192W8, kPExact>(prm, stream) : launch_fwd<CfgF8D192, kPExact>(prm, stream);
  if (d_qk == 192) return wave8 ? launch_fwd<CfgBFD192W8, kPExact>(prm, stream) : launch_fwd<CfgBFD192, kPExact>(prm, stream);
  return wave8 ? launch_fwd<CfgBFD128W8, kPExact>(prm, stream) : launch_fwd<CfgBFD128, kPExact>(prm, stream);
}

}  // namespace attn
