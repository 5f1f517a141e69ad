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
// (BF16 d_qk = 128: 8-wave workgroups, one per CU; measured 1.5-1.7% faster
// than two 4-wave ones on the 16K GQA layer, where FP8 is 0.2-1.8% slower)
using CfgBFD128 = FwdCfg<false, 128, 128, 32, 4, true, 2, 8>;
using CfgBFD192 = FwdCfg<false, 192, 128, 32, 4>;

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
  if (fp8 && pmode == kPLean)
    return d_qk == 128 ? launch_fwd<CfgF8D128, kPLean>(prm, stream) : launch_fwd<CfgF8D192, kPLean>(prm, stream);
  if (fp8)
    return d_qk == 128 ? launch_fwd<CfgF8D128, kPExact>(prm, stream) : launch_fwd<CfgF8D192, kPExact>(prm, stream);
  return d_qk == 128 ? launch_fwd<CfgBFD128, kPExact>(prm, stream) : launch_fwd<CfgBFD192, kPExact>(prm, stream);
}

}  // namespace attn
