// fa_fwd_bf16.hip -- forward instances for D = 64 and D = 128 and the
// dispatch over head dimensions (the D = 256 instance lives in its own
// translation unit, fa_fwd_bf16_d256.hip, built with different flags).
#include "fa_fwd_bf16.h"

namespace fa {
namespace fwd {

template <int D, bool CAUSAL, int QB, int W>
int launch(const FwdArgs& a, hipStream_t stream) {
  using C = FwdCfg<D, QB, W>;
  const int n_qtiles = (a.N + C::kBlockM - 1) / C::kBlockM;
  const TileSched sched = make_sched(n_qtiles, a.B * a.H, CAUSAL);
  const long grid = (long)n_qtiles * a.B * a.H;
  if (a.N < 64)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, QB, W, true>), dim3((unsigned)grid), dim3(64 * W), 0, stream, a, sched);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, QB, W, false>), dim3((unsigned)grid), dim3(64 * W), 0, stream, a, sched);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace fwd

int launch_fwd_bf16_d256(const FwdArgs& a, hipStream_t stream);
int launch_fwd_d64(const FwdArgs& a, hipStream_t stream);  // fa_fwd_d64.hip

// Query blocks of 32 rows per wave, and waves per workgroup by head
// dimension: at D = 128 one 8-wave workgroup per CU (two waves per SIMD;
// the K/V ring takes 128 KB of LDS), at D = 64 three 4-wave workgroups per
// CU, which do not share barriers and so drift into complementary phases
// (the D = 64 step is bound by its VALU work).  At D = 128 (and 96) a grid
// of fewer 256-row workgroups than CUs takes 4-wave, 128-row workgroups
// instead: twice the workgroups, one wave on each SIMD of twice the CUs.
// Under causal masking (uneven blocks) this pays up to twice as many
// 256-row blocks as CUs; measured on one MI355X: B=2 H=4 N=2048, 54 -> 39 us
// with and without the mask, B=1 H=8 N=8192 causal 210 -> 182 us, while
// non-causal grids of 256..511 blocks lose (B=1 H=8 N=8192: 263 -> 310 us).
int launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  constexpr int QB = 1, W64 = 4, W128 = 8;
  if (a.D == 128 || a.D == 96 || a.D == 64) {
    const long blocks = (long)((a.N + 255) / 256) * a.B * a.H;
    const int cus = device_cus();
    const bool small = blocks < cus || (a.causal && blocks < 2 * cus);
    if (a.D == 64) {
      if (!small && a.N >= 64) return launch_fwd_d64(a, stream);  // 64 rows per wave, assembly key loop
      return a.causal ? fwd::launch<64, true, QB, W64>(a, stream) : fwd::launch<64, false, QB, W64>(a, stream);
    }
    if (small) {
      if (a.D == 128)
        return a.causal ? fwd::launch<128, true, QB, 4>(a, stream) : fwd::launch<128, false, QB, 4>(a, stream);
      return a.causal ? fwd::launch<96, true, QB, 4>(a, stream) : fwd::launch<96, false, QB, 4>(a, stream);
    }
  }
  if (a.D == 32)  // the D = 64 workgroup shape and LDS layout, 32 columns unused
    return a.causal ? fwd::launch<32, true, QB, W64>(a, stream) : fwd::launch<32, false, QB, W64>(a, stream);
  if (a.D == 128) {
    if (a.N >= 64) return launch_fwd_d128(a, stream);  // 64 rows per wave, assembly key loop
    return a.causal ? fwd::launch<128, true, QB, W128>(a, stream) : fwd::launch<128, false, QB, W128>(a, stream);
  }
  if (a.D == 96)  // the D = 128 workgroup shape and LDS layout, 32 columns unused
    return a.causal ? fwd::launch<96, true, QB, W128>(a, stream) : fwd::launch<96, false, QB, W128>(a, stream);
  if (a.D == 256 || a.D == 160) return launch_fwd_bf16_d256(a, stream);
  return -2;
}

}  // namespace fa
