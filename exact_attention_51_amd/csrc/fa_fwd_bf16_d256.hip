// fa_fwd_bf16_d256.hip -- forward instance for D = 256 (one 32-row query
// block per wave, each tile's keys split between two waves, two-deep K/V
// ring, the workgroup's Q rows in LDS so that the 128 O accumulator
// registers and the rest fit the architectural VGPRs).
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

int launch_fwd_d256(const FwdArgs& a, hipStream_t stream);  // fa_fwd_d256.hip

// D = 256, and D = 160 with the same workgroup shape and LDS layout (96
// columns of each LDS row unused).  Without causal masking and from N = 64
// on, D = 256 runs the kernel with the assembly key loop (fa_fwd_d256.hip).
int launch_fwd_bf16_d256(const FwdArgs& a, hipStream_t stream) {
  if (a.D == 256 && !a.causal && a.N >= 64) return launch_fwd_d256(a, stream);
  if (a.D == 160) return a.causal ? fwd::launch<160, true, 1, 4>(a, stream) : fwd::launch<160, false, 1, 4>(a, stream);
  return a.causal ? fwd::launch<256, true, 1, 4>(a, stream) : fwd::launch<256, false, 1, 4>(a, stream);
}

}  // namespace fa
