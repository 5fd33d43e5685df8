// fa_fwd_kv_d256.hip -- the D = 256 instance of the forward with query and
// key lengths apart and split key ranges (see fa_fwd_kv.hip); workgroup
// shape as for the square D = 256 forward.
#include "fa_fwd_bf16.h"

namespace fa {
namespace fwd {

template <int D, bool CAUSAL>
int launch_kv_d256(const FwdArgs& a, hipStream_t stream) {
  using C = FwdCfg<D, 1, 4>;
  const int n_qtiles = (a.N + C::kBlockM - 1) / C::kBlockM;
  const TileSched sched = make_sched(n_qtiles * a.n_split, a.B * a.H, CAUSAL);
  const long grid = (long)n_qtiles * a.n_split * a.B * a.H;
  if (a.Nk < 64)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, 1, 4, true, true>), dim3((unsigned)grid), dim3(256), 0, stream,
                       a, sched);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, 1, 4, false, true>), dim3((unsigned)grid), dim3(256), 0, stream,
                       a, sched);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace fwd

// D = 256, and D = 160 with the same workgroup shape and LDS layout.
int launch_fwd_bf16_kv_d256(const FwdArgs& a, hipStream_t stream) {
  if (a.D == 160) return a.causal ? fwd::launch_kv_d256<160, true>(a, stream) : fwd::launch_kv_d256<160, false>(a, stream);
  return a.causal ? fwd::launch_kv_d256<256, true>(a, stream) : fwd::launch_kv_d256<256, false>(a, stream);
}

}  // namespace fa
