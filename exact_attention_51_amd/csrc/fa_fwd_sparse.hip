// fa_fwd_sparse.hip -- block-sparse forward instances for D = 32, 64, 96,
// 128, 160 and 256.  The 256-wide layout (D = 160, 256) fills all 160 KB of
// LDS with its K/V ring and Q rows in the square kernel; its block-sparse
// instances keep the Q rows in registers instead, which frees the LDS for
// the tile list.
//
// The causal tile skip generalised: a block mask over (64-row query block,
// 64-key block) pairs says which key tiles a query block reads, and each
// workgroup builds the list of the tiles any of its rows may see before
// its loop (see the SPARSE parts of fa_fwd_bf16.h).  The metal-flash-
// attention README names block sparsity as the natural extension of the
// tile skip; the "Flash Attention" page's kernel anatomy is the tile skip
// itself.
#include "fa_fwd_bf16.h"

namespace fa {
namespace fwd {

template <int D, bool CAUSAL, int QB, int W>
int launch_sparse(const FwdArgs& a, hipStream_t stream) {
  using C = FwdCfg<D, QB, W, true>;
  const int n_qtiles = (a.N + C::kBlockM - 1) / C::kBlockM;
  const TileSched sched = make_sched(n_qtiles, a.B * a.H, CAUSAL);
  const long grid = (long)n_qtiles * a.B * a.H;
  if (a.N < 64)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, QB, W, true, false, true>), dim3((unsigned)grid), dim3(64 * W), 0,
                       stream, a, sched);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, QB, W, false, false, true>), dim3((unsigned)grid), dim3(64 * W), 0,
                       stream, a, sched);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace fwd

// Workgroup shapes as for the square forward (fa_fwd_bf16.hip).
int launch_fwd_bf16_sparse(const FwdArgs& a, hipStream_t stream) {
  if (a.D == 64)
    return a.causal ? fwd::launch_sparse<64, true, 1, 4>(a, stream) : fwd::launch_sparse<64, false, 1, 4>(a, stream);
  if (a.D == 128)
    return a.causal ? fwd::launch_sparse<128, true, 1, 8>(a, stream) : fwd::launch_sparse<128, false, 1, 8>(a, stream);
  if (a.D == 96)
    return a.causal ? fwd::launch_sparse<96, true, 1, 8>(a, stream) : fwd::launch_sparse<96, false, 1, 8>(a, stream);
  if (a.D == 32)
    return a.causal ? fwd::launch_sparse<32, true, 1, 4>(a, stream) : fwd::launch_sparse<32, false, 1, 4>(a, stream);
  if (a.D == 256)
    return a.causal ? fwd::launch_sparse<256, true, 1, 4>(a, stream) : fwd::launch_sparse<256, false, 1, 4>(a, stream);
  if (a.D == 160)
    return a.causal ? fwd::launch_sparse<160, true, 1, 4>(a, stream) : fwd::launch_sparse<160, false, 1, 4>(a, stream);
  return -2;
}

}  // namespace fa
