// fa_bwd.hip -- split backward kernels (dQ; dK/dV).  Not yet implemented.
#include "fa_kernels.h"

namespace fa {
int launch_fwd_bf16_d256(const FwdArgs&, hipStream_t) { return -2; }
int launch_bwd_dq(const BwdArgs&, hipStream_t) { return -2; }
int launch_bwd_dkdv(const BwdArgs&, hipStream_t) { return -2; }
}  // namespace fa
