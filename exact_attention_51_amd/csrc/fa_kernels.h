// fa_kernels.h -- internal launch interface between the C-ABI layer
// (fa_api.hip) and the kernel translation units.  Arguments have already
// been validated when these are called.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, N, D;
  float scale;       // multiplies Q K^T
  float scale_log2;  // scale * log2(e)
  int causal;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dO;
  const float* lse;
  float* delta;
  void* dq;
  void* dk;
  void* dv;
  int B, H, N, D;
  float scale;
  float scale_log2;
  int causal;
};

// Each returns 0 on a successful launch, -1 when the launch failed and -2
// when no kernel instance exists for the shape.
int launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);
int launch_fwd_f32(const FwdArgs& a, hipStream_t stream);
int launch_bwd_dq(const BwdArgs& a, hipStream_t stream);
int launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream);
int launch_bwd_dkdv_d256(const BwdArgs& a, hipStream_t stream);  // fa_bwd_dkdv_d256.hip

}  // namespace fa
