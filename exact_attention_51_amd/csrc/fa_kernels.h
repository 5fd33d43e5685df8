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
  // Query and key lengths apart (fa_fwd_kv): N is the query length, Nk the
  // key length; causal masking aligns the queries with the last keys.  With
  // n_split > 1 each key range writes its normalised O (float32) and its L
  // to part_o [n_split][B*H][N][D] and part_l [n_split][B*H][N], and a
  // second kernel merges them into o and lse.
  int Nk;
  int n_split;
  float* part_o;
  float* part_l;
  // Block-sparse forward (fa_fwd_sparse): uint8 [mask_heads][nb][nb] with
  // nb = ceil(N / 64); entry (a, c) != 0 lets query rows 64a.. see keys 64c..
  // mask_heads is 1 (one mask for every head) or B*H.
  const unsigned char* block_mask;
  int mask_heads;
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

// CUs of the current device, read from the device once and cached per
// device (256 if the query fails); safe to call from several host threads.
int device_cus();

// Each returns 0 on a successful launch, -1 when the launch failed and -2
// when no kernel instance exists for the shape.
int launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);
// fa_fwd_d128.hip: the square forward at D = 128 for N >= 64 (64 query rows
// per wave, key loop in assembly).
int launch_fwd_d128(const FwdArgs& a, hipStream_t stream);
// fa_fwd_kv.hip: query and key lengths apart, keys optionally split over
// n_split workgroups per query block, then the merge of the key ranges.
int launch_fwd_bf16_kv(const FwdArgs& a, hipStream_t stream);
int launch_fwd_bf16_kv_d256(const FwdArgs& a, hipStream_t stream);  // fa_fwd_kv_d256.hip
// Merge: up to kMaxNarrowMerge ranges with D/4 threads per row in 256-thread
// workgroups, more ranges with one 256-thread workgroup per row.
constexpr int kMaxNarrowMerge = 8;
int launch_fwd_kv_merge(const FwdArgs& a, hipStream_t stream);
// fa_decode.hip: a.N <= kDecodeMaxRows query rows per head on the vector
// ALUs, keys split over a.n_split workgroups (same partial-result layout and
// merge as above).
constexpr int kDecodeMaxRows = 4;
// fa_fwd_sparse.hip: the square forward over the key tiles a block mask
// keeps (at most kSparseMaxTiles key tiles of 64; D = 64 and 128).
constexpr int kSparseBlock = 64;
constexpr int kSparseMaxTiles = 4096;
int launch_fwd_bf16_sparse(const FwdArgs& a, hipStream_t stream);
int launch_fwd_decode(const FwdArgs& a, hipStream_t stream);
// Workgroups of the forward kernel one CU runs at a time, by head dimension.
int fwd_workgroups_per_cu(int D);
int fwd_rows_per_workgroup(int D, int Nq);  // query rows per workgroup of the fa_fwd_kv matrix-core path
int fwd_threads_per_workgroup(int D, int Nq);  // threads per workgroup of the same
constexpr int kDecodeThreads = 256;            // threads per workgroup of the decode kernel
int launch_fwd_f32(const FwdArgs& a, hipStream_t stream);
int launch_bwd_dq(const BwdArgs& a, hipStream_t stream);
int launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream);
int launch_bwd_dkdv_d256(const BwdArgs& a, hipStream_t stream);  // fa_bwd_dkdv_d256.hip

}  // namespace fa
