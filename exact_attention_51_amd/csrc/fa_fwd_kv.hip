// fa_fwd_kv.hip -- forward with query and key lengths apart and the key
// tiles of each query block optionally split over several workgroups
// (instances for D = 64 and D = 128; D = 256 in fa_fwd_kv_d256.hip), and
// the kernel that merges the key ranges.
//
// Splitting the keys serves the shapes whose (query block, batch, head)
// grid is too small for 256 CUs: a short query block over a long key
// sequence (one decoded row is the extreme case) or few heads.  Each range
// yields the exact attention of its keys, normalised, with its own L; the
// ranges combine exactly as L = ln sum_s e^{L_s} and
// O = sum_s e^{L_s - L} O_s, the same combination the saved L of the
// metal-flash-attention README's forward ("Quantifying performance") makes
// possible and that the D = 256 kernel already performs between the two
// key halves of a tile inside one workgroup.
#include "fa_fwd_bf16.h"

namespace fa {
namespace fwd {

template <int D, bool CAUSAL, int QB, int W>
int launch_kv(const FwdArgs& a, hipStream_t stream) {
  using C = FwdCfg<D, QB, W>;
  const int n_qtiles = (a.N + C::kBlockM - 1) / C::kBlockM;
  const TileSched sched = make_sched(n_qtiles * a.n_split, a.B * a.H, CAUSAL);
  const long grid = (long)n_qtiles * a.n_split * a.B * a.H;
  if (a.Nk < 64)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, QB, W, true, true>), dim3((unsigned)grid), dim3(64 * W), 0, stream,
                       a, sched);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, QB, W, false, true>), dim3((unsigned)grid), dim3(64 * W), 0,
                       stream, a, sched);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// One thread per four consecutive d of a row, for at most kMaxNarrow ranges:
// the row's L_s of every range give L, then O = sum_s e^{L_s - L} O_s,
// rounded to bf16.  Every range's loads are issued together; a range a row
// does not reach holds O_s = 0 and L_s = -inf, so its term is exactly 0.
constexpr int kMaxNarrow = kMaxNarrowMerge;
template <int D>
__global__ __launch_bounds__(256) void fwd_kv_merge_kernel(FwdArgs a) {
  constexpr int kThreadsPerRow = D / 4;
  constexpr int kRowsPerBlock = 256 / kThreadsPerRow;
  if (threadIdx.x >= kRowsPerBlock * kThreadsPerRow) return;  // threads past the last whole row
  const long rows = (long)a.B * a.H * a.N;
  const long r = (long)blockIdx.x * kRowsPerBlock + threadIdx.x / kThreadsPerRow;
  if (r >= rows) return;
  const int t = threadIdx.x % kThreadsPerRow;
  const int S = a.n_split;
  const float* __restrict__ Lp = a.part_l + r;
  const float* __restrict__ Op = a.part_o + r * D + t * 4;
  float ls[kMaxNarrow];
  f32x4 xs[kMaxNarrow];
#pragma unroll
  for (int s = 0; s < kMaxNarrow; ++s) {
    ls[s] = s < S ? Lp[(size_t)s * rows] : -__builtin_inff();
    xs[s] = s < S ? *(const f32x4*)(Op + (size_t)s * rows * D) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float mx = ls[0];
#pragma unroll
  for (int s = 1; s < kMaxNarrow; ++s) mx = __builtin_fmaxf(mx, ls[s]);
  float w[kMaxNarrow], sum = 0.f;
#pragma unroll
  for (int s = 0; s < kMaxNarrow; ++s) {
    w[s] = fast_exp2((ls[s] - mx) * kLog2e);
    sum += w[s];
  }
  const float inv = 1.0f / sum;
  const float L = mx + fast_log2(sum) * kLn2;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kMaxNarrow; ++s) {
    const float ws = w[s] * inv;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(ws, xs[s][e], acc[e]);
  }
  const u32x2 packed = {pack_bf16_u32(acc[0], acc[1]), pack_bf16_u32(acc[2], acc[3])};
  *(u32x2*)((__bf16*)a.o + r * D + t * 4) = packed;
  if (t == 0) a.lse[r] = L;
}

// The same merge for many key ranges: one workgroup per row, the ranges
// divided among kP groups of D/4 threads (range s goes to group s % kP).
// Each thread merges its ranges in chunks of kChunk, issuing a chunk's loads
// together, as a running (max M, sum l, weighted O) in the exp2 domain; the
// groups' running sums combine through LDS.  The running max starts at a
// finite floor, so ranges with L_s = -inf (O_s = 0) add exactly nothing.
template <int D>
__global__ __launch_bounds__(256) void fwd_kv_merge_wide_kernel(FwdArgs a) {
  constexpr int kThreadsPerRow = D / 4;
  constexpr int kP = 256 / kThreadsPerRow;
  constexpr int kChunk = 8;
  constexpr float kFloor = -1.0e30f;
  __shared__ float red_m[kP], red_l[kP];
  __shared__ f32x4 ored[kP][kThreadsPerRow];
  const long rows = (long)a.B * a.H * a.N;
  const long r = blockIdx.x;
  // threads past kP whole groups (D/4 need not divide 256) take no range
  const bool in_group = threadIdx.x < kP * kThreadsPerRow;
  const int t = threadIdx.x % kThreadsPerRow, p = threadIdx.x / kThreadsPerRow;
  const int S = in_group ? a.n_split : 0;
  const float* __restrict__ Lp = a.part_l + r;
  const float* __restrict__ Op = a.part_o + r * D + t * 4;
  float M = kFloor, l = 0.f;  // exp2 domain
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = p; s0 < S; s0 += kP * kChunk) {
    float ls[kChunk];
    f32x4 xs[kChunk];
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
      const int s = s0 + c * kP;
      ls[c] = s < S ? Lp[(size_t)s * rows] * kLog2e : -__builtin_inff();
      xs[c] = s < S ? *(const f32x4*)(Op + (size_t)s * rows * D) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float mc = M;
#pragma unroll
    for (int c = 0; c < kChunk; ++c) mc = __builtin_fmaxf(mc, ls[c]);
    const float alpha = fast_exp2(M - mc);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] *= alpha;
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
      const float w = fast_exp2(ls[c] - mc);
      l += w;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(w, xs[c][e], acc[e]);
    }
    M = mc;
  }
  if (in_group) {
    ored[p][t] = acc;
    if (t == 0) {
      red_m[p] = M;
      red_l[p] = l;
    }
  }
  __syncthreads();
  if (p != 0) return;
  float Mt = red_m[0];
#pragma unroll
  for (int i = 1; i < kP; ++i) Mt = __builtin_fmaxf(Mt, red_m[i]);
  float lt = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kP; ++i) {
    const float w = fast_exp2(red_m[i] - Mt);
    lt = __builtin_fmaf(w, red_l[i], lt);
    const f32x4 x = ored[i][t];
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = __builtin_fmaf(w, x[e], o[e]);
  }
  // every row sees some key, so lt > 0
  const float inv = 1.0f / lt;
  const u32x2 packed = {pack_bf16_u32(o[0] * inv, o[1] * inv), pack_bf16_u32(o[2] * inv, o[3] * inv)};
  *(u32x2*)((__bf16*)a.o + r * D + t * 4) = packed;
  if (t == 0) a.lse[r] = (Mt + fast_log2(lt)) * kLn2;
}

}  // namespace fwd

// At D = 128 and 96, up to 128 query rows run on 4-wave, 128-row
// workgroups rather than 8-wave, 256-row ones: half the idle rows.  Measured
// on one MI355X at the split count the library picks: 16 rows x 8192 keys x
// 128 heads 127 -> 98 us, 64 rows x 8192 keys x 32 heads 37 -> 29 us,
// 128 rows x 32768 keys x 8 heads 45 -> 36 us; longer query blocks gain
// nothing (the pages' shape: 38.5 us either way at the best split count).
static bool kv_small_block(int D, int Nq) { return (D == 128 || D == 96) && Nq <= 128; }

int fwd_workgroups_per_cu(int D) { return D <= 64 ? 3 : 1; }
int fwd_threads_per_workgroup(int D, int Nq) {
  if (D <= 64) return 64 * fwd::FwdCfg<64, 1, 4>::kWaves;
  if (kv_small_block(D, Nq)) return 64 * fwd::FwdCfg<128, 1, 4>::kWaves;
  if (D == 96 || D == 128) return 64 * fwd::FwdCfg<128, 1, 8>::kWaves;
  return 64 * fwd::FwdCfg<256, 1, 4>::kWaves;
}
int fwd_rows_per_workgroup(int D, int Nq) {
  if (D <= 64) return fwd::FwdCfg<64, 1, 4>::kBlockM;
  if (kv_small_block(D, Nq)) return fwd::FwdCfg<128, 1, 4>::kBlockM;
  if (D == 96 || D == 128) return fwd::FwdCfg<128, 1, 8>::kBlockM;
  return fwd::FwdCfg<256, 1, 4>::kBlockM;
}

// Workgroup shapes as for the square forward (fa_fwd_bf16.hip).
int launch_fwd_bf16_kv(const FwdArgs& a, hipStream_t stream) {
  if (a.D == 64) return a.causal ? fwd::launch_kv<64, true, 1, 4>(a, stream) : fwd::launch_kv<64, false, 1, 4>(a, stream);
  if (kv_small_block(a.D, a.N)) {
    if (a.D == 128)
      return a.causal ? fwd::launch_kv<128, true, 1, 4>(a, stream) : fwd::launch_kv<128, false, 1, 4>(a, stream);
    return a.causal ? fwd::launch_kv<96, true, 1, 4>(a, stream) : fwd::launch_kv<96, false, 1, 4>(a, stream);
  }
  if (a.D == 128)
    return a.causal ? fwd::launch_kv<128, true, 1, 8>(a, stream) : fwd::launch_kv<128, false, 1, 8>(a, stream);
  if (a.D == 96) return a.causal ? fwd::launch_kv<96, true, 1, 8>(a, stream) : fwd::launch_kv<96, false, 1, 8>(a, stream);
  if (a.D == 32) return a.causal ? fwd::launch_kv<32, true, 1, 4>(a, stream) : fwd::launch_kv<32, false, 1, 4>(a, stream);
  if (a.D == 256 || a.D == 160) return launch_fwd_bf16_kv_d256(a, stream);
  return -2;
}

// Few ranges (at most 8): one thread per 4 columns of a row loads every
// range at once.  Many ranges: one workgroup per row with the ranges spread over
// its threads, so a row's loads do not form one long dependent chain.
int launch_fwd_kv_merge(const FwdArgs& a, hipStream_t stream) {
  const long rows = (long)a.B * a.H * a.N;
  if (a.n_split > fwd::kMaxNarrow) {
    const dim3 grid((unsigned)rows), block(256);
    if (a.D == 32) hipLaunchKernelGGL(fwd::fwd_kv_merge_wide_kernel<32>, grid, block, 0, stream, a);
    else if (a.D == 64) hipLaunchKernelGGL(fwd::fwd_kv_merge_wide_kernel<64>, grid, block, 0, stream, a);
    else if (a.D == 96) hipLaunchKernelGGL(fwd::fwd_kv_merge_wide_kernel<96>, grid, block, 0, stream, a);
    else if (a.D == 128) hipLaunchKernelGGL(fwd::fwd_kv_merge_wide_kernel<128>, grid, block, 0, stream, a);
    else if (a.D == 160) hipLaunchKernelGGL(fwd::fwd_kv_merge_wide_kernel<160>, grid, block, 0, stream, a);
    else if (a.D == 256) hipLaunchKernelGGL(fwd::fwd_kv_merge_wide_kernel<256>, grid, block, 0, stream, a);
    else return -2;
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  auto go = [&](auto kern, int rows_per_block) {
    const long blocks = (rows + rows_per_block - 1) / rows_per_block;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  };
  if (a.D == 32) return go(fwd::fwd_kv_merge_kernel<32>, 256 / 8);
  if (a.D == 64) return go(fwd::fwd_kv_merge_kernel<64>, 256 / 16);
  if (a.D == 96) return go(fwd::fwd_kv_merge_kernel<96>, 256 / 24);
  if (a.D == 128) return go(fwd::fwd_kv_merge_kernel<128>, 256 / 32);
  if (a.D == 160) return go(fwd::fwd_kv_merge_kernel<160>, 256 / 40);
  if (a.D == 256) return go(fwd::fwd_kv_merge_kernel<256>, 256 / 64);
  return -2;
}

}  // namespace fa
