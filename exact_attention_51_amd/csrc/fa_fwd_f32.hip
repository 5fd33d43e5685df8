// fa_fwd_f32.hip -- exact-attention forward with float32 inputs, outputs and
// arithmetic (gfx950).
//
// This is the float32 twin of the bf16 kernel, kept simple: it exists for
// float32 callers and small problems, where precision (1e-4 against the
// float64 oracle) matters more than throughput.  Four lanes share one query
// row, each holding a quarter of the head dimension in float4 chunks; the
// partial dot products are combined with two cross-lane xor steps.  K/V
// tiles of 32 keys are staged in LDS and read as broadcasts.  The online
// softmax is the pages' recurrence ("Learning Metal with FlashAttention",
// section FlashAttention): per key tile, raise the running max, shrink the
// running sum and accumulator by exp(m_old - m_new), add the tile's terms.
// Full-precision expf/logf are used.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr int kRowsPerBlock = 64;  // 4 waves x 16 rows
constexpr int kTileKeys = 32;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_f32_kernel(FwdArgs a) {
  constexpr int kChunks = D / 16;  // float4 chunks per lane
  __shared__ float4 ks[kTileKeys][D / 4];
  __shared__ float4 vs[kTileKeys][D / 4];

  const int tid = threadIdx.x;
  const int t = tid & 3;          // quarter of the head dim this lane holds
  const int rr = tid >> 2;        // row within the block
  const int N = a.N;
  const int n_qtiles = (N + kRowsPerBlock - 1) / kRowsPerBlock;
  const int bh = blockIdx.x / n_qtiles;
  const int q0 = (blockIdx.x % n_qtiles) * kRowsPerBlock;
  const int row = q0 + rr;
  const size_t head_off = (size_t)bh * N * D;
  const float4* __restrict__ Q4 = (const float4*)((const float*)a.q + head_off);
  const float4* __restrict__ K4 = (const float4*)((const float*)a.k + head_off);
  const float4* __restrict__ V4 = (const float4*)((const float*)a.v + head_off);

  const int qrow = row < N ? row : N - 1;
  float4 q[kChunks], o[kChunks];
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    q[i] = Q4[(size_t)qrow * (D / 4) + i * 4 + t];
    o[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float m = -__builtin_inff(), l = 0.f;

  int nkt = (N + kTileKeys - 1) / kTileKeys;
  if constexpr (CAUSAL) nkt = min(q0 + kRowsPerBlock - 1, N - 1) / kTileKeys + 1;

  for (int kt = 0; kt < nkt; ++kt) {
    __syncthreads();
    for (int idx = tid; idx < kTileKeys * (D / 4); idx += 256) {
      const int r = idx / (D / 4), cidx = idx % (D / 4);
      int grow = kt * kTileKeys + r;
      grow = grow < N ? grow : N - 1;
      ks[r][cidx] = K4[(size_t)grow * (D / 4) + cidx];
      vs[r][cidx] = V4[(size_t)grow * (D / 4) + cidx];
    }
    __syncthreads();

    float s[kTileKeys];
    float tmax = -__builtin_inff();
#pragma unroll
    for (int jj = 0; jj < kTileKeys; ++jj) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < kChunks; ++i) {
        const float4 kv = ks[jj][i * 4 + t];
        acc = __builtin_fmaf(q[i].x, kv.x, acc);
        acc = __builtin_fmaf(q[i].y, kv.y, acc);
        acc = __builtin_fmaf(q[i].z, kv.z, acc);
        acc = __builtin_fmaf(q[i].w, kv.w, acc);
      }
      acc += __shfl_xor(acc, 1);
      acc += __shfl_xor(acc, 2);
      const int key = kt * kTileKeys + jj;
      bool keep = key < N;
      if constexpr (CAUSAL) keep = keep && key <= row;
      s[jj] = keep ? acc * a.scale : -__builtin_inff();
      tmax = __builtin_fmaxf(tmax, s[jj]);
    }
    const float m_new = __builtin_fmaxf(m, tmax);
    const float alpha = expf(m - m_new);  // 0 on the first tile (m = -inf)
    l *= alpha;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      o[i].x *= alpha;
      o[i].y *= alpha;
      o[i].z *= alpha;
      o[i].w *= alpha;
    }
#pragma unroll
    for (int jj = 0; jj < kTileKeys; ++jj) {
      const float p = expf(s[jj] - m_new);
      l += p;
#pragma unroll
      for (int i = 0; i < kChunks; ++i) {
        const float4 vv = vs[jj][i * 4 + t];
        o[i].x = __builtin_fmaf(p, vv.x, o[i].x);
        o[i].y = __builtin_fmaf(p, vv.y, o[i].y);
        o[i].z = __builtin_fmaf(p, vv.z, o[i].z);
        o[i].w = __builtin_fmaf(p, vv.w, o[i].w);
      }
    }
    m = m_new;
  }

  if (row < N) {
    const float inv = 1.0f / l;
    float4* __restrict__ O4 = (float4*)((float*)a.o + head_off);
#pragma unroll
    for (int i = 0; i < kChunks; ++i)
      O4[(size_t)row * (D / 4) + i * 4 + t] = make_float4(o[i].x * inv, o[i].y * inv, o[i].z * inv, o[i].w * inv);
    if (t == 0) a.lse[(size_t)bh * N + row] = m + logf(l);
  }
}

template <int D, bool CAUSAL>
int launch(const FwdArgs& a, hipStream_t stream) {
  const long grid = (long)((a.N + kRowsPerBlock - 1) / kRowsPerBlock) * a.B * a.H;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int launch_fwd_f32(const FwdArgs& a, hipStream_t stream) {
  switch (a.D) {
    case 64:
      return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
    case 128:
      return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
    case 256:
      return a.causal ? launch<256, true>(a, stream) : launch<256, false>(a, stream);
  }
  return -2;
}

}  // namespace fa
