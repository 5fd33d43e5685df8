// fa_decode.hip -- forward for a few query rows per head (decoding), on the
// vector ALUs, with the keys split over many workgroups.
//
// The "Flash Attention" page (section on the technique's boundaries) notes
// that one query row cannot fill a matrix tile, so decoding needs its own
// vector kernel.  With Nq <= 4 rows per head each key is used by at most four
// dot products, so the kernel is bound by reading K and V from HBM, not by
// arithmetic: it streams every K and V row once, straight from global
// memory into registers (no LDS staging, nothing is reused), and spreads
// the key sequence over enough workgroups to keep every CU's loads in
// flight.
//
// Layout of the work:
// * A key row of D bf16 is split over LPK = D/8 lanes, 16 bytes each (one
//   global_load_dwordx4 per lane per row of K and of V; a wave reads
//   64/LPK whole rows per load instruction, fully coalesced).
// * A group of LPK lanes keeps its own online-softmax state (running max m
//   and sum l per query row, in the exp2 domain) and its slice of the
//   unnormalised O; the dot product of a row is summed over the group with
//   DPP lane permutations (mirror and quad swaps), so no LDS is touched in
//   the loop.
// * Each wave loads the next U rows per lane group while it computes the
//   current ones (register double buffering).
// * At the end the groups of the workgroup combine through LDS, rescaled to
//   their common max; the workgroup writes O and L directly (one key range)
//   or its range's normalised O and L_s for the merge kernel (several).
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace dec {

constexpr int kWaves = kDecodeThreads / 64;
constexpr int kUnroll = 4;                 // key rows per lane group in flight per buffer
constexpr float kMaxFloor = 1.0e30f;       // running max starts at -kMaxFloor (masked keys give p = 0)

// x + (x moved by a DPP permutation): the permutation is a template so the
// control word is an immediate.
template <int CTRL>
__device__ __forceinline__ float add_dpp(float x) {
  const int moved = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false);
  return x + __builtin_bit_cast(float, moved);
}

// Sum over aligned groups of LPK lanes (8, 16 or 32); every lane of the
// group gets the sum.  Mirrors pair lane i with lane LPK-1-i, so after the
// mirror steps the distinct partial sums sit in each quad, which two quad
// swaps finish.
template <int LPK>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (LPK == 32) x += __shfl_xor(x, 16);
  if constexpr (LPK >= 16) x = add_dpp<0x140>(x);  // row_mirror (16 lanes)
  x = add_dpp<0x141>(x);                            // row_half_mirror (8 lanes)
  x = add_dpp<0xB1>(x);                             // quad_perm [1,0,3,2]
  x = add_dpp<0x4E>(x);                             // quad_perm [2,3,0,1]
  return x;
}

__device__ __forceinline__ void unpack8(const u32x4& w, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __builtin_bit_cast(float, w[i] << 16);
    f[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
  }
}

template <int D, int NQ>
struct DecCfg {
  static constexpr int kLpk = D / 8;             // lanes per key row
  static constexpr int kGroups = 64 / kLpk;      // key rows per wave per load
  static constexpr int kStride = kWaves * kGroups;  // key rows per workgroup per load
};

template <int D, int NQ>
__global__ __launch_bounds__(64 * kWaves) void decode_kernel(FwdArgs a) {
  using C = DecCfg<D, NQ>;
  constexpr int LPK = C::kLpk, G = C::kGroups, STRIDE = C::kStride, U = kUnroll;
  __shared__ float sm_o[STRIDE][NQ][D];
  __shared__ float sm_ml[STRIDE][NQ][2];

  const int S = a.n_split;
  const int bh = blockIdx.x / S;
  const int split = blockIdx.x - bh * S;
  const int Nq = a.N, Nk = a.Nk;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int grp = lane / LPK, dl = lane % LPK;
  const int gi = wave * G + grp;  // lane group within the workgroup

  // key range of this workgroup, in 64-key units
  const int chunk = (((Nk + S - 1) / S) + 63) & ~63;
  const int k_lo = min(split * chunk, Nk), k_hi = min(k_lo + chunk, Nk);
  const int off = a.causal ? Nk - Nq : Nk;  // row r sees keys <= r + off (all keys without causal)

  const __bf16* __restrict__ Kh = (const __bf16*)a.k + (size_t)bh * Nk * D + dl * 8;
  const __bf16* __restrict__ Vh = (const __bf16*)a.v + (size_t)bh * Nk * D + dl * 8;

  // this lane's slice of the query rows, pre-multiplied by scale*log2(e)
  float q[NQ][8];
#pragma unroll
  for (int r = 0; r < NQ; ++r) {
    const int row = min(r, Nq - 1);
    const u32x4 w = *(const u32x4*)((const __bf16*)a.q + ((size_t)bh * Nq + row) * D + dl * 8);
    unpack8(w, q[r]);
#pragma unroll
    for (int e = 0; e < 8; ++e) q[r][e] *= a.scale_log2;
  }
  float m[NQ], l[NQ], o[NQ][8];
#pragma unroll
  for (int r = 0; r < NQ; ++r) {
    m[r] = -kMaxFloor;
    l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[r][e] = 0.f;
  }

  u32x4 kc[U], vc[U], kn[U], vn[U];
  // rows of the load at wave-uniform base b: key b + grp + u*STRIDE (clamped inside the tensor)
  auto load = [&](int b, u32x4 (&kk)[U], u32x4 (&vv)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = min(b + grp + u * STRIDE, Nk - 1);
      kk[u] = *(const u32x4*)(Kh + (size_t)key * D);
      vv[u] = *(const u32x4*)(Vh + (size_t)key * D);
    }
  };
  int base = k_lo + wave * G;
  if (base < k_hi) load(base, kc, vc);
  for (; base < k_hi; base += U * STRIDE) {
    const bool more = base + U * STRIDE < k_hi;  // wave-uniform
    if (more) load(base + U * STRIDE, kn, vn);
    float s[NQ][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[8];
      unpack8(kc[u], kf);
#pragma unroll
      for (int r = 0; r < NQ; ++r) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(q[r][e], kf[e], acc);
        s[r][u] = acc;
      }
    }
#pragma unroll
    for (int r = 0; r < NQ; ++r)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int key = base + grp + u * STRIDE;
        const float t = group_sum<LPK>(s[r][u]);
        s[r][u] = (key < k_hi && key <= r + off) ? t : -__builtin_inff();
      }
    // online softmax over the U rows of each lane group: one rescale per U keys
    float p[NQ][U];
#pragma unroll
    for (int r = 0; r < NQ; ++r) {
      float mx = s[r][0];
#pragma unroll
      for (int u = 1; u < U; ++u) mx = __builtin_fmaxf(mx, s[r][u]);
      const float m_new = __builtin_fmaxf(m[r], mx);
      const float alpha = fast_exp2(m[r] - m_new);
      m[r] = m_new;
      float ls = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        p[r][u] = fast_exp2(s[r][u] - m_new);
        ls += p[r][u];
      }
      l[r] = __builtin_fmaf(l[r], alpha, ls);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[r][e] *= alpha;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vf[8];
      unpack8(vc[u], vf);
#pragma unroll
      for (int r = 0; r < NQ; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[r][e] = __builtin_fmaf(p[r][u], vf[e], o[r][e]);
    }
    if (more) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        kc[u] = kn[u];
        vc[u] = vn[u];
      }
    }
  }

  // combine the lane groups of the workgroup
#pragma unroll
  for (int r = 0; r < NQ; ++r) {
#pragma unroll
    for (int e = 0; e < 8; ++e) sm_o[gi][r][dl * 8 + e] = o[r][e];
    if (dl == 0) {
      sm_ml[gi][r][0] = m[r];
      sm_ml[gi][r][1] = l[r];
    }
  }
  __syncthreads();
  for (int item = threadIdx.x; item < NQ * D; item += 64 * kWaves) {
    const int r = item / D, d = item % D;
    if (r >= Nq) continue;
    float M = -kMaxFloor;
#pragma unroll
    for (int g = 0; g < STRIDE; ++g) M = __builtin_fmaxf(M, sm_ml[g][r][0]);
    float lsum = 0.f, osum = 0.f;
#pragma unroll
    for (int g = 0; g < STRIDE; ++g) {
      const float w = fast_exp2(sm_ml[g][r][0] - M);
      lsum = __builtin_fmaf(w, sm_ml[g][r][1], lsum);
      osum = __builtin_fmaf(w, sm_o[g][r][d], osum);
    }
    const size_t orow = (size_t)bh * Nq + r;
    if (S == 1) {
      // every row sees at least key 0, so lsum > 0
      ((__bf16*)a.o)[orow * D + d] = (__bf16)(osum / lsum);
      if (d == 0) a.lse[orow] = (M + fast_log2(lsum)) * kLn2;
    } else {
      const size_t prow = (size_t)split * a.B * a.H * Nq + orow;
      // a range the row does not reach: O_s = 0, L_s = -inf (weight 0 in the merge)
      a.part_o[prow * D + d] = lsum > 0.f ? osum / lsum : 0.f;
      if (d == 0) a.part_l[prow] = lsum > 0.f ? (M + fast_log2(lsum)) * kLn2 : -__builtin_inff();
    }
  }
}

template <int D>
int launch_d(const FwdArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)((long)a.B * a.H * a.n_split)), block(64 * kWaves);
  if (a.N == 1) hipLaunchKernelGGL((decode_kernel<D, 1>), grid, block, 0, stream, a);
  else if (a.N == 2) hipLaunchKernelGGL((decode_kernel<D, 2>), grid, block, 0, stream, a);
  else hipLaunchKernelGGL((decode_kernel<D, 4>), grid, block, 0, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace dec

int launch_fwd_decode(const FwdArgs& a, hipStream_t stream) {
  if (a.N > kDecodeMaxRows) return -2;
  if (a.D == 64) return dec::launch_d<64>(a, stream);
  if (a.D == 128) return dec::launch_d<128>(a, stream);
  if (a.D == 256) return dec::launch_d<256>(a, stream);
  return -2;
}

}  // namespace fa
