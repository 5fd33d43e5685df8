// fa_bwd_dkdv_d256.hip -- dK/dV kernel of the split backward at D = 256 (gfx950).
//
// The operation is the key/value side of the metal-flash-attention README's
// backward ("Quantifying performance", backward-key-value pseudocode): a
// workgroup owns a block of key rows and loops over query blocks,
// rebuilding P = exp(S - L) and dS = P (dP - delta) to accumulate
//   dV_j += sum_i P_ij dO_i,   dK_j += scale sum_i dS_ij Q_i.
//
// At D = 256 one wave per 32 keys holding all of dK and dV needs 256
// accumulator registers, and a workgroup whose K/V block and query tiles
// fill the LDS can only run one wave per SIMD pair.  Here the head
// dimension of the outputs is split instead: a key group of 32 keys has
// two waves; for every query tile one forms S = Q K^T, the other
// dP = dO V^T, they swap P and dP through LDS, and each accumulates dK and
// dV for its half of the 256 output columns.  The work per key group is
// unchanged, a wave holds 128 accumulator registers, and a 4-wave
// workgroup (two key groups, 64 keys) keeps every SIMD busy.
//
// Layouts are those of the general kernel (fa_bwd.hip): S = Q K^T and
// dP = dO V^T put a key in every lane column and 16 queries in its
// registers; P and dS packed to bf16 are the k-operands of dV^T += dO^T P
// and dK^T += Q^T dS, with dO^T and Q^T read transposed from the query tile.
#include "fa_device.h"
#include "fa_kernels.h"
#include "fa_sched.h"

namespace fa {

namespace {

struct KvDsplitCfg {
  static constexpr int D = 256;
  static constexpr int kWaves = 4;   // 2 key groups x 2 output halves
  static constexpr int kKeys = 64;   // key rows per workgroup
  static constexpr int kQTile = 32;  // query rows per streamed tile
  static constexpr int kKvBytes = kKeys * D * 2;
  static constexpr int kTileBytes = kQTile * D * 2;
  static constexpr int kStatBytes = 256;        // 64 floats of L or delta (rows past the tile are spare)
  static constexpr int kXBytes = 16 * 64 * 4;   // one wave's 32x32 fp32 accumulator, lane-major
  static constexpr int kLdsBytes = 2 * kKvBytes + 4 * kTileBytes + 4 * kStatBytes + 2 * 2 * kXBytes;
  static_assert(kLdsBytes <= 160 * 1024, "LDS of one workgroup");
};

template <bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1))) void bwd_dkdv_d256_kernel(
    BwdArgs a, TileSched sched) {
  using C = KvDsplitCfg;
  constexpr int D = C::D, kDSteps = D / 16, kHalfBlocks = D / 64, W = C::kWaves;
  __shared__ __attribute__((aligned(1024))) char smem_raw[C::kLdsBytes];
  lds_char* smem = (lds_char*)smem_raw;
  lds_char* kres = smem;
  lds_char* vres = smem + C::kKvBytes;
  lds_char* qbuf[2] = {smem + 2 * C::kKvBytes, smem + 2 * C::kKvBytes + C::kTileBytes};
  lds_char* obuf[2] = {smem + 2 * C::kKvBytes + 2 * C::kTileBytes, smem + 2 * C::kKvBytes + 3 * C::kTileBytes};
  lds_char* stat0 = smem + 2 * C::kKvBytes + 4 * C::kTileBytes;
  lds_char* lbuf[2] = {stat0, stat0 + C::kStatBytes};
  lds_char* dbuf[2] = {stat0 + 2 * C::kStatBytes, stat0 + 3 * C::kStatBytes};
  lds_char* xbase = stat0 + 4 * C::kStatBytes;  // [key group][P, dP] exchange

  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, l32 = lane & 31,
            half = lane >> 5;
  const int kgrp = wave & 1, dh = wave >> 1;  // key group; output half (0: forms S, 1: forms dP)
  int ktile, bh;
  sched_item(sched, blockIdx.x, ktile, bh);
  const int N = a.N;
  const size_t head_off = (size_t)bh * N * D;
  const __bf16* __restrict__ Q = (const __bf16*)a.q + head_off;
  const __bf16* __restrict__ K = (const __bf16*)a.k + head_off;
  const __bf16* __restrict__ V = (const __bf16*)a.v + head_off;
  const __bf16* __restrict__ dO = (const __bf16*)a.dO + head_off;
  const float* __restrict__ Lg = a.lse + (size_t)bh * N;
  const float* __restrict__ Dg = a.delta + (size_t)bh * N;

  const int k0 = ktile * C::kKeys;
  const int wk0 = k0 + kgrp * 32;
  const int key = wk0 + l32;
  const bool group_active = wk0 < N;
  const int n_qtiles = (N + C::kQTile - 1) / C::kQTile;
  const int t_begin = CAUSAL ? k0 / C::kQTile : 0;  // earlier query tiles see none of these keys
  float __attribute__((address_space(3)))* xp = (float __attribute__((address_space(3)))*)(xbase + kgrp * 2 * C::kXBytes) + lane;
  float __attribute__((address_space(3)))* xdp = xp + C::kXBytes / 4;

  auto load_qtile = [&](int t, int b) {
    copy_rows_lds<D, C::kQTile, W>(Q, N, t * C::kQTile, qbuf[b], wave, lane);
    copy_rows_lds<D, C::kQTile, W>(dO, N, t * C::kQTile, obuf[b], wave, lane);
    if (wave == 0) {
      int r = t * C::kQTile + lane;
      r = r < N ? r : N - 1;
      load_lds4(Lg + r, lbuf[b]);
      load_lds4(Dg + r, dbuf[b]);
    }
  };
  copy_rows_lds<D, C::kKeys, W>(K, N, k0, kres, wave, lane);
  copy_rows_lds<D, C::kKeys, W>(V, N, k0, vres, wave, lane);
  load_qtile(t_begin, 0);

  // this wave's half of dK^T and dV^T: d blocks dh*4 .. dh*4+3
  f32x16 dk[kHalfBlocks], dv[kHalfBlocks];
#pragma unroll
  for (int i = 0; i < kHalfBlocks; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[i][r] = dv[i][r] = 0.f;
  const float c = a.scale_log2;
  // the S-forming wave reads K, the dP-forming wave V, and their query-side tile
  const lds_char* kv = dh == 0 ? kres : vres;

  for (int t = t_begin; t < n_qtiles; ++t) {
    const int b = (t - t_begin) & 1;
    wait_vmcnt<0>();
    __syncthreads();
    if (t + 1 < n_qtiles) load_qtile(t + 1, b ^ 1);
    const int tq0 = t * C::kQTile;
    // every wave passes both barriers of the step; only the work is skipped
    const bool work = group_active && !(CAUSAL && tq0 + C::kQTile - 1 < wk0);
    const lds_char* qt = qbuf[b];
    const lds_char* ot = obuf[b];

    // 1. S = Q_t K^T (dh = 0) or dP = dO_t V^T (dh = 1), published to the partner
    f32x16 mine;
    if (work) {
      const lds_char* at = dh == 0 ? qt : ot;
#pragma unroll
      for (int ds = 0; ds < kDSteps; ++ds)
        mine = mfma32(read_row_operand<D>(at, l32, ds, half), read_row_operand<D>(kv, kgrp * 32 + l32, ds, half),
                      ds == 0 ? f32x16{} : mine);
      if (dh == 0) {  // P = exp(S - L), masked; queries of register r: (r/4)*8 + half*4 + r%4
        const bool masked = (CAUSAL && tq0 < wk0 + 31) || (tq0 + C::kQTile > N);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qr = (r >> 2) * 8 + half * 4 + (r & 3);
          const float lq = *(const float __attribute__((address_space(3)))*)(lbuf[b] + 4 * qr);
          float x = __builtin_fmaf(mine[r], c, -lq * kLog2e);
          if (masked) {
            bool keep = tq0 + qr < N;
            if constexpr (CAUSAL) keep = keep && key <= tq0 + qr;
            x = keep ? x : -__builtin_inff();
          }
          mine[r] = fast_exp2(x);
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) (dh == 0 ? xp : xdp)[r * 64] = mine[r];
    }
    __syncthreads();

    // 2. both waves: P and dS = P (dP - delta) as bf16 operands, then their half of dV and dK
    if (work) {
      bf16x8 ppk[2], dspk[2];
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        bf16x2 pp[4], dd[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float pv[2], dsv[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int r = cc * 8 + 2 * i + u;
            const int qr = (r >> 2) * 8 + half * 4 + (r & 3);
            const float p = dh == 0 ? mine[r] : xp[r * 64];
            const float dp = dh == 1 ? mine[r] : xdp[r * 64];
            const float dq = *(const float __attribute__((address_space(3)))*)(dbuf[b] + 4 * qr);
            pv[u] = p;
            dsv[u] = p * (dp - dq);
          }
          pp[i] = pack_bf16(pv[0], pv[1]);
          dd[i] = pack_bf16(dsv[0], dsv[1]);
        }
        ppk[cc] = join8(pp[0], pp[1], pp[2], pp[3]);
        dspk[cc] = join8(dd[0], dd[1], dd[2], dd[3]);
      }
      // dV^T += dO_t^T P,  dK^T += Q_t^T dS over d blocks dh*4 ..
#pragma unroll
      for (int i = 0; i < kHalfBlocks; ++i)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const int d0 = (dh * kHalfBlocks + i) * 32;
          dv[i] = mfma32(read_tr_operand<D>(ot, cc * 16, d0, lane), ppk[cc], dv[i]);
          dk[i] = mfma32(read_tr_operand<D>(qt, cc * 16, d0, lane), dspk[cc], dk[i]);
        }
    }
  }

  wait_vmcnt<0>();  // no direct-to-LDS copy may outlive the workgroup
  if (!group_active || key >= N) return;
  __bf16* __restrict__ dK = (__bf16*)a.dk + head_off;
  __bf16* __restrict__ dV = (__bf16*)a.dv + head_off;
#pragma unroll
  for (int i = 0; i < kHalfBlocks; ++i)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const size_t off = (size_t)key * D + (dh * kHalfBlocks + i) * 32 + g4 * 8 + half * 4;
      u32x2 wk = {pack_bf16_u32(dk[i][g4 * 4 + 0] * a.scale, dk[i][g4 * 4 + 1] * a.scale),
                  pack_bf16_u32(dk[i][g4 * 4 + 2] * a.scale, dk[i][g4 * 4 + 3] * a.scale)};
      u32x2 wv = {pack_bf16_u32(dv[i][g4 * 4 + 0], dv[i][g4 * 4 + 1]),
                  pack_bf16_u32(dv[i][g4 * 4 + 2], dv[i][g4 * 4 + 3])};
      *(u32x2*)(dK + off) = wk;
      *(u32x2*)(dV + off) = wv;
    }
}

template <bool CAUSAL>
int launch(const BwdArgs& a, hipStream_t stream) {
  const int n_tiles = (a.N + KvDsplitCfg::kKeys - 1) / KvDsplitCfg::kKeys;
  // causal: the first key blocks see the most query tiles, so ascending order is heaviest first
  const TileSched sched = make_sched(n_tiles, a.B * a.H, false);
  const long grid = (long)n_tiles * a.B * a.H;
  hipLaunchKernelGGL((bwd_dkdv_d256_kernel<CAUSAL>), dim3((unsigned)grid), dim3(256), 0, stream, a, sched);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int launch_bwd_dkdv_d256(const BwdArgs& a, hipStream_t stream) {
  return a.causal ? launch<true>(a, stream) : launch<false>(a, stream);
}

}  // namespace fa
