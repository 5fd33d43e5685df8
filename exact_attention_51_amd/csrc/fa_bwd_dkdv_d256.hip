// fa_bwd_dkdv_d256.hip -- dK/dV kernel of the split backward at D = 256 and
// D = 160 (gfx950).
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
// dP = dO V^T, they swap P (bf16, as it enters the products) and dP (fp32)
// through LDS, and each accumulates dK and dV for its half of the 256
// output columns.  The work per key group is unchanged and a wave holds 128
// accumulator registers.  The K (or V) rows of a wave's keys stay in
// registers as MFMA operands.  D = 160 runs the same kernel on the 256-wide
// LDS rows of D = 256 (the chunks past 160 unused, global rows 160 wide);
// its five 32-column output blocks split 3 + 2 over the two waves.
//
// The loop is skewed by one query tile so that a step has one barrier and
// two independent halves of MFMA work: step i forms S (or dP) of tile i and
// publishes P (or dP) to the exchange, then finishes tile i-1 from the
// exchange the previous step published (dS, dV, dK).  Query tiles live two
// steps (a 3-slot ring) and the exchange is double-buffered.
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

template <int D_>
struct KvDsplitCfg {
  static constexpr int D = D_;
  static constexpr int DP = 256;     // LDS row pitch (elements)
  static constexpr int kDBlocks = D / 32;                 // 32-column output blocks
  static constexpr int kHalfBlocks = (kDBlocks + 1) / 2;  // blocks of output half 0 (half 1: the rest)
  static constexpr int kWaves = 4;   // 2 key groups x 2 output halves
  static constexpr int kKeys = 64;   // key rows per workgroup
  static constexpr int kQTile = 32;  // query rows per streamed tile
  static constexpr int kTileBytes = kQTile * DP * 2;
  static constexpr int kStatBytes = 256;       // 64 floats of L or delta (rows past the tile are spare)
  static constexpr int kXpBytes = 2 * 64 * 16;  // P: two bf16x8 operands per lane
  static constexpr int kXdBytes = 16 * 64 * 4;  // dP: a 32x32 fp32 accumulator, [r/4][lane] x 4
  static constexpr int kSlotBytes = 2 * kTileBytes + 2 * kStatBytes;  // Q, dO, L, delta of one tile
  static constexpr int kXBytes = 2 * (kXpBytes + kXdBytes);            // both key groups
  static constexpr int kLdsBytes = 3 * kSlotBytes + 2 * kXBytes;
  static_assert(kLdsBytes <= 160 * 1024, "LDS of one workgroup");
};

template <int D_, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1))) void bwd_dkdv_d256_kernel(
    BwdArgs a, TileSched sched) {
  using C = KvDsplitCfg<D_>;
  constexpr int D = C::D, DP = C::DP, kDSteps = D / 16, kHalfBlocks = C::kHalfBlocks, W = C::kWaves;
  __shared__ __attribute__((aligned(1024))) char smem_raw[C::kLdsBytes];
  lds_char* smem = (lds_char*)smem_raw;
  // query-tile ring: tile t in slot t % 3 (Q, dO, L, delta)
  auto qbuf = [&](int sl) { return smem + sl * C::kSlotBytes; };
  auto obuf = [&](int sl) { return qbuf(sl) + C::kTileBytes; };
  auto lbuf = [&](int sl) { return qbuf(sl) + 2 * C::kTileBytes; };
  auto dbuf = [&](int sl) { return qbuf(sl) + 2 * C::kTileBytes + C::kStatBytes; };

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
  // exchange of tile t in buffer t % 2: [key group][P (bf16x8 [cc][lane]),
  // dP (fp32x4 [r/4][lane]: each lane's 16 values as four 16-byte runs)]
  auto xp = [&](int xb) {
    return (bf16x8 __attribute__((address_space(3)))*)(smem + 3 * C::kSlotBytes + xb * C::kXBytes +
                                                         kgrp * (C::kXpBytes + C::kXdBytes)) + lane;
  };
  auto xdp = [&](int xb) {
    return (f32x4 __attribute__((address_space(3)))*)(smem + 3 * C::kSlotBytes + xb * C::kXBytes +
                                                      kgrp * (C::kXpBytes + C::kXdBytes) + C::kXpBytes) + lane;
  };

  auto load_qtile = [&](int t) {
    const int sl = t % 3;
    copy_rows_lds<D, DP, C::kQTile, W>(Q, N, t * C::kQTile, qbuf(sl), wave, lane);
    copy_rows_lds<D, DP, C::kQTile, W>(dO, N, t * C::kQTile, obuf(sl), wave, lane);
    if (wave == 0) {
      int r = t * C::kQTile + lane;
      r = r < N ? r : N - 1;
      load_lds4(Lg + r, lbuf(sl));
      load_lds4(Dg + r, dbuf(sl));
    }
  };
  load_qtile(t_begin);

  // this wave's half of dK^T and dV^T: d blocks dh*kHalfBlocks .. (those below kDBlocks)
  f32x16 dk[kHalfBlocks], dv[kHalfBlocks];
#pragma unroll
  for (int i = 0; i < kHalfBlocks; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[i][r] = dv[i][r] = 0.f;
  const float c = a.scale_log2;
  // K (S-forming wave) or V (dP-forming wave) of this wave's keys as B
  // operands: key column l32, d = ds*16 + half*8 + 0..7
  bf16x8 kvf[kDSteps];
  {
    const __bf16* __restrict__ src = dh == 0 ? K : V;
    const int crow = key < N ? key : N - 1;
#pragma unroll
    for (int ds = 0; ds < kDSteps; ++ds) kvf[ds] = *(const bf16x8*)(src + (size_t)crow * D + ds * 16 + half * 8);
  }

  // does key group kgrp see any query of tile t?
  auto tile_work = [&](int t) { return group_active && !(CAUSAL && t * C::kQTile + C::kQTile - 1 < wk0); };

  for (int t = t_begin; t <= n_qtiles; ++t) {
    // publishes tile t (loaded last step) and the exchange of tile t-1
    wait_vmcnt<0>();
    __syncthreads();
    if (t + 1 < n_qtiles) load_qtile(t + 1);  // into the slot of tile t-2, finished last step

    // 1. tile t: S = Q_t K^T (dh = 0) or dP = dO_t V^T (dh = 1), to the exchange
    if (t < n_qtiles && tile_work(t)) {
      const int sl = t % 3, xb = t & 1, tq0 = t * C::kQTile;
      const lds_char* at = dh == 0 ? qbuf(sl) : obuf(sl);
      f32x16 mine;
#pragma unroll
      for (int ds = 0; ds < kDSteps; ++ds)
        mine = mfma32(read_row_operand<DP>(at, l32, ds, half), kvf[ds], ds == 0 ? f32x16{} : mine);
      if (dh == 0) {  // P = exp(S - L), masked; queries of register r: (r/4)*8 + half*4 + r%4
        const bool masked = (CAUSAL && tq0 < wk0 + 31) || (tq0 + C::kQTile > N);
        // L of the lane's 16 queries: four runs of four consecutive rows
        float lq[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 l4 = *(const f32x4 __attribute__((address_space(3)))*)(lbuf(sl) + 4 * (g * 8 + half * 4));
#pragma unroll
          for (int i = 0; i < 4; ++i) lq[g * 4 + i] = l4[i];
        }
        // two instances: tiles that need no mask carry no selects
        auto exp_p = [&](auto mconst) {
          constexpr bool MASKED = decltype(mconst)::value;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int qr = (r >> 2) * 8 + half * 4 + (r & 3);
            float x = __builtin_fmaf(mine[r], c, -lq[r] * kLog2e);
            if constexpr (MASKED) {
              bool keep = tq0 + qr < N;
              if constexpr (CAUSAL) keep = keep && key <= tq0 + qr;
              x = keep ? x : -__builtin_inff();
            }
            mine[r] = fast_exp2(x);
          }
        };
        if (masked)
          exp_p(std::integral_constant<bool, true>());
        else
          exp_p(std::integral_constant<bool, false>());
        // P rounded to bf16 once; both waves form dS from this rounded P
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          bf16x2 pp[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) pp[i] = pack_bf16(mine[cc * 8 + 2 * i], mine[cc * 8 + 2 * i + 1]);
          xp(xb)[cc * 64] = join8(pp[0], pp[1], pp[2], pp[3]);
        }
      } else {
#pragma unroll
        for (int g = 0; g < 4; ++g)
          xdp(xb)[g * 64] = f32x4{mine[4 * g], mine[4 * g + 1], mine[4 * g + 2], mine[4 * g + 3]};
      }
    }

    // 2. tile t-1, both waves: P (bf16) and dS = P (dP - delta) as bf16
    // operands from the exchange, then their half of dV and dK
    if (t > t_begin && tile_work(t - 1)) {
      const int sl = (t - 1) % 3, xb = (t - 1) & 1;
      float dl[16];  // delta of the lane's 16 queries, read as four runs of four
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 d4 = *(const f32x4 __attribute__((address_space(3)))*)(dbuf(sl) + 4 * (g * 8 + half * 4));
#pragma unroll
        for (int i = 0; i < 4; ++i) dl[g * 4 + i] = d4[i];
      }
      float dpv[16];  // dP of the lane's 16 queries
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 p4 = xdp(xb)[g * 64];
#pragma unroll
        for (int i = 0; i < 4; ++i) dpv[g * 4 + i] = p4[i];
      }
      bf16x8 ppk[2], dspk[2];
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        ppk[cc] = xp(xb)[cc * 64];
        const bf16x2* pp = (const bf16x2*)&ppk[cc];
        bf16x2 dd[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float dsv[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int r = cc * 8 + 2 * i + u;
            dsv[u] = (float)pp[i][u] * (dpv[r] - dl[r]);
          }
          dd[i] = pack_bf16(dsv[0], dsv[1]);
        }
        dspk[cc] = join8(dd[0], dd[1], dd[2], dd[3]);
      }
      // dV^T += dO^T P,  dK^T += Q^T dS over d blocks dh*kHalfBlocks ..
#pragma unroll
      for (int i = 0; i < kHalfBlocks; ++i) {
        if (dh * kHalfBlocks + i >= C::kDBlocks) break;  // D = 160: half 1 has one block fewer
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const int d0 = (dh * kHalfBlocks + i) * 32;
          dv[i] = mfma32(read_tr_operand<DP>(obuf(sl), cc * 16, d0, lane), ppk[cc], dv[i]);
          dk[i] = mfma32(read_tr_operand<DP>(qbuf(sl), cc * 16, d0, lane), dspk[cc], dk[i]);
        }
      }
    }
  }

  wait_vmcnt<0>();  // no direct-to-LDS copy may outlive the workgroup
  if (!group_active || key >= N) return;
  __bf16* __restrict__ dK = (__bf16*)a.dk + head_off;
  __bf16* __restrict__ dV = (__bf16*)a.dv + head_off;
#pragma unroll
  for (int i = 0; i < kHalfBlocks; ++i) {
    if (dh * kHalfBlocks + i >= C::kDBlocks) break;
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
}

template <int D, bool CAUSAL>
int launch(const BwdArgs& a, hipStream_t stream) {
  const int n_tiles = (a.N + KvDsplitCfg<D>::kKeys - 1) / KvDsplitCfg<D>::kKeys;
  // causal: the first key blocks see the most query tiles, so ascending order is heaviest first
  const TileSched sched = make_sched(n_tiles, a.B * a.H, false);
  const long grid = (long)n_tiles * a.B * a.H;
  hipLaunchKernelGGL((bwd_dkdv_d256_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(256), 0, stream, a, sched);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int launch_bwd_dkdv_d256(const BwdArgs& a, hipStream_t stream) {
  if (a.D == 160) return a.causal ? launch<160, true>(a, stream) : launch<160, false>(a, stream);
  if (a.D == 256) return a.causal ? launch<256, true>(a, stream) : launch<256, false>(a, stream);
  return -2;
}

}  // namespace fa
