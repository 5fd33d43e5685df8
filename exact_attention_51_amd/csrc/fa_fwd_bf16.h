// fa_fwd_bf16.h -- exact-attention forward kernel template, bf16 in/out, gfx950.
// Instantiated in fa_fwd_bf16.hip (D = 64, 128) and fa_fwd_bf16_d256.hip.
//
// One workgroup = 8 waves (two per SIMD; 4 at D = 256); each wave owns
// 32*QB query rows of one (batch, head) and the whole loop over keys for
// them.  The streaming
// structure is the one every page describes ("Learning Metal with
// FlashAttention", section FlashAttention; "Flash Attention" page, kernel
// anatomy; metal-flash-attention README, "Quantifying performance", forward
// pseudocode): the Q rows are loaded once and stay resident (in registers,
// or in LDS when two waves share a SIMD at D >= 128), K and V
// stream through LDS in tiles of 64 keys, the running row max m and row sum
// l rescale the unnormalised accumulator, and the score matrix only ever
// exists as MFMA accumulator registers.
//
// MI355X-specific choices:
// * Scores are computed transposed, S^T = K Q^T, with 32x32x16 bf16 MFMA.
//   In the 32x32 accumulator layout every lane then holds one query column
//   and 16 keys, so the row max and row sum are in-lane reductions plus one
//   exchange between the two 32-lane halves (v_permlane32_swap).
// * The same accumulators, rounded to bf16, are directly the B operand of
//   O^T += V^T P^T; keys are a summation index, so the V operand is read
//   from LDS in the matching key order with ds_read_b64_tr_b16, which also
//   does the transpose V needs.  P never touches LDS.
// * Software pipeline inside each wave: while the MFMA pipe computes the
//   scores of tile j+1, the VALU exponentiates, packs and sums tile j; while
//   it accumulates P_j V_j, the VALU takes the row max of tile j+1.  The
//   rescale decision for a tile sits between the two.
// * K/V tiles go global -> LDS with 16-byte direct loads (no VGPR staging)
//   into a ring of NB buffers per tensor, issued NB-1 tiles ahead.  The
//   loop is unrolled over the ring so every LDS address is a per-lane
//   offset computed once plus an instruction immediate.  Rows are
//   XOR-swizzled in 16-byte chunks (see swz) so that both LDS read patterns
//   are free of bank conflicts.
// * exp is exp2 with scale*log2(e) folded into one FMA per score.  The
//   rescale of O is skipped while the running max has grown by less than
//   2^8 in the exp2 domain (the stale max is still an exact reference
//   point: P and l are just both scaled by the same bounded factor).
// * Causal masking skips every key tile above a wave's diagonal; only the
//   diagonal tile is masked element by element.  The tiles that need a mask
//   (a block's diagonal region, or a ragged last tile) are processed first
//   by a plain serial step, so the pipelined main loop carries no mask code.
#pragma once

#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"
#include "fa_sched.h"

namespace fa {
namespace fwd {

constexpr int kBlockN = 64;                // keys per K/V tile
constexpr float kRescaleThreshold = 8.0f;  // exp2-domain growth allowed before O is rescaled

template <int D, int QB, int W>
struct FwdCfg {
  static constexpr int kWaves = W;                       // waves per workgroup (4 or 8)
  static constexpr int kRowsPerWave = 32 * QB;
  static constexpr int kBlockM = kWaves * kRowsPerWave;  // query rows per workgroup
  static constexpr int kDSteps = D / 16;                 // k-steps of the S product
  static constexpr int kDBlocks = D / 32;                // 32-wide d blocks of O
  static constexpr int kTileBytes = kBlockN * D * 2;     // one K or V tile
#ifndef FA_FWD_NB
#define FA_FWD_NB 3
#endif
  static constexpr int kNB = D <= 128 ? FA_FWD_NB : 2;   // ring depth (D = 256: 2 x 2 x 32 KB)
  static_assert(kNB == 2 || kNB == 3, "the main loop is unrolled for a ring of 2 or 3 slots");
  // With two waves per SIMD at D >= 128 the Q^T operands move from
  // registers to LDS (same swizzled row layout as K) to stay within 256
  // registers; the LDS then holds the K/V ring plus every wave's Q rows.
#ifndef FA_FWD_QLDS
#define FA_FWD_QLDS 0
#endif
  static constexpr bool kQInLds = FA_FWD_QLDS && W == 8 && D >= 128;
  static constexpr int kQBytes = kQInLds ? W * kRowsPerWave * D * 2 : 0;
  static constexpr int kLdsBytes = 2 * kNB * kTileBytes + kQBytes;
  // one group = the K tile and the V tile a loop step issues
  static constexpr int kLoadsPerGroup = 2 * (kTileBytes / 16 / kWaves / 64);
  // 8-wave workgroups put two waves on each SIMD (registers must stay <= 256)
  static constexpr int kWavesPerEU = W / 4;
};

template <int D, bool CAUSAL, int QB, int W>
struct FwdKernel {
  using C = FwdCfg<D, QB, W>;
  static constexpr int NB = C::kNB;

  // per-wave state
  bf16x8 qf[QB][C::kDSteps];  // Q^T as B operands: query column l32, d = ds*16 + half*8 + 0..7
  f32x16 o[QB][C::kDBlocks];  // O^T accumulators
  f32x16 s[2][2][QB];         // two score tiles in ping-pong: [set][kb][qb]
  float m[QB], l[QB], mx[QB];
  int koff[C::kDSteps];      // per-lane K operand offsets within a K tile
  int voff[C::kDBlocks][2];  // per-lane V operand offsets, V region base included
  lds_char* smem;
  int lane, l32, half, wave;

  // K ring at [0, NB tiles), V ring at [NB, 2 NB tiles).  Reads address a
  // ring slot as (per-lane offset) + (slot and block immediates); the V
  // region base is folded into voff so every immediate stays below 64 KB.
  __device__ __forceinline__ lds_char* kbuf(int b) const { return smem + b * C::kTileBytes; }
  __device__ __forceinline__ lds_char* vbuf(int b) const { return smem + (NB + b) * C::kTileBytes; }
  __device__ __forceinline__ const lds_char* vslot(int b) const { return smem + b * C::kTileBytes; }
  __device__ __forceinline__ lds_char* qtile() const { return smem + 2 * NB * C::kTileBytes + wave * C::kRowsPerWave * D * 2; }
  // Q^T operand for query block qb, d-step ds (LDS copy shares K's row layout)
  __device__ __forceinline__ bf16x8 qfrag(int qb, int ds) const {
    if constexpr (C::kQInLds)
      return *(const bf16x8 __attribute__((address_space(3)))*)(qtile() + koff[ds] + qb * 32 * D * 2);
    else
      return qf[qb][ds];
  }

  // S^T tile from the K buffer kt: acc[kb][qb]
  __device__ __forceinline__ void scores(const lds_char* kt, f32x16 (&acc)[2][QB]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[kb][qb][r] = 0.f;
#pragma unroll
    for (int ds = 0; ds < C::kDSteps; ++ds)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf = *(const bf16x8 __attribute__((address_space(3)))*)(kt + koff[ds] + kb * 32 * D * 2);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) acc[kb][qb] = mfma32(kf, qfrag(qb, ds), acc[kb][qb]);
      }
  }

  // -inf where a key is invisible: above the causal diagonal, past N, or
  // (in a ragged last tile, loaded shifted to end at row N-1) already
  // covered by the previous tile.  key0 is the tile's first row, kmin the
  // first key the tile contributes.
  __device__ __forceinline__ void mask(f32x16 (&acc)[2][QB], int key0, int kmin, int wq0, int N) {
    // Element (kb, r) of this lane holds key base + off with a compile-time
    // offset off; the visible keys are the offsets in [lo, hi).
    const int base = key0 + half * 4;
    const int lo = kmin - base;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      int hi = N - base;
      if constexpr (CAUSAL) hi = min(hi, wq0 + qb * 32 + l32 + 1 - base);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = kb * 32 + (r >> 2) * 8 + (r & 3);
          acc[kb][qb][r] = (off >= lo && off < hi) ? acc[kb][qb][r] : -__builtin_inff();
        }
    }
  }

  // Row max of a score tile (both halves agree afterwards).
  __device__ __forceinline__ void rowmax(const f32x16 (&acc)[2][QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float t[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int kb = i >> 2, r = (i & 3) * 4;
        t[i] = __builtin_fmaxf(__builtin_fmaxf(acc[kb][qb][r], acc[kb][qb][r + 1]),
                               __builtin_fmaxf(acc[kb][qb][r + 2], acc[kb][qb][r + 3]));
      }
      const float a = __builtin_fmaxf(__builtin_fmaxf(t[0], t[1]), __builtin_fmaxf(t[2], t[3]));
      const float b = __builtin_fmaxf(__builtin_fmaxf(t[4], t[5]), __builtin_fmaxf(t[6], t[7]));
      mx[qb] = max_halves(__builtin_fmaxf(a, b));
    }
  }

  // Raise the running max to include mx; rescale O and l when it grew by
  // more than the threshold in any lane of the wave (a wave-uniform branch).
  __device__ __forceinline__ void update_max(float c) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float m_new = __builtin_fmaxf(m[qb], mx[qb]);
      const bool grow = (m_new - m[qb]) * c > kRescaleThreshold;
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        const float alpha = fast_exp2((m[qb] - m_new) * c);  // 0 on the first tile (m = -inf)
#pragma unroll
        for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[qb][db][r] *= alpha;
        l[qb] *= alpha;
        m[qb] = m_new;
      }
    }
  }

  // P = exp2(S c - m c) packed to bf16 B operands; the row sum is taken over
  // the rounded P that enters the product.
  __device__ __forceinline__ void exponentiate(const f32x16 (&sc)[2][QB], float c, bf16x8 (&pk)[QB][2][2]) {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float mc = m[qb] * c;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          bf16x2 pr[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float e0 = fast_exp2(__builtin_fmaf(sc[kb][qb][cc * 8 + 2 * i], c, -mc));
            const float e1 = fast_exp2(__builtin_fmaf(sc[kb][qb][cc * 8 + 2 * i + 1], c, -mc));
            pr[i] = pack_bf16(e0, e1);
            l[qb] = __builtin_amdgcn_fdot2_f32_bf16(pr[i], ones, l[qb], false);
          }
          pk[qb][kb][cc] = join8(pr[0], pr[1], pr[2], pr[3]);
        }
    }
  }

  // ---- pipelined step, written in issue order -------------------------
  // The S MFMAs of the next tile each carry their share of this tile's
  // exponentials; the P V MFMAs of this tile each carry a share of the
  // next tile's row max; every LDS fragment is read kPf fragments ahead of
  // the MFMA that consumes it.  sched_barrier fences keep the compiler from
  // regrouping the sequence (it would otherwise cluster reads next to their
  // use and the MFMAs of one product together).
  static constexpr int kKFrags = 2 * C::kDSteps;   // K fragments per tile, QB MFMAs each
  static constexpr int kVFrags = 4 * C::kDBlocks;  // V fragments per tile, QB MFMAs each
  static constexpr int kPf = 3;                    // read-ahead in fragments
  static constexpr int kPairs = 16 * QB;           // exp pairs per tile and lane
  static constexpr int kMaxUnits = 9 * QB;         // row-max work units per tile
  static constexpr int kMaxStart = 2;              // first P V MFMA that carries row-max work

  // K fragment i = (ds, kb) = (i / 2, i % 2)
  __device__ __forceinline__ bf16x8 kfrag(const lds_char* kt, int i) const {
    return *(const bf16x8 __attribute__((address_space(3)))*)(kt + koff[i >> 1] + (i & 1) * 32 * D * 2);
  }
  // V fragment j = (kb, cc, db): (kb, cc) = j / kDBlocks, db = j % kDBlocks
  __device__ __forceinline__ bf16x8 vfrag(const lds_char* vt, int j) const {
    const int kc = j / C::kDBlocks, db = j % C::kDBlocks;
    const int rows = ((kc >> 1) * 32 + (kc & 1) * 16) * D * 2;
    const s16x4 va = ds_read_tr(vt + voff[db][0] + rows);
    const s16x4 vb = ds_read_tr(vt + voff[db][1] + rows);
    const s16x8 v8 = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
    return __builtin_bit_cast(bf16x8, v8);
  }

  __device__ __forceinline__ void pipelined(const lds_char* kt, const lds_char* vt, const f32x16 (&sc)[2][QB],
                                            f32x16 (&sn)[2][QB], float c) {
    constexpr int nS = kKFrags * QB;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    float mc[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) mc[qb] = m[qb] * c;
    bf16x8 kf[kKFrags];
    bf16x8 vf[kVFrags];
    bf16x2 pr[QB][2][2][4];
    bf16x8 pk[QB][2][2];
    float t[QB][8];

#pragma unroll
    for (int i = 0; i < kPf; ++i) kf[i] = kfrag(kt, i);
    __builtin_amdgcn_sched_barrier(0);

    // phase A: S of the next tile + exp of this tile
#pragma unroll
    for (int i = 0; i < kKFrags; ++i) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int ds = i >> 1, kb = i & 1;
        sn[kb][qb] = mfma32(kf[i], qfrag(qb, ds), ds == 0 ? f32x16{} : sn[kb][qb]);
        const int mi = i * QB + qb;
#pragma unroll
        for (int e = mi * kPairs / nS; e < (mi + 1) * kPairs / nS; ++e) {
          const int eq = e / 16, kb2 = (e / 8) & 1, cc = (e / 4) & 1, w = e & 3;
          const float e0 = fast_exp2(__builtin_fmaf(sc[kb2][eq][cc * 8 + 2 * w], c, -mc[eq]));
          const float e1 = fast_exp2(__builtin_fmaf(sc[kb2][eq][cc * 8 + 2 * w + 1], c, -mc[eq]));
          pr[eq][kb2][cc][w] = pack_bf16(e0, e1);
          l[eq] = __builtin_amdgcn_fdot2_f32_bf16(pr[eq][kb2][cc][w], ones, l[eq], false);
          if (w == 3)
            pk[eq][kb2][cc] = join8(pr[eq][kb2][cc][0], pr[eq][kb2][cc][1], pr[eq][kb2][cc][2], pr[eq][kb2][cc][3]);
        }
      }
      if (i + kPf < kKFrags)
        kf[i + kPf] = kfrag(kt, i + kPf);
      else
        vf[i + kPf - kKFrags] = vfrag(vt, i + kPf - kKFrags);
      __builtin_amdgcn_sched_barrier(0);
    }

    // phase B: P V of this tile + row max of the next tile
#pragma unroll
    for (int j = 0; j < kVFrags; ++j) {
      const int kc = j / C::kDBlocks, db = j % C::kDBlocks;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) o[qb][db] = mfma32(vf[j], pk[qb][kc >> 1][kc & 1], o[qb][db]);
      if (j + kPf < kVFrags) vf[j + kPf] = vfrag(vt, j + kPf);
      if (j >= kMaxStart) {
        constexpr int nPos = kVFrags - kMaxStart;
        const int p = j - kMaxStart;
#pragma unroll
        for (int u = p * kMaxUnits / nPos; u < (p + 1) * kMaxUnits / nPos; ++u) {
          if (u < 8 * QB) {  // max of four scores
            const int qb = u / 8, i = u % 8, kb = i >> 2, r = (i & 3) * 4;
            t[qb][i] = __builtin_fmaxf(__builtin_fmaxf(sn[kb][qb][r], sn[kb][qb][r + 1]),
                                       __builtin_fmaxf(sn[kb][qb][r + 2], sn[kb][qb][r + 3]));
          } else {  // combine, then across the two halves of the wave
            const int qb = u - 8 * QB;
            const float a = __builtin_fmaxf(__builtin_fmaxf(t[qb][0], t[qb][1]), __builtin_fmaxf(t[qb][2], t[qb][3]));
            const float b = __builtin_fmaxf(__builtin_fmaxf(t[qb][4], t[qb][5]), __builtin_fmaxf(t[qb][6], t[qb][7]));
            mx[qb] = max_halves(__builtin_fmaxf(a, b));
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // O^T += V^T P^T from V ring slot vt (see vslot)
  __device__ __forceinline__ void accumulate(const lds_char* vt, const bf16x8 (&pk)[QB][2][2]) {
#pragma unroll
    for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const int rows = (kb * 32 + cc * 16) * D * 2;
          const s16x4 va = ds_read_tr(vt + voff[db][0] + rows);
          const s16x4 vb = ds_read_tr(vt + voff[db][1] + rows);
          const s16x8 v8 = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
          const bf16x8 vf = __builtin_bit_cast(bf16x8, v8);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) o[qb][db] = mfma32(vf, pk[qb][kb][cc], o[qb][db]);
        }
  }
};

// SMALL: N < 64, a single tile whose missing rows are clamped per lane.
template <int D, bool CAUSAL, int QB, int W, bool SMALL>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * W, 64 * W),
                          amdgpu_waves_per_eu(FwdCfg<D, QB, W>::kWavesPerEU, FwdCfg<D, QB, W>::kWavesPerEU))) void
fwd_bf16_kernel(FwdArgs a, TileSched sched) {
  using C = FwdCfg<D, QB, W>;
  constexpr int NB = C::kNB;
  constexpr int kWaves = C::kWaves;
  __shared__ __attribute__((aligned(1024))) char smem_raw[C::kLdsBytes];
  FwdKernel<D, CAUSAL, QB, W> k;
  k.smem = (lds_char*)smem_raw;

  const int tid = threadIdx.x;
  k.wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps wave-derived values scalar
  k.lane = tid & 63;
  k.l32 = k.lane & 31;
  k.half = k.lane >> 5;
  const int wave = k.wave, lane = k.lane;

  int qtile, bh;
  sched_item(sched, blockIdx.x, qtile, bh);
  const int N = a.N;
  const size_t head_off = (size_t)bh * N * D;
  const __bf16* __restrict__ Q = (const __bf16*)a.q + head_off;
  const __bf16* __restrict__ K = (const __bf16*)a.k + head_off;
  const __bf16* __restrict__ V = (const __bf16*)a.v + head_off;

  const int q0 = qtile * C::kBlockM;
  const int wq0 = q0 + wave * C::kRowsPerWave;
  const bool wave_active = wq0 < N;
  const int n_ktiles_all = (N + kBlockN - 1) / kBlockN;
  int nt = n_ktiles_all;
  int wave_last = n_ktiles_all - 1;
  if constexpr (CAUSAL) {
    nt = min(q0 + C::kBlockM - 1, N - 1) / kBlockN + 1;
    wave_last = min(wq0 + C::kRowsPerWave - 1, N - 1) / kBlockN;
  }
  const bool ragged = (N % kBlockN) != 0;

  // Processing order.  Online softmax does not depend on the order of the
  // key tiles, so the tiles that need a mask go first: the block's diagonal
  // region under causal masking (tiles q0/64 .. nt-1), else a ragged last
  // tile (or the single tile of a short tensor), else none.  These R tiles
  // run through a plain serial step; the remaining main tiles 0 .. nt-R-1
  // are below every wave's diagonal and run through the pipelined step,
  // which then needs no mask code and no per-wave skip.
  int first_masked = nt;
  if (SMALL) first_masked = 0;
  else if (CAUSAL) first_masked = q0 / kBlockN;
  else if (ragged) first_masked = n_ktiles_all - 1;
  const int R = nt - first_masked;
  // tile at sequence position p (positions past the end repeat the last tile)
  auto seq_tile = [&](int p) { return p < R ? first_masked + p : p - R; };
  // First row of key tile t: tiles lie inside the tensor, a ragged last
  // tile is shifted back to end at row N-1 (its keys below t*64 are masked).
  auto tile_row0 = [&](int t) { return SMALL ? 0 : min(min(t, n_ktiles_all - 1) * kBlockN, N - kBlockN); };
  // Ring slots are counted from the first main position, so that the
  // unrolled main loop sees compile-time slots.
  auto ring = [&](int p) { return ((p - R) % NB + NB) % NB; };

  // Load group g = (K at position g+1, V at position g).  Groups past the
  // end repeat the last tile: they keep the per-step vmcnt count fixed and
  // are never read.
  RowTileCopier<D, kBlockN, kWaves> cp;
  cp.init(wave, lane);
  auto issue_k = [&](int p, int b) {
    if constexpr (SMALL) cp.copy_clamped(K, N, 0, k.kbuf(b));
    else cp.copy(K, tile_row0(seq_tile(p)), k.kbuf(b));
  };
  auto issue_v = [&](int p, int b) {
    if constexpr (SMALL) cp.copy_clamped(V, N, 0, k.vbuf(b));
    else cp.copy(V, tile_row0(seq_tile(p)), k.vbuf(b));
  };

  issue_k(0, ring(0));
  if constexpr (C::kQInLds) {  // this wave's Q rows, behind K at position 0 in the load order
    RowTileCopier<D, C::kRowsPerWave, 1> cq;
    cq.init(0, lane);
    if (wq0 + C::kRowsPerWave <= N)
      cq.copy(Q, wq0, k.qtile());
    else
      cq.copy_clamped(Q, N, min(wq0, N - 1), k.qtile());
  }
#pragma unroll
  for (int g = 0; g < NB - 1; ++g) {
    issue_k(g + 1, ring(g + 1));
    issue_v(g, ring(g));
  }

  // per-lane loop-invariant LDS offsets (row offsets of kb/cc blocks keep the swizzle)
#pragma unroll
  for (int ds = 0; ds < C::kDSteps; ++ds) k.koff[ds] = lds_off_bytes<D>(k.l32, ds * 2 + k.half);
  {
    const int g = lane >> 4, j16 = lane & 15;
#pragma unroll
    for (int db = 0; db < C::kDBlocks; ++db) {
      const int dcol = db * 32 + (g & 1) * 16 + (j16 & 3) * 4;
      const int r1 = k.half * 4 + (j16 >> 2);
#pragma unroll
      for (int t = 0; t < 2; ++t)
        k.voff[db][t] = NB * C::kTileBytes + lds_off_bytes<D>(r1 + 8 * t, dcol >> 3) + (dcol & 7) * 2;
    }
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    int row = wq0 + qb * 32 + k.l32;
    row = row < N ? row : N - 1;
    if constexpr (!C::kQInLds) {
#pragma unroll
      for (int ds = 0; ds < C::kDSteps; ++ds) k.qf[qb][ds] = *(const bf16x8*)(Q + (size_t)row * D + ds * 16 + k.half * 8);
    }
#pragma unroll
    for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) k.o[qb][db][r] = 0.f;
    k.m[qb] = -__builtin_inff();
    k.l[qb] = 0.f;
  }
  const float c = a.scale_log2;

  // ---- masked region: serial steps, position p = tile first_masked + p
  for (int p = 0; p < R; ++p) {
    // group p holds V at p; K at p came with group p-1 (K at 0 and Q first)
    wait_vmcnt<(NB - 2) * C::kLoadsPerGroup>();
    __syncthreads();
    const int t = first_masked + p;
    if (wave_active && t <= wave_last) {
      bf16x8 pk[QB][2][2];
      k.scores(k.kbuf(ring(p)), k.s[0]);
      if (SMALL || (CAUSAL && t == wave_last) || (ragged && t == n_ktiles_all - 1))
        k.mask(k.s[0], tile_row0(t), t * kBlockN, wq0, N);
      k.rowmax(k.s[0]);
      k.update_max(c);
      k.exponentiate(k.s[0], c, pk);
      k.accumulate(k.vslot(ring(p)), pk);
    }
    __syncthreads();  // K at p is read in this step: refill its slot only now
    issue_k(p + NB, ring(p + NB));
    issue_v(p + NB - 1, ring(p + NB - 1));
  }

  // ---- main region: pipelined steps at positions p = R .. nt-1
  const int n_main = nt - R;
  if (n_main > 0) {
    // K at position R: K at 0 (and Q) when there is no masked region, else
    // it came with group R-1, which the last masked step waited for.
    if (R == 0) {
      wait_vmcnt<(NB - 1) * C::kLoadsPerGroup>();
      __syncthreads();
    }
    k.scores(k.kbuf(0), k.s[0]);
    k.rowmax(k.s[0]);
  }
  // One step at position p (main index i = p - R): wait for group p
  // (K at p+1, V at p), refill, then S at p+1 alongside exp(S at p), then
  // P V at p alongside rowmax(S at p+1).  Ring slot and score set are the
  // compile-time constants i % NB and i % 2.
  auto step = [&](int p, auto bconst, auto curconst) {
    constexpr int b = decltype(bconst)::value;
    constexpr int cur = decltype(curconst)::value;
    wait_vmcnt<(NB - 2) * C::kLoadsPerGroup>();
    __syncthreads();
    issue_k(p + NB, b);
    issue_v(p + NB - 1, (b + NB - 1) % NB);
    k.update_max(c);
    k.pipelined(k.kbuf((b + 1) % NB), k.vslot(b), k.s[cur], k.s[cur ^ 1], c);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2 % NB>;
  using I3 = std::integral_constant<int, 3 % NB>;
  using I4 = std::integral_constant<int, 4 % NB>;
  using I5 = std::integral_constant<int, 5 % NB>;
  // unrolled over lcm(2, NB) steps so that ring slot and score set are static
  for (int i = 0; i < n_main; i += 2 * NB) {
    const int p = R + i;
    step(p, I0(), I0());
    if (i + 1 >= n_main) break;
    step(p + 1, I1(), I1());
    if (i + 2 >= n_main) break;
    if constexpr (NB == 3) {
      step(p + 2, I2(), I0());
      if (i + 3 >= n_main) break;
      step(p + 3, I3(), I1());
      if (i + 4 >= n_main) break;
      step(p + 4, I4(), I0());
      if (i + 5 >= n_main) break;
      step(p + 5, I5(), I1());
    } else {
      step(p + 2, I0(), I0());
      if (i + 3 >= n_main) break;
      step(p + 3, I1(), I1());
    }
  }
  wait_vmcnt<0>();  // no direct-to-LDS copy may outlive the workgroup

  // ---- epilogue: O = acc / l, L = m*scale + ln l
  if (!wave_active) return;
  __bf16* __restrict__ O = (__bf16*)a.o + head_off;
  float* __restrict__ Lse = a.lse + (size_t)bh * N;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = sum_halves(k.l[qb]);
    const float inv = 1.0f / lt;
    const int row = wq0 + qb * 32 + k.l32;
    if (row < N) {
#pragma unroll
      for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          u32x2 w = {pack_bf16_u32(k.o[qb][db][g4 * 4 + 0] * inv, k.o[qb][db][g4 * 4 + 1] * inv),
                     pack_bf16_u32(k.o[qb][db][g4 * 4 + 2] * inv, k.o[qb][db][g4 * 4 + 3] * inv)};
          *(u32x2*)(O + (size_t)row * D + db * 32 + g4 * 8 + k.half * 4) = w;
        }
      if (k.half == 0) Lse[row] = k.m[qb] * a.scale + fast_log2(lt) * kLn2;
    }
  }
}

}  // namespace fwd
}  // namespace fa
