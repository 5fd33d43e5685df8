// fa_fwd_bf16.h -- exact-attention forward kernel template, bf16 in/out, gfx950.
// Instantiated in fa_fwd_bf16.hip (D = 64, 128) and fa_fwd_bf16_d256.hip.
//
// One workgroup = 8 waves at D = 128 (two per SIMD), 4 waves at D = 64
// (three workgroups per CU) and at D = 256 (one wave per SIMD, each tile's
// keys split between two waves of the same rows); a wave owns 32*QB query
// rows of one (batch, head) and the loop over keys for them.  The streaming structure is the one every page
// describes ("Learning Metal with FlashAttention", section FlashAttention;
// "Flash Attention" page, kernel anatomy; metal-flash-attention README,
// "Quantifying performance", forward pseudocode): the Q rows are loaded once
// and stay in registers, K and V stream through LDS in tiles of 64 keys, the
// running row max m and row sum l rescale the unnormalised accumulator, and
// the score matrix only ever exists as MFMA accumulator registers.
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
// * Software pipeline inside each wave, written in issue order: phase A
//   issues the score MFMAs of tile j+1, each carrying a share of the
//   exponentials of tile j; phase B issues the P V MFMAs of tile j.
// * K/V tiles go global -> LDS with 16-byte direct loads (no VGPR staging)
//   into a ring of NB slots per tensor (4 at D = 128, else 2), issued up to
//   4 steps ahead.  The loop is
//   unrolled over the ring so every LDS address is a per-lane offset
//   computed once plus an instruction immediate.  Rows are XOR-swizzled in
//   16-byte chunks (see swz) so that both LDS read patterns are free of bank
//   conflicts.
// * exp is exp2 with scale*log2(e) folded into one FMA per score.  The
//   running max m is only a reference point: any m gives the same O and L
//   as long as no exp2(s*c - m*c) overflows.  So the tiles after the first
//   are exponentiated against the current m without computing their row
//   max; each lane's share of the tile's row sum (its P values of the tile)
//   is then checked against 2^16, which bounds every P of the tile.  Only
//   when a lane of the wave exceeds it (or got inf) does the wave take the
//   row max of the tile, raise m, rescale O and l, and redo the tile's
//   exponentials, all before the P V products read P.
// * Causal masking skips every key tile above the workgroup's last row.
//   The tiles that need a mask (the block's diagonal region, or a ragged
//   last tile) come first in the processing order and run through the same
//   pipelined step, with the mask applied to their scores between the two
//   phases.
#pragma once

#include <type_traits>
#include <utility>

#include "fa_device.h"
#include "fa_kernels.h"
#include "fa_sched.h"

namespace fa {
namespace fwd {

constexpr int kBlockN = 64;                // keys per K/V tile
constexpr float kRescaleThreshold = 8.0f;  // exp2-domain growth allowed before O is rescaled
constexpr float kMaxFloor = 1.0e30f;       // the running max starts at -kMaxFloor
constexpr float kTileSumLimit = 65536.0f;  // bound on a lane's share of a tile's row sum

// QREG: keep the Q rows in registers even where the layout would put them in
// LDS (the block-sparse instances of the 256-wide layout need that LDS for
// their tile list).
template <int D, int QB, int W, bool QREG = false>
struct FwdCfg {
  static constexpr int kWaves = W;                       // waves per workgroup (4 or 8)
  static constexpr int kRowsPerWave = 32 * QB;
  // Row width of the LDS tiles: D rounded up to 64, 128 or 256.  D = 32, 96
  // and 160 keep the layout (and swizzle) of D = 64, 128 and 256 with the
  // chunks past D unused; global rows are D wide.
  static constexpr int kDP = D <= 64 ? 64 : D <= 128 ? 128 : 256;
  static_assert(D % 32 == 0 && D <= 256, "head dimension");
  // Key split: with kSplit = 2 the two 32-key halves of every tile go to two
  // waves that own the same query rows; their partial results are merged
  // at the end.  D = 256 uses it: its work is B*H*N/32 waves of 32 rows,
  // which without the split fills only half of the SIMDs at the sizes of
  // interest (and it halves the score registers of a wave).
  static constexpr int kSplit = kDP == 256 ? 2 : 1;
  static constexpr int kKB = 2 / kSplit;                 // 32-key blocks a wave takes per tile
  static constexpr int kQBlocks = kWaves / kSplit;       // waves with distinct query rows
  static constexpr int kBlockM = kQBlocks * kRowsPerWave;  // query rows per workgroup
  static constexpr int kDSteps = D / 16;                 // k-steps of the S product
  static constexpr int kDBlocks = D / 32;                // 32-wide d blocks of O
  static constexpr int kTileBytes = kBlockN * kDP * 2;   // one K or V tile in LDS
  // K/V ring: kNB slots each; K of position p is issued kLeadK steps
  // before the step that first reads it, V kLeadV steps before.  Step p
  // reads K(p+1) and V(p) and refills the slots of K(p) and V(p-1).
  static constexpr int kNB = kDP == 128 ? 4 : 2;
  static constexpr int kLeadK = kNB;
  static constexpr int kLeadV = kNB - 1;
  static constexpr int kRingBytes = 2 * kNB * kTileBytes;
  // Q rows in LDS (D = 256) instead of registers: with them in registers
  // the O accumulators no longer fit beside the rest and the compiler
  // copies them between VGPRs and AGPRs around every P V MFMA.
  static constexpr bool kQInLds = kDP == 256 && !QREG;
  static constexpr int kQBytes = kQInLds ? kQBlocks * 32 * QB * kDP * 2 : 0;
  static constexpr int kLdsBytes = kRingBytes + kQBytes;
  static_assert(kLdsBytes <= 160 * 1024, "LDS of one workgroup");
  static_assert(!kQInLds || QB == 1, "Q fragments from LDS are read for one 32-row block");
  // merge of a key split: per query block, 64 lanes x (O accumulators + m + l) floats
  static constexpr int kMergeFloats = QB * kDBlocks * 16 + 2 * QB;
  static_assert(kSplit == 1 || kLdsBytes >= kQBlocks * 64 * 4 * kMergeFloats,
                "the merge of a key split reuses the ring");
  // direct-to-LDS loads per wave for one K or V tile
  static constexpr int kLoadsPerTile = kTileBytes / 16 / kWaves / 64;
  // Loads a step may leave in flight when it starts (those of the
  // kStepsInFlight previous steps): its barrier must publish K(p+1) and V(p).
  static constexpr int kStepsInFlight = kNB - 2;
  static_assert(kNB % 2 == 0, "the loop is unrolled over the ring and the two score sets");
  static constexpr int kUnroll = kNB;
  // Waves per SIMD the register budget is cut for: two (<= 256 VGPRs) for
  // the 8-wave workgroups of D = 128; three (<= 168 VGPRs) at D = 64, where
  // three 4-wave workgroups share a CU (32 KB ring each) and the third wave
  // per SIMD hides more of the exponentials, which at D = 64 cost as much
  // issue time as the MFMAs; one for D = 256 (4 waves, 128 KB ring).
  static constexpr int kWavesPerEU = kDP == 64 ? 3 : W == 8 ? 2 : 1;
  // Where a step issues its ring refills: right after its barrier, or (D =
  // 128, ring of 4) after phase A, which keeps the copies' address and M0
  // set-up off the path from the barrier to the first score MFMAs.  The
  // 2-slot ring of D = 256 cannot spare the half step of lead.
  static constexpr bool kLateRefill = kDP == 128;
  // 256-wide rows: the refill loads go between the step's MFMAs instead
  // (K tile during phase A, V tile during phase B, about one load per two
  // MFMAs).  Issued in one burst, the 16 loads of 1 KB per wave stalled
  // the wave for about a thousand cycles a step while the vector memory
  // path drained them, with the matrix core idle.
  static constexpr bool kSpreadRefill = kDP == 256;
};

template <int D, bool CAUSAL, int QB, int W, bool QREG = false>
struct FwdKernel {
  using C = FwdCfg<D, QB, W, QREG>;
  static constexpr int NB = C::kNB;
  static constexpr int KB = C::kKB;

  // per-wave state
  // Q^T as B operands: query column l32, d = ds*16 + half*8 + 0..7 (in
  // registers, or read from the LDS copy at qoff with kQInLds)
  bf16x8 qf[C::kQInLds ? 1 : QB][C::kQInLds ? 1 : C::kDSteps];
  int qoff[8];
  f32x16 o[QB][C::kDBlocks];  // O^T accumulators
  f32x16 s[2][KB][QB];        // two score tiles in ping-pong: [set][kb][qb]
  bf16x8 pk[QB][KB][2];       // P of the tile in flight, as B operands
  float m[QB], l[QB], mx[QB], lt[QB];  // lt: this lane's share of the current tile's row sums
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

  // S^T tile from the K buffer kt: acc[kb][qb]
  __device__ __forceinline__ void scores(const lds_char* kt, f32x16 (&acc)[KB][QB]) {
#pragma unroll
    for (int ds = 0; ds < C::kDSteps; ++ds)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 kf = *(const bf16x8 __attribute__((address_space(3)))*)(kt + koff[ds] + kb * 32 * C::kDP * 2);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) acc[kb][qb] = mfma32(kf, qfrag(qb, ds), ds == 0 ? f32x16{} : acc[kb][qb]);
      }
  }

  // -inf where a key is invisible: above the causal diagonal, past N, or
  // (in a ragged last tile, loaded shifted to end at row N-1) already
  // covered by the previous tile.  key0 is the tile's first row, kmin the
  // first key the tile contributes.
  __device__ __forceinline__ void mask(f32x16 (&acc)[KB][QB], int key0, int kmin, int wq0, int N) {
    // Element (kb, r) of this lane holds key base + off with a compile-time
    // offset off; the visible keys are the offsets in [lo, hi).
    const int base = key0 + half * 4;
    const int lo = kmin - base;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      int hi = N - base;
      if constexpr (CAUSAL) hi = min(hi, wq0 + qb * 32 + l32 + 1 - base);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = kb * 32 + (r >> 2) * 8 + (r & 3);
          acc[kb][qb][r] = (off >= lo && off < hi) ? acc[kb][qb][r] : -__builtin_inff();
        }
    }
  }

  // Row max of a score tile (both halves agree afterwards).
  __device__ __forceinline__ void rowmax(const f32x16 (&acc)[KB][QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float t[4 * KB];
#pragma unroll
      for (int i = 0; i < 4 * KB; ++i) t[i] = max4(acc[i >> 2][qb], (i & 3) * 4);
      mx[qb] = max_halves(maxn(t));
    }
  }
  __device__ __forceinline__ static float max4(const f32x16& a, int r) {
    return __builtin_fmaxf(__builtin_fmaxf(a[r], a[r + 1]), __builtin_fmaxf(a[r + 2], a[r + 3]));
  }
  __device__ __forceinline__ static float maxn(const float (&t)[4 * KB]) {
    float a = __builtin_fmaxf(__builtin_fmaxf(t[0], t[1]), __builtin_fmaxf(t[2], t[3]));
#pragma unroll
    for (int i = 4; i < 4 * KB; i += 4)
      a = __builtin_fmaxf(a, __builtin_fmaxf(__builtin_fmaxf(t[i], t[i + 1]), __builtin_fmaxf(t[i + 2], t[i + 3])));
    return a;
  }

  // Raise the running max to include mx; rescale O and l when it grew by
  // more than the threshold in any lane of the wave (a wave-uniform branch;
  // rows that grew less keep their reference point).
  // The running max starts at a finite floor, not -inf: a row may see only
  // masked keys in its first tiles, and exp2(-inf - floor) is then 0.
  __device__ __forceinline__ void update_max(float c) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float m_new = __builtin_fmaxf(m[qb], mx[qb]);
      const bool grow = (m_new - m[qb]) * c > kRescaleThreshold;
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        const float alpha = fast_exp2((m[qb] - m_new) * c);  // 0 on the first tile (m at the floor)
#pragma unroll
        for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[qb][db][r] *= alpha;
        l[qb] *= alpha;
        m[qb] = m_new;
      }
    }
  }

  // Exponentials of a whole score tile against the running max: P as bf16
  // B operands in pk, this lane's share of the row sums (over the rounded
  // P) in lt.
  __device__ __forceinline__ void exp_tile(const f32x16 (&sc)[KB][QB], float c) {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float mc = m[qb] * c;
      lt[qb] = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          bf16x2 pr[4];
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            pr[w] = pack_bf16(fast_exp2(__builtin_fmaf(sc[kb][qb][cc * 8 + 2 * w], c, -mc)),
                              fast_exp2(__builtin_fmaf(sc[kb][qb][cc * 8 + 2 * w + 1], c, -mc)));
            lt[qb] = __builtin_amdgcn_fdot2_f32_bf16(pr[w], ones, lt[qb], false);
          }
          pk[qb][kb][cc] = join8(pr[0], pr[1], pr[2], pr[3]);
        }
    }
  }

  // After the exponentials of tile sc: if a lane's share of a row sum is
  // above kTileSumLimit or not finite, raise the running max to the tile's
  // row max (rescaling O and l) and redo the tile; then add the tile's sums.
  __device__ __forceinline__ void settle_tile(const f32x16 (&sc)[KB][QB], float c) {
    bool over = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) over |= !(lt[qb] <= kTileSumLimit);
    if (__builtin_amdgcn_ballot_w64(over) != 0) {
      rowmax(sc);
      update_max(c);
      exp_tile(sc, c);
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) l[qb] += lt[qb];
  }

  // ---- the two halves of a pipelined step, written in issue order -----
  // Phase A issues the score MFMAs of the next tile, each carrying its
  // share of this tile's exponentials (P rounded to bf16, row sum over the
  // rounded P).  Phase B issues the P V MFMAs of this tile.  LDS fragments
  // are read kPf fragments ahead of the MFMA that consumes them.
  // sched_barrier fences keep the compiler from regrouping the sequence (it
  // would otherwise cluster reads next to their use and the MFMAs of one
  // product together).
  static constexpr int kKFrags = KB * C::kDSteps;      // K fragments per tile, QB MFMAs each
  static constexpr int kVFrags = 2 * KB * C::kDBlocks;  // V fragments per tile, QB MFMAs each
  static constexpr int kPf = 3;                    // read-ahead in fragments
  static constexpr int nS = kKFrags * QB;          // score MFMAs per step
  static constexpr int nP = kVFrags * QB;          // P V MFMAs per step
  static constexpr int kPairs = 8 * KB * QB;       // exp pairs per tile and lane

  // Q fragment for k-step ds (block qb): the swizzle of a D = 256 row
  // repeats past chunk 16, so k-steps 8.. are the first eight + 256 bytes
  __device__ __forceinline__ bf16x8 qfrag(int qb, int ds) const {
    if constexpr (C::kQInLds)
      return *(const bf16x8 __attribute__((address_space(3)))*)(smem + qoff[ds % 8] + (ds / 8) * 256);
    else
      return qf[qb][ds];
  }

  // K fragment i = (ds, kb) = (i / KB, i % KB)
  __device__ __forceinline__ bf16x8 kfrag(const lds_char* kt, int i) const {
    return *(const bf16x8 __attribute__((address_space(3)))*)(kt + koff[i / KB] + (i % KB) * 32 * C::kDP * 2);
  }
  // V fragment j = (kb, cc, db): (kb, cc) = j / kDBlocks, db = j % kDBlocks
  __device__ __forceinline__ bf16x8 vfrag(const lds_char* vt, int j) const {
    const int kc = j / C::kDBlocks, db = j % C::kDBlocks;
    const int rows = ((kc >> 1) * 32 + (kc & 1) * 16) * C::kDP * 2;
    const s16x4 va = ds_read_tr(vt + voff[db][0] + rows);
    const s16x4 vb = ds_read_tr(vt + voff[db][1] + rows);
    const s16x8 v8 = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
    return __builtin_bit_cast(bf16x8, v8);
  }

  // Loads n of a refill of L loads that go after MFMA i of M: [i L / M, (i + 1) L / M)
  template <typename R>
  __device__ __forceinline__ static void refill_after(R& refill, int i, int M) {
    constexpr int L = C::kLoadsPerTile;
#pragma unroll
    for (int n = i * L / M; n < (i + 1) * L / M; ++n) refill(n);
  }

  // S of the next tile (K buffer kt, into sn) + exp of this tile (sc);
  // refill(n) issues load n of a K refill (with kSpreadRefill).
  template <typename R>
  __device__ __forceinline__ void phase_a(const lds_char* kt, const f32x16 (&sc)[KB][QB], f32x16 (&sn)[KB][QB],
                                          float c, R& refill) {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    float mc[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      mc[qb] = m[qb] * c;
      lt[qb] = 0.f;
    }
    bf16x8 kf[kKFrags];
    bf16x8 qv[C::kQInLds ? C::kDSteps : 1];  // Q fragments read with the K fragments (kQInLds)
    bf16x2 pr[QB][KB][2][4];
#pragma unroll
    for (int i = 0; i < kPf; ++i) {
      kf[i] = kfrag(kt, i);
      if (C::kQInLds && i % KB == 0) qv[i / KB] = qfrag(0, i / KB);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kKFrags; ++i) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int ds = i / KB, kb = i % KB;
        sn[kb][qb] = mfma32(kf[i], C::kQInLds ? qv[ds] : qf[qb][ds], ds == 0 ? f32x16{} : sn[kb][qb]);
        // exp pairs e = (qb, kb, cc, w) carried by this MFMA
        const int mi = i * QB + qb;
#pragma unroll
        for (int e = mi * kPairs / nS; e < (mi + 1) * kPairs / nS; ++e) {
          const int eq = e / (8 * KB), kb2 = (e / 8) % KB, cc = (e / 4) & 1, w = e & 3;
          const float e0 = fast_exp2(__builtin_fmaf(sc[kb2][eq][cc * 8 + 2 * w], c, -mc[eq]));
          const float e1 = fast_exp2(__builtin_fmaf(sc[kb2][eq][cc * 8 + 2 * w + 1], c, -mc[eq]));
          pr[eq][kb2][cc][w] = pack_bf16(e0, e1);
          lt[eq] = __builtin_amdgcn_fdot2_f32_bf16(pr[eq][kb2][cc][w], ones, lt[eq], false);
          if (w == 3)
            pk[eq][kb2][cc] = join8(pr[eq][kb2][cc][0], pr[eq][kb2][cc][1], pr[eq][kb2][cc][2], pr[eq][kb2][cc][3]);
        }
      }
      if (i + kPf < kKFrags) {
        kf[i + kPf] = kfrag(kt, i + kPf);
        if (C::kQInLds && (i + kPf) % KB == 0) qv[(i + kPf) / KB] = qfrag(0, (i + kPf) / KB);
      }
      if constexpr (C::kSpreadRefill) refill_after(refill, i, kKFrags);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // P V of the tile whose P is in pk (V buffer vt); refill(n) issues load n
  // of a V refill (with kSpreadRefill).
  template <typename R>
  __device__ __forceinline__ void phase_b(const lds_char* vt, R& refill) {
    bf16x8 vf[kVFrags];
#pragma unroll
    for (int j = 0; j < kPf; ++j) vf[j] = vfrag(vt, j);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < kVFrags; ++j) {
      const int kc = j / C::kDBlocks, db = j % C::kDBlocks;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) o[qb][db] = mfma32(vf[j], pk[qb][kc >> 1][kc & 1], o[qb][db]);
      if (j + kPf < kVFrags) vf[j + kPf] = vfrag(vt, j + kPf);
      if constexpr (C::kSpreadRefill) refill_after(refill, j, kVFrags);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

// f(i + j, integral_constant<j>) for j = 0, 1, ... while i + j < n
template <typename F, int... J>
__device__ __forceinline__ void unrolled(int i, int n, F& f, std::integer_sequence<int, J...>) {
  (void)((i + J < n && (f(i + J, std::integral_constant<int, J>()), true)) && ...);
}

// SMALL: fewer than 64 keys, a single tile whose missing rows are clamped
// per lane.  KV: query and key lengths apart (a.N queries, a.Nk keys; the
// causal mask lines the queries up with the last keys), and with
// a.n_split > 1 the key tiles of a query block divided into a.n_split
// ranges, one workgroup each, whose results go to a.part_o / a.part_l for
// the merge kernel.  SPARSE: the square forward over the key tiles a block
// mask keeps (a.block_mask; see the list built below).  Without KV and
// SPARSE the kernel is the square forward.
template <int D, bool CAUSAL, int QB, int W, bool SMALL, bool KV = false, bool SPARSE = false>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * W, 64 * W),
                          amdgpu_waves_per_eu(FwdCfg<D, QB, W, SPARSE>::kWavesPerEU,
                                              FwdCfg<D, QB, W, SPARSE>::kWavesPerEU))) void
fwd_bf16_kernel(FwdArgs a, TileSched sched) {
  using C = FwdCfg<D, QB, W, SPARSE>;
  constexpr int NB = C::kNB;
  constexpr int LK = C::kLeadK, LV = C::kLeadV;
  constexpr int kWaves = C::kWaves;
  __shared__ __attribute__((aligned(1024))) char smem_raw[C::kLdsBytes];
  FwdKernel<D, CAUSAL, QB, W, SPARSE> k;
  k.smem = (lds_char*)smem_raw;

  const int tid = threadIdx.x;
  k.wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps wave-derived values scalar
  k.lane = tid & 63;
  k.l32 = k.lane & 31;
  k.half = k.lane >> 5;
  const int wave = k.wave, lane = k.lane;
  // query block and key half of this wave (kpart = 0 without a key split)
  const int qblk = wave % C::kQBlocks, kpart = wave / C::kQBlocks;

  int qtile, bh, split = 0;
  if constexpr (KV) {
    // the scheduler's items are (query tile, key range) pairs, heaviest
    // query tile first under causal masking
    int item;
    sched_item(sched, blockIdx.x, item, bh);
    qtile = item / a.n_split;
    split = item - qtile * a.n_split;
  } else {
    sched_item(sched, blockIdx.x, qtile, bh);
  }
  const int N = a.N;                                  // query rows
  const int Nk = KV ? a.Nk : N;                       // keys
  const int off = (KV && CAUSAL) ? Nk - N : 0;        // query i sees keys <= i + off
  const size_t head_off = (size_t)bh * N * D;
  const size_t kv_head_off = KV ? (size_t)bh * Nk * D : head_off;
  const __bf16* __restrict__ Q = (const __bf16*)a.q + head_off;
  const __bf16* __restrict__ K = (const __bf16*)a.k + kv_head_off;
  const __bf16* __restrict__ V = (const __bf16*)a.v + kv_head_off;

  const int q0 = qtile * C::kBlockM;
  const int wq0 = q0 + qblk * C::kRowsPerWave;
  const bool wave_active = wq0 < N;
  const int n_ktiles_all = (Nk + kBlockN - 1) / kBlockN;
  int nt_q = n_ktiles_all;  // key tiles the block sees
  if constexpr (CAUSAL) nt_q = min(q0 + C::kBlockM - 1 + off, Nk - 1) / kBlockN + 1;
  // this workgroup's key tiles [t_lo, t_hi)
  int t_lo = 0, t_hi = nt_q;
  if constexpr (KV) {
    t_lo = nt_q * split / a.n_split;
    t_hi = nt_q * (split + 1) / a.n_split;
    if (t_lo == t_hi) {
      // an empty key range (fewer tiles than ranges): its rows get O = 0 and
      // L = -inf, which gives the range weight 0 in the merge
      if (wave_active && kpart == 0) {
        float* __restrict__ Op = a.part_o + ((size_t)split * a.B * a.H + bh) * N * D;
        float* __restrict__ Lp = a.part_l + ((size_t)split * a.B * a.H + bh) * N;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int row = wq0 + qb * 32 + k.l32;
          if (row < N) {
#pragma unroll
            for (int c = 0; c < D / 8; ++c)
              *(f32x4*)(Op + (size_t)row * D + c * 8 + k.half * 4) = f32x4{0.f, 0.f, 0.f, 0.f};
            if (k.half == 0) Lp[row] = -__builtin_inff();
          }
        }
      }
      return;
    }
  }
  int nt = t_hi - t_lo;
  const bool ragged = (Nk % kBlockN) != 0;

  // Processing order.  Online softmax does not depend on the order of the
  // key tiles, so the R tiles that need a mask go first: the block's
  // diagonal region under causal masking (tiles q0/64 .. nt-1), else a
  // ragged last tile (or the single tile of a short tensor), else none.
  // Every wave processes every tile of its block; keys a wave may not see
  // are masked.
  int first_masked = nt_q;
  if (SMALL) first_masked = 0;
  else if (CAUSAL) first_masked = (q0 + off) / kBlockN;
  else if (ragged) first_masked = n_ktiles_all - 1;
  if constexpr (KV) first_masked = min(max(first_masked, t_lo), t_hi);
  const int R = t_hi - first_masked;

  // Block-sparse: the list of key tiles the block processes, in LDS.  Tile
  // t is kept if any 64-row sub-block of the query block sees it; its entry
  // is t | (sub-blocks that see it) << 16 | (needs an elementwise mask) << 23.
  // A tile needs the mask if some sub-block does not see it, or it is in
  // the causal diagonal region, the ragged last tile or the single tile of
  // a short tensor.  Kept tiles go in ascending order (the online softmax
  // does not depend on the order).
  constexpr int kSubBlocks = C::kBlockM / kSparseBlock;
  static_assert(!SPARSE || (kSubBlocks >= 1 && kSubBlocks <= 7 && C::kRowsPerWave <= kSparseBlock),
                "sub-block bits of a list entry");
  __shared__ uint8_t sp_flags[SPARSE ? kSparseMaxTiles : 1];
  __shared__ uint32_t sp_list[SPARSE ? kSparseMaxTiles : 1];
  __shared__ int sp_count[1];
  const int sub_block = qblk * C::kRowsPerWave / kSparseBlock;  // this wave's 64-row sub-block
  if constexpr (SPARSE) {
    const int nb = n_ktiles_all;
    const unsigned char* __restrict__ bm = a.block_mask + (a.mask_heads == 1 ? (size_t)0 : (size_t)bh * nb * nb);
    const int a0 = q0 / kSparseBlock;
    unsigned valid = 0;
#pragma unroll
    for (int sb = 0; sb < kSubBlocks; ++sb) valid |= (a0 + sb < nb ? 1u : 0u) << sb;
    for (int t = tid; t < nt; t += 64 * kWaves) {
      unsigned vis = 0;
#pragma unroll
      for (int sb = 0; sb < kSubBlocks; ++sb)
        if (a0 + sb < nb && bm[(size_t)(a0 + sb) * nb + t] != 0) vis |= 1u << sb;
      const bool needs = vis != valid || t >= first_masked;
      sp_flags[t] = (uint8_t)(vis == 0 ? 0u : (vis | (needs ? 0x80u : 0u)));
    }
    __syncthreads();
    if (wave == 0) {
      int count = 0;
      for (int c0 = 0; c0 < nt; c0 += 64) {
        const int t = c0 + lane;
        const unsigned f = t < nt ? sp_flags[t] : 0u;
        const uint64_t kept = __builtin_amdgcn_ballot_w64(f != 0);
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(kept >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)kept, 0u));
        if (f != 0) sp_list[count + below] = (uint32_t)t | (f << 16);
        count += __builtin_popcountll(kept);
      }
      if (lane == 0) sp_count[0] = count;
    }
    __syncthreads();
    nt = __builtin_amdgcn_readfirstlane(sp_count[0]);
    if (nt == 0) {
      // no key tile kept: every row sees no key, O = 0 and L = -inf
      if (wave_active && kpart == 0) {
        __bf16* __restrict__ O = (__bf16*)a.o + head_off;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int row = wq0 + qb * 32 + k.l32;
          if (row < N) {
#pragma unroll
            for (int c = 0; c < D / 8; ++c) *(u32x2*)(O + (size_t)row * D + c * 8 + k.half * 4) = u32x2{0u, 0u};
            if (k.half == 0) a.lse[(size_t)bh * N + row] = -__builtin_inff();
          }
        }
      }
      return;
    }
  }
  // list entry of sequence position p (clamped to the last one)
  auto sp_entry = [&](int p) -> uint32_t {
    return __builtin_amdgcn_readfirstlane(sp_list[min(p, nt - 1)]);
  };
  auto needs_mask = [&](int p) -> bool {
    if constexpr (SPARSE) return (sp_entry(p) >> 23) & 1u;
    else return p < R;
  };
  // tile at sequence position p (positions past the end load a valid tile
  // that is never read)
  auto seq_tile = [&](int p) -> int {
    if constexpr (SPARSE) return (int)(sp_entry(p) & 0xffffu);
    else return p < R ? first_masked + p : t_lo + p - R;
  };
  // First row of key tile t: tiles lie inside the tensor, a ragged last
  // tile is shifted back to end at row Nk-1 (its keys below t*64 are masked).
  auto tile_row0 = [&](int t) { return SMALL ? 0 : min(min(t, n_ktiles_all - 1) * kBlockN, Nk - kBlockN); };
  auto mask_tile = [&](f32x16 (&acc)[C::kKB][QB], int p) {
    const int t = seq_tile(p);
    k.mask(acc, tile_row0(t) + kpart * 32, t * kBlockN, wq0 + off, Nk);
    if constexpr (SPARSE) {
      // the whole tile is invisible to this wave's sub-block
      if (((sp_entry(p) >> (16 + sub_block)) & 1u) == 0) {
#pragma unroll
        for (int kb = 0; kb < C::kKB; ++kb)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[kb][qb][r] = -__builtin_inff();
      }
    }
  };

  // Byte offset of the tile at sequence position p within the head: the
  // same tile as tile_row0(seq_tile(p)) (min(t * 64, N - 64) covers both
  // clamps), in 32 bits (a head holds fewer than 2^31 elements).
  const uint32_t last_tile_bytes = (uint32_t)(Nk - kBlockN) * (D * 2);
  auto tile_bytes = [&](int p) {
    const int t = seq_tile(p);
    return min((uint32_t)t * (kBlockN * D * 2), last_tile_bytes);
  };

  // K and V of sequence position p go to ring slot p % NB.
  RowTileCopier<D, C::kDP, kBlockN, kWaves> cp;
  cp.init(wave, lane);
  auto issue_k = [&](int p, int b) {
    if constexpr (SMALL) cp.copy_clamped(K, Nk, 0, k.kbuf(b));
    else cp.copy_at(K, tile_bytes(p), k.kbuf(b));
  };
  auto issue_v = [&](int p, int b) {
    if constexpr (SMALL) cp.copy_clamped(V, Nk, 0, k.vbuf(b));
    else cp.copy_at(V, tile_bytes(p), k.vbuf(b));
  };
  // Prologue loads, oldest first, in the order the first steps need them:
  // K0, then K(i+1), V(i) for i = 0, 1, ...  Only K0 K1 V0 go before the Q
  // rows are loaded: the compiler cannot see these copies and waits for
  // every load in flight before it first uses Q, so the rest is issued
  // after the first score tile.
  if constexpr (C::kQInLds) {
    // this workgroup's query rows (clamped onto N-1) go to LDS after the
    // ring, oldest of the prologue copies so the first wait covers them
    RowTileCopier<D, C::kDP, C::kBlockM, kWaves> qcp;
    qcp.init(wave, lane);
    qcp.copy_clamped(Q, N, q0, k.smem + C::kRingBytes);
  }
  issue_k(0, 0);
  issue_k(1, 1);
  issue_v(0, 0);
  auto issue_rest_of_prologue = [&]() {
#pragma unroll
    for (int i = 1; i < LK - 1; ++i) {
      issue_k(i + 1, i + 1);
      if (i < LV) issue_v(i, i);
    }
  };
  constexpr int kPrologueAfterK0 = 2;  // tiles issued after K0 before the first score tile

  // per-lane loop-invariant LDS offsets (row offsets of kb/cc blocks keep the swizzle)
#pragma unroll
  for (int ds = 0; ds < C::kDSteps; ++ds) k.koff[ds] = lds_off_bytes<C::kDP>(kpart * 32 + k.l32, ds * 2 + k.half);
  {
    const int g = lane >> 4, j16 = lane & 15;
#pragma unroll
    for (int db = 0; db < C::kDBlocks; ++db) {
      const int dcol = db * 32 + (g & 1) * 16 + (j16 & 3) * 4;
      const int r1 = kpart * 32 + k.half * 4 + (j16 >> 2);
#pragma unroll
      for (int t = 0; t < 2; ++t)
        k.voff[db][t] = NB * C::kTileBytes + lds_off_bytes<C::kDP>(r1 + 8 * t, dcol >> 3) + (dcol & 7) * 2;
    }
  }

  if constexpr (C::kQInLds) {
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) k.qoff[ds] = C::kRingBytes + lds_off_bytes<C::kDP>(qblk * 32 + k.l32, ds * 2 + k.half);
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
    k.m[qb] = -kMaxFloor;
    k.l[qb] = 0.f;
  }
  const float c = a.scale_log2;

  // S of position 0
  wait_vmcnt<kPrologueAfterK0 * C::kLoadsPerTile>();
  __syncthreads();
  k.scores(k.kbuf(0), k.s[0]);
  if (needs_mask(0)) mask_tile(k.s[0], 0);
  k.rowmax(k.s[0]);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) k.m[qb] = __builtin_fmaxf(k.m[qb], k.mx[qb]);  // O and l are still zero
  issue_rest_of_prologue();

  // Step p: exp and P V of position p, S of position p+1, as phase A
  // (score MFMAs + exponentials), the overflow check of the exponentials,
  // then phase B (P V MFMAs).  The step's barrier publishes K(p+1) and V(p)
  // and frees the slots of K(p) and V(p-1), which the step refills with
  // positions p+LK, p+LV (after the barrier or after phase A).
  // Ring slot and score set are compile-time: the loop is unrolled NB times.
  auto step = [&](int p, auto jconst) {
    constexpr int j = decltype(jconst)::value;  // p % kUnroll
    constexpr int b = j % NB;                   // p % NB
    constexpr int cur = j & 1;                  // p % 2
    // spread refills (whole tiles; SMALL copies clamp rows per lane and go
    // in one burst): load n of K(p + LK), V(p + LV), slots freed by the
    // barrier.  The V loads, issued last, may still be in flight here: the
    // step waits for them (and a second barrier publishes them) just before
    // phase B, the first reader of V(p).
    constexpr bool kSpread = C::kSpreadRefill && !SMALL;
    wait_vmcnt<kSpread ? C::kLoadsPerTile : C::kStepsInFlight * 2 * C::kLoadsPerTile>();
    __syncthreads();
    if constexpr (!C::kLateRefill && !kSpread) {
      issue_k(p + LK, (b + LK) % NB);
      issue_v(p + LV, (b + LV) % NB);
    }
    const uint32_t rk_off = kSpread ? tile_bytes(p + LK) : 0u;
    const uint32_t rv_off = kSpread ? tile_bytes(p + LV) : 0u;
    auto refill_k = [&](int n) {
      if constexpr (kSpread) cp.copy_one_at(K, rk_off, k.kbuf((b + LK) % NB), n);
    };
    auto refill_v = [&](int n) {
      if constexpr (kSpread) cp.copy_one_at(V, rv_off, k.vbuf((b + LV) % NB), n);
    };
    k.phase_a(k.kbuf((b + 1) % NB), k.s[cur], k.s[cur ^ 1], c, refill_k);
    if constexpr (C::kLateRefill) {
      issue_k(p + LK, (b + LK) % NB);
      issue_v(p + LV, (b + LV) % NB);
    }
    k.settle_tile(k.s[cur], c);
    if (needs_mask(p + 1)) mask_tile(k.s[cur ^ 1], p + 1);
    if constexpr (kSpread) {
      wait_vmcnt<C::kLoadsPerTile>();  // V(p), older than this step's K loads
      __syncthreads();
    }
    k.phase_b(k.vslot(b), refill_v);
  };
  for (int i = 0; i < nt; i += C::kUnroll)
    unrolled(i, nt, step, std::make_integer_sequence<int, C::kUnroll>());
  wait_vmcnt<0>();  // no direct-to-LDS copy may outlive the workgroup

  if constexpr (C::kSplit == 2) {
    // Merge the two key halves.  The second-half waves hand their running
    // max, row sums and O accumulators to the first-half wave of the same
    // query rows through LDS (lane-major, conflict-free); each pair of
    // partial results is rescaled to the larger max and added.
    constexpr int F = C::kMergeFloats;
    float __attribute__((address_space(3)))* xo =
        (float __attribute__((address_space(3)))*)k.smem + qblk * 64 * F + lane;
    __syncthreads();  // every wave is done with the ring
    if (kpart == 1) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) xo[((qb * C::kDBlocks + db) * 16 + r) * 64] = k.o[qb][db][r];
        xo[(QB * C::kDBlocks * 16 + qb) * 64] = k.m[qb];
        xo[(QB * C::kDBlocks * 16 + QB + qb) * 64] = k.l[qb];
      }
    }
    __syncthreads();
    if (kpart == 1) return;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float m2 = xo[(QB * C::kDBlocks * 16 + qb) * 64];
      const float l2 = xo[(QB * C::kDBlocks * 16 + QB + qb) * 64];
      const float mn = __builtin_fmaxf(k.m[qb], m2);
      const float a1 = fast_exp2((k.m[qb] - mn) * c), a2 = fast_exp2((m2 - mn) * c);
      k.l[qb] = k.l[qb] * a1 + l2 * a2;
      k.m[qb] = mn;
#pragma unroll
      for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          k.o[qb][db][r] = k.o[qb][db][r] * a1 + xo[((qb * C::kDBlocks + db) * 16 + r) * 64] * a2;
    }
  }

  // ---- epilogue: O = acc / l, L = m*scale + ln l
  if (!wave_active) return;
  if constexpr (KV) {
    if (a.n_split > 1) {
      // one key range of several: normalised O in float32 and L of the
      // range; a row that sees no key of the range gets O = 0 and L = -inf
      // (weight 0)
      float* __restrict__ Op = a.part_o + ((size_t)split * a.B * a.H + bh) * N * D;
      float* __restrict__ Lp = a.part_l + ((size_t)split * a.B * a.H + bh) * N;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float lt = sum_halves(k.l[qb]);
        const int row = wq0 + qb * 32 + k.l32;
        if (row < N) {
          if (lt > 0.f) {
            const float inv = 1.0f / lt;
#pragma unroll
            for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
              for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 w = {k.o[qb][db][g4 * 4 + 0] * inv, k.o[qb][db][g4 * 4 + 1] * inv,
                                 k.o[qb][db][g4 * 4 + 2] * inv, k.o[qb][db][g4 * 4 + 3] * inv};
                *(f32x4*)(Op + (size_t)row * D + db * 32 + g4 * 8 + k.half * 4) = w;
              }
            if (k.half == 0) Lp[row] = k.m[qb] * a.scale + fast_log2(lt) * kLn2;
          } else {
#pragma unroll
            for (int c = 0; c < D / 8; ++c)
              *(f32x4*)(Op + (size_t)row * D + c * 8 + k.half * 4) = f32x4{0.f, 0.f, 0.f, 0.f};
            if (k.half == 0) Lp[row] = -__builtin_inff();
          }
        }
      }
      return;
    }
  }
  __bf16* __restrict__ O = (__bf16*)a.o + head_off;
  float* __restrict__ Lse = a.lse + (size_t)bh * N;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = sum_halves(k.l[qb]);
    // block-sparse: a row that sees no key gets O = 0 and L = -inf
    const float inv = SPARSE ? (lt > 0.f ? 1.0f / lt : 0.f) : 1.0f / lt;
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
      if (k.half == 0) Lse[row] = (SPARSE && !(lt > 0.f)) ? -__builtin_inff() : k.m[qb] * a.scale + fast_log2(lt) * kLn2;
    }
  }
}

}  // namespace fwd
}  // namespace fa
