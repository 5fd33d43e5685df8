// fa_bwd.hip -- split attention backward (gfx950): a query-side kernel for
// dQ and a key/value-side kernel for dK and dV, with no floating-point
// atomics and no workspace.
//
// The split is the one the metal-flash-attention README describes
// ("Quantifying performance", backward-query and backward-key-value
// pseudocode): the dQ kernel owns a block of query rows and loops over key
// blocks; the dK/dV kernel owns a block of key rows and loops over query
// blocks.  Each rebuilds P = exp(S - L) from the forward's saved L, so the
// scores are computed twice in total (seven products instead of five), and
// every output element has exactly one writer.
//
// Per (query i, key j), with S the scaled scores:
//   delta_i = sum_d dO_id O_id          (dQ kernel, written for dK/dV)
//   P_ij    = exp(S_ij - L_i)
//   dP_ij   = sum_d dO_id V_jd
//   dS_ij   = P_ij (dP_ij - delta_i)
//   dQ_i   += scale sum_j dS_ij K_j,  dK_j += scale sum_i dS_ij Q_i,  dV_j += sum_i P_ij dO_i
//
// Layout tricks are those of the forward kernel: a 32x32 MFMA accumulator
// holds one column per lane, an accumulator packed to bf16 is directly the
// k-operand of the next product, and the matching transposed operand is
// read from LDS with ds_read_b64_tr_b16.
#include "fa_device.h"
#include "fa_kernels.h"
#include "fa_sched.h"

namespace fa {

namespace {

constexpr int kWavesQ = 4;    // dQ kernel: 4 waves per workgroup
constexpr int kKeyTile = 64;  // dQ kernel: keys per streamed K/V tile

// dQ kernel key split: at D = 256 the two 32-key halves of every K/V tile
// go to two waves that own the same 32 query rows (their dQ partial sums
// are added at the end), so a workgroup covers 64 rows and the B*H*N/32
// query blocks of a workload fill twice as many SIMDs.
// LDS rows are DP wide: D = 32, 96 and 160 use the layout of 64, 128 and 256 with the
// chunks past D unused (global rows stay D wide).
template <int D>
constexpr int lds_width() {
  return D <= 64 ? 64 : D <= 128 ? 128 : 256;
}

template <int D>
struct DqCfg {
  static constexpr int kDP = lds_width<D>();
  static constexpr int kSplit = kDP == 256 ? 2 : 1;
  static constexpr int kKB = 2 / kSplit;               // 32-key blocks a wave takes per tile
  static constexpr int kRows = 32 * kWavesQ / kSplit;  // query rows per workgroup
};

// ============================================================== dQ kernel
//
// Each wave owns 32 query rows (one lane column each).  Scores and dP are
// formed transposed (S^T = K Q^T, dP^T = V dO^T) so that L_i and delta_i
// are per-lane scalars; dQ^T += K^T dS^T takes dS^T straight from the
// accumulators and K^T through the transpose read of the K tile.
template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1))) void bwd_dq_kernel(
    BwdArgs a, TileSched sched) {
  constexpr int kDSteps = D / 16, kDBlocks = D / 32;
  constexpr int KB = DqCfg<D>::kKB, kRowsQ = DqCfg<D>::kRows, kQBlocks = kWavesQ / DqCfg<D>::kSplit;
  constexpr int DP = DqCfg<D>::kDP;
  constexpr int kTileBytes = kKeyTile * DP * 2;
  __shared__ __attribute__((aligned(1024))) char smem_raw[4 * kTileBytes];
  lds_char* smem = (lds_char*)smem_raw;
  lds_char* kbuf[2] = {smem, smem + kTileBytes};
  lds_char* vbuf[2] = {smem + 2 * kTileBytes, smem + 3 * kTileBytes};

  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, l32 = lane & 31,
            half = lane >> 5;
  int qtile, bh;
  sched_item(sched, blockIdx.x, qtile, bh);
  const int N = a.N;
  const size_t head_off = (size_t)bh * N * D;
  const __bf16* __restrict__ Q = (const __bf16*)a.q + head_off;
  const __bf16* __restrict__ K = (const __bf16*)a.k + head_off;
  const __bf16* __restrict__ V = (const __bf16*)a.v + head_off;
  const __bf16* __restrict__ O = (const __bf16*)a.o + head_off;
  const __bf16* __restrict__ dO = (const __bf16*)a.dO + head_off;

  // query block and key half of this wave (kpart = 0 without a key split)
  const int qblk = wave % kQBlocks, kpart = wave / kQBlocks;
  const int q0 = qtile * kRowsQ;
  const int wq0 = q0 + qblk * 32;
  const bool wave_active = wq0 < N;
  const int n_ktiles_all = (N + kKeyTile - 1) / kKeyTile;
  int nt = n_ktiles_all, wave_last = n_ktiles_all - 1;
  if constexpr (CAUSAL) {
    nt = min(q0 + kRowsQ - 1, N - 1) / kKeyTile + 1;
    wave_last = min(wq0 + 31, N - 1) / kKeyTile;
  }

  // K/V tile t into ring slot b: scalar-base copies with loop-invariant
  // per-lane offsets, rows clamped onto N-1 only for a ragged last tile
  RowTileCopier<D, DP, kKeyTile, kWavesQ> cp;
  cp.init(wave, lane);
  auto copy_tile = [&](int t, int b) {
    const int row0 = t * kKeyTile;
    if (row0 + kKeyTile <= N) {
      cp.copy_at(K, (uint32_t)row0 * (D * 2), kbuf[b]);
      cp.copy_at(V, (uint32_t)row0 * (D * 2), vbuf[b]);
    } else {
      cp.copy_clamped(K, N, row0, kbuf[b]);
      cp.copy_clamped(V, N, row0, vbuf[b]);
    }
  };
  copy_tile(0, 0);

  // Q^T and dO^T as B operands (lane = query column), delta and L per lane.
  const int row = wq0 + l32;
  const int crow = row < N ? row : N - 1;
  bf16x8 qf[kDSteps], dof[kDSteps];
  float dpart = 0.f;
#pragma unroll
  for (int ds = 0; ds < kDSteps; ++ds) {
    const size_t off = (size_t)crow * D + ds * 16 + half * 8;
    qf[ds] = *(const bf16x8*)(Q + off);
    dof[ds] = *(const bf16x8*)(dO + off);
    const bf16x8 of = *(const bf16x8*)(O + off);
#pragma unroll
    for (int i = 0; i < 8; ++i) dpart = __builtin_fmaf((float)dof[ds][i], (float)of[i], dpart);
  }
  const float delta = sum_halves(dpart);
  const float lse2 = a.lse[(size_t)bh * N + crow] * kLog2e;  // L in the exp2 domain
  if (wave_active && kpart == 0 && half == 0 && row < N) a.delta[(size_t)bh * N + row] = delta;
  const float c = a.scale_log2;

  f32x16 dq[kDBlocks];
#pragma unroll
  for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[db][r] = 0.f;

  for (int j = 0; j < nt; ++j) {
    wait_vmcnt<0>();
    __syncthreads();
    if (j + 1 < nt) copy_tile(j + 1, (j + 1) & 1);
    if (!wave_active || j > wave_last) continue;
    const lds_char* kt = kbuf[j & 1];
    const lds_char* vt = vbuf[j & 1];

    // S^T = K_j Q^T and dP^T = V_j dO^T, keys kr0 + kb*32.. (rows), this wave's queries (columns)
    const int kr0 = kpart * 32;
    f32x16 s[KB], dp[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = dp[kb][r] = 0.f;
#pragma unroll
    for (int ds = 0; ds < kDSteps; ++ds)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        s[kb] = mfma32(read_row_operand<DP>(kt, kr0 + kb * 32 + l32, ds, half), qf[ds], s[kb]);
        dp[kb] = mfma32(read_row_operand<DP>(vt, kr0 + kb * 32 + l32, ds, half), dof[ds], dp[kb]);
      }

    const bool masked = (CAUSAL && j == wave_last) || (j == n_ktiles_all - 1 && (N % kKeyTile) != 0);
    bf16x8 dsk[KB][2];  // dS^T packed: [key block][16-key chunk]
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        bf16x2 pr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float e[2];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int r = cc * 8 + 2 * i + t;
            float x = __builtin_fmaf(s[kb][r], c, -lse2);
            if (masked) {
              const int key = j * kKeyTile + kr0 + kb * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
              bool keep = key < N;
              if constexpr (CAUSAL) keep = keep && key <= row;
              x = keep ? x : -__builtin_inff();
            }
            const float p = fast_exp2(x);
            e[t] = p * (dp[kb][r] - delta);
          }
          pr[i] = pack_bf16(e[0], e[1]);
        }
        dsk[kb][cc] = join8(pr[0], pr[1], pr[2], pr[3]);
      }

    // dQ^T += K_j^T dS^T
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
          dq[db] = mfma32(read_tr_operand<DP>(kt, kr0 + kb * 32 + cc * 16, db * 32, lane), dsk[kb][cc], dq[db]);
  }

  if constexpr (DqCfg<D>::kSplit == 2) {
    // add the second key half's dQ partial sums (lane-major through LDS)
    float __attribute__((address_space(3)))* x =
        (float __attribute__((address_space(3)))*)smem + qblk * 64 * kDBlocks * 16 + lane;
    static_assert(kQBlocks * 64 * kDBlocks * 16 * 4 <= 4 * kTileBytes, "merge buffer exceeds the ring");
    wait_vmcnt<0>();
    __syncthreads();  // every wave is done with the K/V tiles
    if (kpart == 1) {
#pragma unroll
      for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) x[(db * 16 + r) * 64] = dq[db][r];
    }
    __syncthreads();
    if (kpart == 1) return;
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) dq[db][r] += x[(db * 16 + r) * 64];
  }

  if (!wave_active || row >= N) return;
  __bf16* __restrict__ dQ = (__bf16*)a.dq + head_off;
#pragma unroll
  for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      u32x2 w = {pack_bf16_u32(dq[db][g4 * 4 + 0] * a.scale, dq[db][g4 * 4 + 1] * a.scale),
                 pack_bf16_u32(dq[db][g4 * 4 + 2] * a.scale, dq[db][g4 * 4 + 3] * a.scale)};
      *(u32x2*)(dQ + (size_t)row * D + db * 32 + g4 * 8 + half * 4) = w;
    }
}

// ========================================================== dK/dV kernel
//
// Each wave owns 32 key rows (one lane column each); the workgroup's key
// block stays in LDS while query tiles (Q, dO, L, delta) stream through a
// double buffer.  S = Q K^T and dP = dO V^T put a key in every lane column
// and 16 queries in its registers; P and dS packed to bf16 are then the
// k-operands of dV^T += dO^T P and dK^T += Q^T dS, with dO^T and Q^T read
// transposed from the query tile.
// (D = 160 and 256 have their own kernel, fa_bwd_dkdv_d256.hip.)
template <int D>
struct KvCfg {
  static_assert(D <= 128, "");
  static constexpr int kDP = lds_width<D>();
  static constexpr int kWaves = 4;
  static constexpr int kKeys = 32 * kWaves;  // key rows per workgroup
  static constexpr int kQTile = 64;
  static constexpr int kQB = kQTile / 32;
  static constexpr int kKvBytes = kKeys * kDP * 2;
  static constexpr int kTileBytes = kQTile * kDP * 2;
  static constexpr int kStatBytes = 256;  // 64 floats of L or delta
  static constexpr int kLdsBytes = 2 * kKvBytes + 4 * kTileBytes + 4 * kStatBytes;
};

template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * KvCfg<D>::kWaves, 64 * KvCfg<D>::kWaves),
                          amdgpu_waves_per_eu(1, 1))) void bwd_dkdv_kernel(BwdArgs a, TileSched sched) {
  using C = KvCfg<D>;
  constexpr int kDSteps = D / 16, kDBlocks = D / 32, QB = C::kQB, W = C::kWaves, DP = C::kDP;
  __shared__ __attribute__((aligned(1024))) char smem_raw[C::kLdsBytes];
  lds_char* smem = (lds_char*)smem_raw;
  lds_char* kres = smem;
  lds_char* vres = smem + C::kKvBytes;
  lds_char* qbuf[2] = {smem + 2 * C::kKvBytes, smem + 2 * C::kKvBytes + C::kTileBytes};
  lds_char* obuf[2] = {smem + 2 * C::kKvBytes + 2 * C::kTileBytes, smem + 2 * C::kKvBytes + 3 * C::kTileBytes};
  lds_char* stat0 = smem + 2 * C::kKvBytes + 4 * C::kTileBytes;
  lds_char* lbuf[2] = {stat0, stat0 + C::kStatBytes};
  lds_char* dbuf[2] = {stat0 + 2 * C::kStatBytes, stat0 + 3 * C::kStatBytes};

  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, l32 = lane & 31,
            half = lane >> 5;
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
  const int wk0 = k0 + wave * 32;
  const int key = wk0 + l32;
  const bool wave_active = wk0 < N;
  const int n_qtiles = (N + C::kQTile - 1) / C::kQTile;
  const int t_begin = CAUSAL ? k0 / C::kQTile : 0;

  auto load_qtile = [&](int t, int b) {
    copy_rows_lds<D, DP, C::kQTile, W>(Q, N, t * C::kQTile, qbuf[b], wave, lane);
    copy_rows_lds<D, DP, C::kQTile, W>(dO, N, t * C::kQTile, obuf[b], wave, lane);
    if (wave == 0) {
      int r = t * C::kQTile + lane;
      r = r < N ? r : N - 1;
      load_lds4(Lg + r, lbuf[b]);
      load_lds4(Dg + r, dbuf[b]);
    }
  };
  copy_rows_lds<D, DP, C::kKeys, W>(K, N, k0, kres, wave, lane);
  copy_rows_lds<D, DP, C::kKeys, W>(V, N, k0, vres, wave, lane);
  load_qtile(t_begin, 0);

  f32x16 dk[kDBlocks], dv[kDBlocks];
#pragma unroll
  for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[db][r] = dv[db][r] = 0.f;
  const float c = a.scale_log2;

  for (int t = t_begin; t < n_qtiles; ++t) {
    const int b = (t - t_begin) & 1;
    wait_vmcnt<0>();
    __syncthreads();
    if (t + 1 < n_qtiles) load_qtile(t + 1, b ^ 1);
    const int tq0 = t * C::kQTile;
    if (!wave_active) continue;
    if (CAUSAL && tq0 + C::kQTile - 1 < wk0) continue;  // every query of the tile precedes every key of the wave
    const lds_char* qt = qbuf[b];
    const lds_char* ot = obuf[b];

    // S = Q_t K^T, dP = dO_t V^T : query rows qb*32.., this wave's keys as columns
    f32x16 s[QB], dp[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[qb][r] = dp[qb][r] = 0.f;
#pragma unroll
    for (int ds = 0; ds < kDSteps; ++ds) {
      const bf16x8 kf = read_row_operand<DP>(kres, wave * 32 + l32, ds, half);
      const bf16x8 vf = read_row_operand<DP>(vres, wave * 32 + l32, ds, half);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        s[qb] = mfma32(read_row_operand<DP>(qt, qb * 32 + l32, ds, half), kf, s[qb]);
        dp[qb] = mfma32(read_row_operand<DP>(ot, qb * 32 + l32, ds, half), vf, dp[qb]);
      }
    }

    // a mask is needed when some query of the tile precedes some key of the wave, or past N
    __builtin_amdgcn_sched_barrier(0);
    const bool masked = (CAUSAL && tq0 < wk0 + 31) || (tq0 + C::kQTile > N);
    bf16x8 ppk[QB][2], dspk[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        // queries of register r: qb*32 + (r/4)*8 + half*4 + r%4; registers 8cc..8cc+7 cover two runs of 4
        const f32x4 la = *(const f32x4 __attribute__((address_space(3)))*)(lbuf[b] + 4 * (qb * 32 + cc * 16 + half * 4));
        const f32x4 lb = *(const f32x4 __attribute__((address_space(3)))*)(lbuf[b] + 4 * (qb * 32 + cc * 16 + 8 + half * 4));
        const f32x4 da = *(const f32x4 __attribute__((address_space(3)))*)(dbuf[b] + 4 * (qb * 32 + cc * 16 + half * 4));
        const f32x4 dbv = *(const f32x4 __attribute__((address_space(3)))*)(dbuf[b] + 4 * (qb * 32 + cc * 16 + 8 + half * 4));
        bf16x2 pp[4], dd[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float pv[2], dsv[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int ii = 2 * i + u;  // 0..7 within the 16-query chunk
            const int r = cc * 8 + ii;
            const float lq = ii < 4 ? la[ii] : lb[ii - 4];
            const float dq = ii < 4 ? da[ii] : dbv[ii - 4];
            float x = __builtin_fmaf(s[qb][r], c, -lq * kLog2e);
            if (masked) {
              const int query = tq0 + qb * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
              bool keep = query < N;
              if constexpr (CAUSAL) keep = keep && key <= query;
              x = keep ? x : -__builtin_inff();
            }
            const float p = fast_exp2(x);
            pv[u] = p;
            dsv[u] = p * (dp[qb][r] - dq);
          }
          pp[i] = pack_bf16(pv[0], pv[1]);
          dd[i] = pack_bf16(dsv[0], dsv[1]);
        }
        ppk[qb][cc] = join8(pp[0], pp[1], pp[2], pp[3]);
        dspk[qb][cc] = join8(dd[0], dd[1], dd[2], dd[3]);
      }
    }

    __builtin_amdgcn_sched_barrier(0);
    // dV^T += dO_t^T P,  dK^T += Q_t^T dS
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          dv[db] = mfma32(read_tr_operand<DP>(ot, qb * 32 + cc * 16, db * 32, lane), ppk[qb][cc], dv[db]);
          dk[db] = mfma32(read_tr_operand<DP>(qt, qb * 32 + cc * 16, db * 32, lane), dspk[qb][cc], dk[db]);
        }
  }

  if (!wave_active || key >= N) return;
  __bf16* __restrict__ dK = (__bf16*)a.dk + head_off;
  __bf16* __restrict__ dV = (__bf16*)a.dv + head_off;
#pragma unroll
  for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const size_t off = (size_t)key * D + db * 32 + g4 * 8 + half * 4;
      u32x2 wk = {pack_bf16_u32(dk[db][g4 * 4 + 0] * a.scale, dk[db][g4 * 4 + 1] * a.scale),
                  pack_bf16_u32(dk[db][g4 * 4 + 2] * a.scale, dk[db][g4 * 4 + 3] * a.scale)};
      u32x2 wv = {pack_bf16_u32(dv[db][g4 * 4 + 0], dv[db][g4 * 4 + 1]),
                  pack_bf16_u32(dv[db][g4 * 4 + 2], dv[db][g4 * 4 + 3])};
      *(u32x2*)(dK + off) = wk;
      *(u32x2*)(dV + off) = wv;
    }
}

template <int D, bool CAUSAL>
int launch_dq(const BwdArgs& a, hipStream_t stream) {
  constexpr int kRowsQ = DqCfg<D>::kRows;
  const int n_tiles = (a.N + kRowsQ - 1) / kRowsQ;
  const TileSched sched = make_sched(n_tiles, a.B * a.H, CAUSAL);
  const long grid = (long)n_tiles * a.B * a.H;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(256), 0, stream, a, sched);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int D, bool CAUSAL>
int launch_dkdv(const BwdArgs& a, hipStream_t stream) {
  using C = KvCfg<D>;
  const int n_tiles = (a.N + C::kKeys - 1) / C::kKeys;
  // causal: the first key blocks see the most query tiles, so ascending order is heaviest first
  TileSched sched = make_sched(n_tiles, a.B * a.H, false);
  const long grid = (long)n_tiles * a.B * a.H;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(64 * C::kWaves), 0, stream, a, sched);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int launch_bwd_dq(const BwdArgs& a, hipStream_t stream) {
  switch (a.D) {
    case 32:
      return a.causal ? launch_dq<32, true>(a, stream) : launch_dq<32, false>(a, stream);
    case 64:
      return a.causal ? launch_dq<64, true>(a, stream) : launch_dq<64, false>(a, stream);
    case 96:
      return a.causal ? launch_dq<96, true>(a, stream) : launch_dq<96, false>(a, stream);
    case 128:
      return a.causal ? launch_dq<128, true>(a, stream) : launch_dq<128, false>(a, stream);
    case 160:  // the D = 256 layout and key split, 96 columns unused
      return a.causal ? launch_dq<160, true>(a, stream) : launch_dq<160, false>(a, stream);
    case 256:
      return a.causal ? launch_dq<256, true>(a, stream) : launch_dq<256, false>(a, stream);
  }
  return -2;
}

int launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream) {
  switch (a.D) {
    case 32:
      return a.causal ? launch_dkdv<32, true>(a, stream) : launch_dkdv<32, false>(a, stream);
    case 64:
      return a.causal ? launch_dkdv<64, true>(a, stream) : launch_dkdv<64, false>(a, stream);
    case 96:
      return a.causal ? launch_dkdv<96, true>(a, stream) : launch_dkdv<96, false>(a, stream);
    case 128:
      return a.causal ? launch_dkdv<128, true>(a, stream) : launch_dkdv<128, false>(a, stream);
    case 160:
    case 256:
      return launch_bwd_dkdv_d256(a, stream);
  }
  return -2;
}

}  // namespace fa
