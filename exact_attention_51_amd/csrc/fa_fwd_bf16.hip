// fa_fwd_bf16.hip -- exact-attention forward, bf16 in/out, gfx950.
//
// One workgroup = 4 waves = 256 query rows of one (batch, head); each wave
// owns 64 query rows and the whole loop over keys for them.  The streaming
// structure is the one every page describes ("Learning Metal with
// FlashAttention", section FlashAttention; "Flash Attention" page, kernel
// anatomy; metal-flash-attention README, "Quantifying performance", forward
// pseudocode): the Q rows are loaded once and stay in registers, K and V
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
// * K/V tiles go global -> LDS with 16-byte direct loads (no VGPR staging)
//   into two buffers: the load of tile j+1 overlaps the math on tile j.
//   Rows are XOR-swizzled in 16-byte chunks (see swz) for conflict-free
//   ds_read_b128 and ds_read_b64_tr_b16.
// * exp is exp2 with scale*log2(e) folded into one FMA per score.  The
//   rescale of O is skipped while the running max has grown by less than
//   2^8 in the exp2 domain (the stale max is still an exact reference
//   point: P and l are just both scaled by the same bounded factor).
// * Causal masking skips every key tile above a wave's diagonal; only the
//   diagonal tile is masked element by element.
#include "fa_device.h"
#include "fa_kernels.h"
#include "fa_sched.h"

namespace fa {

namespace {

constexpr int kWaves = 4;
constexpr int kBlockN = 64;                // keys per K/V tile
constexpr float kRescaleThreshold = 8.0f;  // exp2-domain growth allowed before O is rescaled

template <int D>
struct FwdCfg {
  // Query blocks of 32 rows per wave: two for D <= 128 (64 rows, O in 2*D/32*16
  // registers), one for D = 256 so that O and Q^T still fit the register file.
  static constexpr int kQB = D <= 128 ? 2 : 1;
  static constexpr int kRowsPerWave = 32 * kQB;
  static constexpr int kBlockM = kWaves * kRowsPerWave;        // query rows per workgroup
  static constexpr int kDSteps = D / 16;                       // k-steps of the S product
  static constexpr int kDBlocks = D / 32;                      // 32-wide d blocks of O
  static constexpr int kTileBytes = kBlockN * D * 2;           // one K or V tile
  static constexpr int kLdsBytes = 4 * kTileBytes;             // K and V, two buffers each
};

template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1))) void fwd_bf16_kernel(
    FwdArgs a, TileSched sched) {
  using C = FwdCfg<D>;
  __shared__ __attribute__((aligned(1024))) char smem_raw[C::kLdsBytes];
  lds_char* smem = (lds_char*)smem_raw;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  int qtile, bh;
  sched_item(sched, blockIdx.x, qtile, bh);
  const int N = a.N;
  const size_t head_off = (size_t)bh * N * D;
  const __bf16* __restrict__ Q = (const __bf16*)a.q + head_off;
  const __bf16* __restrict__ K = (const __bf16*)a.k + head_off;
  const __bf16* __restrict__ V = (const __bf16*)a.v + head_off;

  constexpr int QB = C::kQB;
  const int q0 = qtile * C::kBlockM;
  const int wq0 = q0 + wave * C::kRowsPerWave;
  const bool wave_active = wq0 < N;
  const int n_ktiles_all = (N + kBlockN - 1) / kBlockN;
  int nt = n_ktiles_all;
  int wave_last = n_ktiles_all - 1;
  if constexpr (CAUSAL) {
    const int blk_last_row = min(q0 + C::kBlockM - 1, N - 1);
    nt = blk_last_row / kBlockN + 1;
    wave_last = min(wq0 + C::kRowsPerWave - 1, N - 1) / kBlockN;
  }

  lds_char* kbuf[2] = {smem, smem + C::kTileBytes};
  lds_char* vbuf[2] = {smem + 2 * C::kTileBytes, smem + 3 * C::kTileBytes};

  // Tile 0 in flight while Q is fetched.
  copy_rows_lds<D, kBlockN, kWaves>(K, N, 0, kbuf[0], wave, lane);
  copy_rows_lds<D, kBlockN, kWaves>(V, N, 0, vbuf[0], wave, lane);

  // Q^T as MFMA B operands: lane holds query column l32, d = ds*16 + half*8 + 0..7.
  bf16x8 qf[QB][C::kDSteps];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    int row = wq0 + qb * 32 + l32;
    row = row < N ? row : N - 1;
#pragma unroll
    for (int ds = 0; ds < C::kDSteps; ++ds)
      qf[qb][ds] = *(const bf16x8*)(Q + (size_t)row * D + ds * 16 + half * 8);
  }

  f32x16 o[QB][C::kDBlocks];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[qb][db][r] = 0.f;
  float m[QB], l[QB];  // running max (raw, unscaled score units); this lane's partial row sum
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -__builtin_inff();
    l[qb] = 0.f;
  }
  const float c = a.scale_log2;                           // scale * log2(e)
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  for (int j = 0; j < nt; ++j) {
    wait_vmcnt<0>();
    __syncthreads();
    if (j + 1 < nt) {
      copy_rows_lds<D, kBlockN, kWaves>(K, N, (j + 1) * kBlockN, kbuf[(j + 1) & 1], wave, lane);
      copy_rows_lds<D, kBlockN, kWaves>(V, N, (j + 1) * kBlockN, vbuf[(j + 1) & 1], wave, lane);
    }
    if (!wave_active || j > wave_last) continue;
    const lds_char* kb_ = kbuf[j & 1];
    const lds_char* vb_ = vbuf[j & 1];

    // ---- S^T = K_j Q^T : s[kb][qb], keys kb*32.., queries qb*32..
    f32x16 s[2][QB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][qb][r] = 0.f;
#pragma unroll
    for (int ds = 0; ds < C::kDSteps; ++ds) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf = read_row_operand<D>(kb_, kb * 32 + l32, ds, half);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = mfma32(kf, qf[qb][ds], s[kb][qb]);
      }
    }

    // ---- mask: causal diagonal tile, or keys past N in the last tile
    const bool diag = CAUSAL && j == wave_last;
    const bool tail = (j == n_ktiles_all - 1) && (N % kBlockN) != 0;
    if (diag || tail) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int query = wq0 + qb * 32 + l32;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = j * kBlockN + kb * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
            bool keep = key < N;
            if constexpr (CAUSAL) keep = keep && key <= query;
            s[kb][qb][r] = keep ? s[kb][qb][r] : -__builtin_inff();
          }
        }
    }

    // ---- online softmax per query block; P packed to bf16 B operands
    bf16x8 pk[QB][2][2];  // [qb][kb][16-key chunk]
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) mx = max3f(mx, s[kb][qb][r], s[kb][qb][r + 1]);
      mx = max_halves(mx);
      const float m_new = __builtin_fmaxf(m[qb], mx);
      const bool grow = (m_new - m[qb]) * c > kRescaleThreshold;
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        const float alpha = fast_exp2((m[qb] - m_new) * c);
#pragma unroll
        for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[qb][db][r] *= alpha;
        l[qb] *= alpha;
        m[qb] = m_new;
      }
      const float mc = m[qb] * c;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          bf16x2 pr[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float e0 = fast_exp2(__builtin_fmaf(s[kb][qb][cc * 8 + 2 * i], c, -mc));
            const float e1 = fast_exp2(__builtin_fmaf(s[kb][qb][cc * 8 + 2 * i + 1], c, -mc));
            pr[i] = pack_bf16(e0, e1);
            // the row sum is taken over the rounded P that enters the product
            l[qb] = __builtin_amdgcn_fdot2_f32_bf16(pr[i], ones, l[qb], false);
          }
          pk[qb][kb][cc] = join8(pr[0], pr[1], pr[2], pr[3]);
        }
      }
    }

    // ---- O^T += V_j^T P^T
#pragma unroll
    for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const bf16x8 vf = read_tr_operand<D>(vb_, kb * 32 + cc * 16, db * 32, lane);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) o[qb][db] = mfma32(vf, pk[qb][kb][cc], o[qb][db]);
        }
  }

  // ---- epilogue: O = acc / l, L = m*scale + ln l
  if (!wave_active) return;
  __bf16* __restrict__ O = (__bf16*)a.o + head_off;
  float* __restrict__ Lse = a.lse + (size_t)bh * N;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = sum_halves(l[qb]);
    const float inv = 1.0f / lt;
    const int row = wq0 + qb * 32 + l32;
    if (row < N) {
#pragma unroll
      for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          u32x2 w = {pack_bf16_u32(o[qb][db][g4 * 4 + 0] * inv, o[qb][db][g4 * 4 + 1] * inv),
                     pack_bf16_u32(o[qb][db][g4 * 4 + 2] * inv, o[qb][db][g4 * 4 + 3] * inv)};
          *(u32x2*)(O + (size_t)row * D + db * 32 + g4 * 8 + half * 4) = w;
        }
      if (half == 0) Lse[row] = m[qb] * a.scale + fast_log2(lt) * kLn2;
    }
  }
}

template <int D, bool CAUSAL>
int launch(const FwdArgs& a, hipStream_t stream) {
  const int n_qtiles = (a.N + FwdCfg<D>::kBlockM - 1) / FwdCfg<D>::kBlockM;
  const TileSched sched = make_sched(n_qtiles, a.B * a.H, CAUSAL);
  const long grid = (long)n_qtiles * a.B * a.H;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(256), 0, stream, a, sched);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  if (a.D == 64) return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
  if (a.D == 128) return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
  if (a.D == 256) return a.causal ? launch<256, true>(a, stream) : launch<256, false>(a, stream);
  return -2;
}

}  // namespace fa
