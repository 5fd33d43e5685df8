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

// ------------------------------------------- dQ chains for 256-wide LDS rows
//
// At D = 160 and 256 a wave's step is 2 NS + 2 NB MFMAs whose A operands
// all come from LDS.  Compiled from C++ the reads were issued one MFMA
// ahead of their use, so every MFMA waited out an LDS round trip; these
// two chains keep six fragments in flight instead.  Fixed registers: the
// Q^T fragment of k-step ds in a[4 ds : 4 ds + 3] and the dO^T fragment in
// a[64 + 4 ds : ...] (bound by the callers' operand constraints), six
// fragment buffers in v[232:255], read addresses formed in v230 and v231.
//
// Read addresses: a tile row is 512 bytes and 512-aligned in LDS, and the
// swizzle only permutes 16-byte chunks inside each 256-byte half, so the
// lane's address of chunk c ^ swz equals its address of chunk swz with
// the chunk bits flipped by c: one XOR with a constant per read.

// DQ_WAIT n: s_waitcnt lgkmcnt(n) for an assemble-time n in 0..11
#define DQ_WAIT_MACRO                                \
  ".macro DQ_WAIT n\n"                               \
  "  .if (\\n) <= 0\n    s_waitcnt lgkmcnt(0)\n"     \
  "  .elseif (\\n) == 1\n    s_waitcnt lgkmcnt(1)\n" \
  "  .elseif (\\n) == 2\n    s_waitcnt lgkmcnt(2)\n" \
  "  .elseif (\\n) == 3\n    s_waitcnt lgkmcnt(3)\n" \
  "  .elseif (\\n) == 4\n    s_waitcnt lgkmcnt(4)\n" \
  "  .elseif (\\n) == 5\n    s_waitcnt lgkmcnt(5)\n" \
  "  .elseif (\\n) == 6\n    s_waitcnt lgkmcnt(6)\n" \
  "  .elseif (\\n) == 7\n    s_waitcnt lgkmcnt(7)\n" \
  "  .elseif (\\n) == 8\n    s_waitcnt lgkmcnt(8)\n" \
  "  .elseif (\\n) == 9\n    s_waitcnt lgkmcnt(9)\n" \
  "  .elseif (\\n) == 10\n    s_waitcnt lgkmcnt(10)\n" \
  "  .else\n    s_waitcnt lgkmcnt(11)\n"             \
  "  .endif\n"                                       \
  ".endm\n"

#define DQ_CHAIN_CLOBBERS                                                                                      \
  "memory", "v230", "v231", "v232", "v233", "v234", "v235", "v236", "v237", "v238", "v239", "v240", "v241", \
      "v242", "v243", "v244", "v245", "v246", "v247", "v248", "v249", "v250", "v251", "v252", "v253", "v254", "v255"

// S^T = K_j Q^T and dP^T = V_j dO^T over NS k-steps of 16 columns,
// interleaved: MFMA i takes k-step i/2, S for even i and dP for odd i.  rb
// is the lane's address of chunk 0 of its K row in the ring slot; k-step ds
// is chunk 2 ds + half: rb ^ 32 (ds mod 8), 256 bytes further for ds >= 8,
// and the V slot lies 32768 bytes after the K slot.  Each accumulator runs
// its k-steps in order, as the plain loop does.
template <int NS>
__device__ __forceinline__ void dq_sdp_chain(int rb, const f32x16 (&qo)[8], f32x16& s, f32x16& dp) {
  static_assert(NS >= 4 && NS <= 16, "chain length");
  asm volatile(
      DQ_WAIT_MACRO
      // read fragment i into buffer i mod 6
      ".macro DQ_RD i\n"
      "  .if (\\i) < 2 * %[ns]\n"
      "    .if (((\\i) >> 1) & 7) == 0\n"
      "      ds_read_b128 v[232 + ((\\i) %% 6) * 4 : 235 + ((\\i) %% 6) * 4], %[rb] "
      "offset:(((\\i) & 1) * 32768 + (((\\i) >> 4) & 1) * 256)\n"
      "    .else\n"
      "      v_xor_b32 v[230 + ((\\i) & 1)], 32 * (((\\i) >> 1) & 7), %[rb]\n"
      "      ds_read_b128 v[232 + ((\\i) %% 6) * 4 : 235 + ((\\i) %% 6) * 4], v[230 + ((\\i) & 1)] "
      "offset:(((\\i) & 1) * 32768 + (((\\i) >> 4) & 1) * 256)\n"
      "    .endif\n"
      "  .endif\n"
      ".endm\n"
      ".macro DQ_MM i, acc\n"
      "  .if (\\i) < 2 * %[ns]\n"
      "    .if (\\i) + 6 < 2 * %[ns]\n"
      "      DQ_WAIT 5\n"
      "    .else\n"
      "      DQ_WAIT (2 * %[ns] - (\\i) - 1)\n"
      "    .endif\n"
      "    .if ((\\i) >> 1) == 0\n"
      "      v_mfma_f32_32x32x16_bf16 \\acc, v[232 + ((\\i) %% 6) * 4 : 235 + ((\\i) %% 6) * 4], "
      "a[((\\i) & 1) * 64 + ((\\i) >> 1) * 4 : ((\\i) & 1) * 64 + ((\\i) >> 1) * 4 + 3], 0\n"
      "    .else\n"
      "      v_mfma_f32_32x32x16_bf16 \\acc, v[232 + ((\\i) %% 6) * 4 : 235 + ((\\i) %% 6) * 4], "
      "a[((\\i) & 1) * 64 + ((\\i) >> 1) * 4 : ((\\i) & 1) * 64 + ((\\i) >> 1) * 4 + 3], \\acc\n"
      "    .endif\n"
      "    DQ_RD (\\i) + 6\n"
      "  .endif\n"
      ".endm\n"
      "DQ_RD 0\nDQ_RD 1\nDQ_RD 2\nDQ_RD 3\nDQ_RD 4\nDQ_RD 5\n"
      "DQ_MM 0, %[s]\nDQ_MM 1, %[dp]\nDQ_MM 2, %[s]\nDQ_MM 3, %[dp]\n"
      "DQ_MM 4, %[s]\nDQ_MM 5, %[dp]\nDQ_MM 6, %[s]\nDQ_MM 7, %[dp]\n"
      "DQ_MM 8, %[s]\nDQ_MM 9, %[dp]\nDQ_MM 10, %[s]\nDQ_MM 11, %[dp]\n"
      "DQ_MM 12, %[s]\nDQ_MM 13, %[dp]\nDQ_MM 14, %[s]\nDQ_MM 15, %[dp]\n"
      "DQ_MM 16, %[s]\nDQ_MM 17, %[dp]\nDQ_MM 18, %[s]\nDQ_MM 19, %[dp]\n"
      "DQ_MM 20, %[s]\nDQ_MM 21, %[dp]\nDQ_MM 22, %[s]\nDQ_MM 23, %[dp]\n"
      "DQ_MM 24, %[s]\nDQ_MM 25, %[dp]\nDQ_MM 26, %[s]\nDQ_MM 27, %[dp]\n"
      "DQ_MM 28, %[s]\nDQ_MM 29, %[dp]\nDQ_MM 30, %[s]\nDQ_MM 31, %[dp]\n"
      "s_nop 7\ns_nop 7\ns_nop 7\n"  // S and dP are read by vector instructions next
      ".purgem DQ_WAIT\n.purgem DQ_RD\n.purgem DQ_MM\n"
      : [s] "=&v"(s), [dp] "=&v"(dp)
      : [ns] "i"(NS), [rb] "v"(rb), "{a[0:15]}"(qo[0]), "{a[16:31]}"(qo[1]), "{a[32:47]}"(qo[2]),
        "{a[48:63]}"(qo[3]), "{a[64:79]}"(qo[4]), "{a[80:95]}"(qo[5]), "{a[96:111]}"(qo[6]), "{a[112:127]}"(qo[7])
      : DQ_CHAIN_CLOBBERS);
}

// dQ^T += K_j^T dS^T over NB 32-column blocks, K_j^T read transposed
// (two ds_read_b64_tr_b16 per fragment, 8 rows apart).  Fragment order:
// the first 16 keys (dS^T chunk d0) for blocks 0..NB-1, then the second 16
// (d1), so each accumulator takes its two chunks in order.  t1 and t2 are
// the lane's addresses of the two reads of block 0's first chunk; block db
// is t ^ 64 (db mod 4), 256 bytes further for db >= 4, and the second chunk
// 8192.  Accumulators past NB are not touched.
template <int NB>
__device__ __forceinline__ void dq_tr_chain(int t1, int t2, const bf16x8& d0, const bf16x8& d1, f32x16& q0,
                                            f32x16& q1, f32x16& q2, f32x16& q3, f32x16& q4, f32x16& q5,
                                            f32x16& q6, f32x16& q7) {
  static_assert(NB >= 4 && NB <= 8, "blocks");
  asm volatile(
      DQ_WAIT_MACRO
      // the two reads of block db, chunk offset co, into buffer f mod 6
      ".macro DT_RDX db, co, f\n"
      "  .if ((\\db) & 3) == 0\n"
      "    ds_read_b64_tr_b16 v[232 + ((\\f) %% 6) * 4 : 233 + ((\\f) %% 6) * 4], %[t1] "
      "offset:((\\co) + ((\\db) >> 2) * 256)\n"
      "    ds_read_b64_tr_b16 v[234 + ((\\f) %% 6) * 4 : 235 + ((\\f) %% 6) * 4], %[t2] "
      "offset:((\\co) + ((\\db) >> 2) * 256)\n"
      "  .else\n"
      "    v_xor_b32 v230, 64 * ((\\db) & 3), %[t1]\n"
      "    v_xor_b32 v231, 64 * ((\\db) & 3), %[t2]\n"
      "    ds_read_b64_tr_b16 v[232 + ((\\f) %% 6) * 4 : 233 + ((\\f) %% 6) * 4], v230 "
      "offset:((\\co) + ((\\db) >> 2) * 256)\n"
      "    ds_read_b64_tr_b16 v[234 + ((\\f) %% 6) * 4 : 235 + ((\\f) %% 6) * 4], v231 "
      "offset:((\\co) + ((\\db) >> 2) * 256)\n"
      "  .endif\n"
      ".endm\n"
      // fragment f: block f of the first chunk (f < NB) or f - NB of the second
      ".macro DT_RD f\n"
      "  .if (\\f) < %[nb]\n"
      "    DT_RDX (\\f), 0, (\\f)\n"
      "  .elseif (\\f) < 2 * %[nb]\n"
      "    DT_RDX ((\\f) - %[nb]), 8192, (\\f)\n"
      "  .endif\n"
      ".endm\n"
      ".macro DT_MM f, lim, acc, b\n"
      "  .if (\\f) < (\\lim)\n"
      "    .if (\\f) + 6 < 2 * %[nb]\n"
      "      DQ_WAIT 10\n"
      "    .else\n"
      "      DQ_WAIT (2 * (2 * %[nb] - (\\f) - 1))\n"
      "    .endif\n"
      "    v_mfma_f32_32x32x16_bf16 \\acc, v[232 + ((\\f) %% 6) * 4 : 235 + ((\\f) %% 6) * 4], \\b, \\acc\n"
      "    DT_RD (\\f) + 6\n"
      "  .endif\n"
      ".endm\n"
      "DT_RD 0\nDT_RD 1\nDT_RD 2\nDT_RD 3\nDT_RD 4\nDT_RD 5\n"
      "DT_MM 0, %[nb], %[q0], %[d0]\nDT_MM 1, %[nb], %[q1], %[d0]\n"
      "DT_MM 2, %[nb], %[q2], %[d0]\nDT_MM 3, %[nb], %[q3], %[d0]\n"
      "DT_MM 4, %[nb], %[q4], %[d0]\nDT_MM 5, %[nb], %[q5], %[d0]\n"
      "DT_MM 6, %[nb], %[q6], %[d0]\nDT_MM 7, %[nb], %[q7], %[d0]\n"
      "DT_MM %[nb]+0, 2*%[nb], %[q0], %[d1]\nDT_MM %[nb]+1, 2*%[nb], %[q1], %[d1]\n"
      "DT_MM %[nb]+2, 2*%[nb], %[q2], %[d1]\nDT_MM %[nb]+3, 2*%[nb], %[q3], %[d1]\n"
      "DT_MM %[nb]+4, 2*%[nb], %[q4], %[d1]\nDT_MM %[nb]+5, 2*%[nb], %[q5], %[d1]\n"
      "DT_MM %[nb]+6, 2*%[nb], %[q6], %[d1]\nDT_MM %[nb]+7, 2*%[nb], %[q7], %[d1]\n"
      "s_nop 7\ns_nop 7\ns_nop 7\n"  // the accumulators may be read by vector instructions next
      ".purgem DQ_WAIT\n.purgem DT_RDX\n.purgem DT_RD\n.purgem DT_MM\n"
      : [q0] "+v"(q0), [q1] "+v"(q1), [q2] "+v"(q2), [q3] "+v"(q3), [q4] "+v"(q4), [q5] "+v"(q5), [q6] "+v"(q6),
        [q7] "+v"(q7)
      : [nb] "i"(NB), [d0] "v"(d0), [d1] "v"(d1), [t1] "v"(t1), [t2] "v"(t2)
      : DQ_CHAIN_CLOBBERS);
}

#undef DQ_WAIT_MACRO
#undef DQ_CHAIN_CLOBBERS

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
  // 256-wide rows run the step as the two asm chains (one 32-key block per wave)
  constexpr bool kChains = DP == 256;
  static_assert(!kChains || (KB == 1 && kTileBytes == 32768), "chain layout");
  constexpr bool kSplitMask = kChains;
  // ring slots K0 V0 K1 V1: a slot's V tile lies kTileBytes after its K tile
  __shared__ __attribute__((aligned(1024))) char smem_raw[4 * kTileBytes];
  lds_char* smem = (lds_char*)smem_raw;
  lds_char* kbuf[2] = {smem, smem + 2 * kTileBytes};
  lds_char* vbuf[2] = {smem + kTileBytes, smem + 3 * kTileBytes};

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

  // the chains take 8 accumulators; at D = 160 the last three stay unused
  constexpr int kAcc = kChains ? 8 : kDBlocks;
  f32x16 dq[kAcc];
#pragma unroll
  for (int db = 0; db < kAcc; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[db][r] = 0.f;

  // chain operands: Q^T and dO^T fragments in groups of four k-steps,
  // loaded again from global memory so that the chains' AGPR operands are
  // their only use (the register allocator then leaves them in place), and
  // the lane's addresses, relative to a K tile, of chunk 0 of its K row (row
  // reads) and of block 0's two transposed reads
  f32x16 qo[kChains ? 8 : 1];
  int rofs = 0, tofs1 = 0, tofs2 = 0;
  if constexpr (kChains) {
#pragma unroll
    for (int g = 0; g < 8; ++g)
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int ds = (g & 3) * 4 + f;
        const __bf16* __restrict__ src = g < 4 ? Q : dO;
        const f32x4 v =
            ds < kDSteps ? *(const f32x4*)(src + (size_t)crow * D + ds * 16 + half * 8) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) qo[g][f * 4 + i] = v[i];
      }
    const int kr0 = kpart * 32, g4 = lane >> 4, j16 = lane & 15;
    rofs = lds_off_bytes<DP>(kr0 + l32, half);
    const int r1 = kr0 + half * 4 + (j16 >> 2), dcol = (g4 & 1) * 16 + (j16 & 3) * 4;
    tofs1 = lds_off_bytes<DP>(r1, dcol >> 3) + (dcol & 7) * 2;
    tofs2 = lds_off_bytes<DP>(r1 + 8, dcol >> 3) + (dcol & 7) * 2;
  }

  for (int j = 0; j < nt; ++j) {
    wait_vmcnt<0>();
    __syncthreads();
    if (j + 1 < nt) copy_tile(j + 1, (j + 1) & 1);
    if (!wave_active || j > wave_last) continue;
    const lds_char* kt = kbuf[j & 1];
    const lds_char* vt = vbuf[j & 1];

    // S^T = K_j Q^T and dP^T = V_j dO^T, keys kr0 + kb*32.. (rows), this wave's queries (columns)
    const int kr0 = kpart * 32;
    const int tb = (int)(uint32_t)(uintptr_t)kt;
    f32x16 s[KB], dp[KB];
    if constexpr (kChains) {
      dq_sdp_chain<kDSteps>(tb + rofs, qo, s[0], dp[0]);
    } else {
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
    }

    const bool masked = (CAUSAL && j == wave_last) || (j == n_ktiles_all - 1 && (N % kKeyTile) != 0);
    bf16x8 dsk[KB][2];  // dS^T packed: [key block][16-key chunk]
    // dS^T = P^T (dP^T - delta), with the key mask only on the tiles that
    // need it (the empty asm keeps the two variants apart: merged, the
    // mask's compares and selects ran on every tile)
    auto make_ds = [&](auto mask_tag) {
      constexpr bool kMask = decltype(mask_tag)::value;
      asm volatile("" ::: "memory");
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
              if (kMask && (kSplitMask || masked)) {
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
    };
    if (!kSplitMask || masked)
      make_ds(std::true_type{});
    else
      make_ds(std::false_type{});

    // dQ^T += K_j^T dS^T
    if constexpr (kChains) {
      dq_tr_chain<kDBlocks>(tb + tofs1, tb + tofs2, dsk[0][0], dsk[0][1], dq[0], dq[1], dq[2], dq[3], dq[4],
                            dq[kAcc - 3], dq[kAcc - 2], dq[kAcc - 1]);
    } else {
#pragma unroll
      for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int cc = 0; cc < 2; ++cc)
            dq[db] = mfma32(read_tr_operand<DP>(kt, kr0 + kb * 32 + cc * 16, db * 32, lane), dsk[kb][cc], dq[db]);
    }
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
