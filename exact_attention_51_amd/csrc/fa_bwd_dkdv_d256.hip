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
// The loop is skewed by one query tile so that a step has two independent
// halves of MFMA work: step i forms S (or dP) of tile i and publishes P (or
// dP) to the exchange, then finishes tile i-1 (dV, dK).  dS of tile i-1 is
// formed once, by the dP wave from the P the S wave published the step
// before, and reaches the S wave through the exchange across a barrier in
// the middle of the step.  Query tiles live two steps (a 3-slot ring) and
// the exchange is triple-buffered (by tile, as the ring).
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
  static constexpr int kXsBytes = 2 * 64 * 16;  // dS: as P
  static constexpr int kSlotBytes = 2 * kTileBytes + 2 * kStatBytes;  // Q, dO, L, delta of one tile
  static constexpr int kXGroupBytes = kXpBytes + kXdBytes + kXsBytes;  // one key group
  static constexpr int kXBytes = 2 * kXGroupBytes;                     // both key groups
  static constexpr int kLdsBytes = 3 * kSlotBytes + 3 * kXBytes;
  static_assert(kLdsBytes <= 160 * 1024, "LDS of one workgroup");
};

// The next query tile's copy, issued from inside the step (one load after
// each of its first 8 MFMAs): 4 loads of Q rows, then 4 of dO rows, from
// global bases qg, og plus the lane's byte offsets off[i] to LDS lq, lo +
// 1024 i.  Issued in one burst after the step's barrier, the 8 loads of 1 KB
// stalled the wave for about 500 cycles while the vector memory path
// drained them.
struct KvCopy {
  uint64_t qg, og;
  uint32_t lq, lo;
  uint32_t off[4];
};

// ------------------------------------------------ one pipelined query-tile step
//
// One asm block per query tile t.  The S wave (dh = 0) runs the NS S MFMAs
// of tile t, then the 4 NB dV/dK MFMAs of tile t-1 with, in their shadow,
// the exponentials of tile t, and publishes P of tile t at the end.  The dP
// wave runs the NS dP MFMAs of tile t with, in their shadow, dS of tile t-1
// (from P the S wave published last step and its own dP), publishes dS
// before a barrier in the middle of the step, then its dV/dK MFMAs of tile
// t-1 and dP of tile t.  The S wave reads dS after that barrier; its dV
// MFMAs, which need none, go first.  So each wave carries one of the two
// element-wise passes (16 exponentials or 16 dS per lane and tile): one
// wave per SIMD issues a vector instruction only every ~9 cycles, and the
// step waits for its slowest wave.  The LDS reads run six fragments ahead
// of their MFMA across both chains, and the next tile's copy goes out
// between the first eight MFMAs.  Per element the arithmetic is the plain
// loop's, instruction for instruction: dS = float(P) (dP - delta),
// P = exp2(fma(S, c, -L log2 e)), pairs packed to bf16 with round to
// nearest even.
//
// mode (wave-uniform): bit 0 tile t is this wave's (S or dP chain), bit 1
// tile t-1 is (dS and the dV/dK chain), bit 2 the exponentials (or dP's
// store) go in the block too -- left out for a masked tile, which the
// caller finishes from the returned S.  Every mode passes the middle
// barrier once.
//
// Registers: K or V rows in a[0:63] (fragment ds at a[4 ds : 4 ds + 3]); S
// or dP of tile t in v[152:167]; L of tile t in v[168:183], whose first 8
// registers then take tile t's packed P; tile t-1's packed P in v[184:191],
// its dP in v[192:207], delta in v[208:223], packed dS in v[224:231]; six
// fragment buffers in v[232:255]; temporaries v148, v149.
// Addresses: r[ds] the lane's row fragment ds (< 8) in tile t's Q or dO
// slot, fragment ds + 8 256 bytes further; ta[i], tb[i] the two transposed
// reads of local d block i in tile t-1's Q slot (queries 16..31 8192 bytes
// further, the dO slot 16384); xpr, xpw the lane's exchange entries of
// tiles t-1 and t (P at +0 and +1024, dP at +2048 + 1024 g, dS at +6144 and
// +7168); dlr delta of tile t-1, llr L of tile t (four runs 32 bytes apart).
#define KS_DSCHK(N) "  .if (" #N " >= (\\lo)) && (" #N " < (\\hi))\n    KS_DS1 " #N "\n  .endif\n"
#define KS_EXCHK(N) "  .if (" #N " >= (\\lo)) && (" #N " < (\\hi))\n    KS_EX1 " #N "\n  .endif\n"
#define KS_SMC(N) "  KS_SM " #N ", \\nsx, \\kv, \\ds, \\lr, \\bs, \\bp\n"
#define KS_KMC(N) "  KS_KM " #N ", \\nsx, \\ex, \\bs, \\bp\n"
#define KS_LGK(N) "  .elseif (\\n) == " #N "\n    s_waitcnt lgkmcnt(" #N ")\n"
#define KV_STEP_TEXT                                                                                               \
  ".macro KS_WAIT n\n"                                                                                             \
  "  .if (\\n) <= 0\n    s_waitcnt lgkmcnt(0)\n"                                                                   \
  KS_LGK(1) KS_LGK(2) KS_LGK(3) KS_LGK(4) KS_LGK(5) KS_LGK(6) KS_LGK(7) KS_LGK(8) KS_LGK(9) KS_LGK(10) KS_LGK(11)   \
  KS_LGK(12) KS_LGK(13) KS_LGK(14)                                                                                 \
  "  .endif\n"                                                                                                     \
  ".endm\n"                                                                                                        \
  /* copy load n: Q rows (n < 4) or dO rows, load n mod 4 of the wave's share; M0 is set one */                \
  /* instruction ahead (a DMA load may not read M0 right after its write) */                                      \
  ".macro KC_M0 n\n"                                                                                               \
  "  .if ((\\n) >> 2) == 0\n    s_add_u32 m0, %[lq], ((\\n) & 3) * 1024\n"                                        \
  "  .else\n    s_add_u32 m0, %[lo], ((\\n) & 3) * 1024\n  .endif\n"                                              \
  ".endm\n"                                                                                                        \
  ".macro KC_LD n\n"                                                                                               \
  "  .if (\\n) == 0\n    global_load_lds_dwordx4 %[o0], %[qg]\n"                                                   \
  "  .elseif (\\n) == 1\n    global_load_lds_dwordx4 %[o1], %[qg]\n"                                               \
  "  .elseif (\\n) == 2\n    global_load_lds_dwordx4 %[o2], %[qg]\n"                                               \
  "  .elseif (\\n) == 3\n    global_load_lds_dwordx4 %[o3], %[qg]\n"                                               \
  "  .elseif (\\n) == 4\n    global_load_lds_dwordx4 %[o0], %[og]\n"                                               \
  "  .elseif (\\n) == 5\n    global_load_lds_dwordx4 %[o1], %[og]\n"                                               \
  "  .elseif (\\n) == 6\n    global_load_lds_dwordx4 %[o2], %[og]\n"                                               \
  "  .else\n    global_load_lds_dwordx4 %[o3], %[og]\n  .endif\n"                                                 \
  ".endm\n"                                                                                                        \
  /* tile t-1's P; for the dP wave also its dP and delta */                                                       \
  ".macro KS_XR\n"                                                                                                 \
  "  ds_read_b128 v[184:187], %[xpr]\n  ds_read_b128 v[188:191], %[xpr] offset:1024\n"                             \
  "  .if %[dh] == 1\n"                                                                                             \
  "    ds_read_b128 v[192:195], %[xpr] offset:2048\n    ds_read_b128 v[196:199], %[xpr] offset:3072\n"             \
  "    ds_read_b128 v[200:203], %[xpr] offset:4096\n    ds_read_b128 v[204:207], %[xpr] offset:5120\n"             \
  "    ds_read_b128 v[208:211], %[dlr]\n    ds_read_b128 v[212:215], %[dlr] offset:32\n"                           \
  "    ds_read_b128 v[216:219], %[dlr] offset:64\n    ds_read_b128 v[220:223], %[dlr] offset:96\n"                 \
  "  .endif\n"                                                                                                     \
  ".endm\n"                                                                                                        \
  /* tile t's L (4 reads, S wave) */                                                                              \
  ".macro KS_LR\n"                                                                                                 \
  "  .if %[dh] == 0\n"                                                                                             \
  "    ds_read_b128 v[168:171], %[llr]\n    ds_read_b128 v[172:175], %[llr] offset:32\n"                           \
  "    ds_read_b128 v[176:179], %[llr] offset:64\n    ds_read_b128 v[180:183], %[llr] offset:96\n"                 \
  "  .endif\n"                                                                                                     \
  ".endm\n"                                                                                                        \
  /* S/dP fragment p (one read) into buffer p mod 6 */                                                            \
  ".macro KS_RX p\n"                                                                                               \
  "  .if ((\\p) & 7) == 0\n    ds_read_b128 v[232 + ((\\p) %% 6) * 4 : 235 + ((\\p) %% 6) * 4], %[r0] "          \
  "offset:(((\\p) >> 3) * 256)\n"                                                                                  \
  "  .elseif ((\\p) & 7) == 1\n    ds_read_b128 v[232 + ((\\p) %% 6) * 4 : 235 + ((\\p) %% 6) * 4], %[r1] "      \
  "offset:(((\\p) >> 3) * 256)\n"                                                                                  \
  "  .elseif ((\\p) & 7) == 2\n    ds_read_b128 v[232 + ((\\p) %% 6) * 4 : 235 + ((\\p) %% 6) * 4], %[r2] "      \
  "offset:(((\\p) >> 3) * 256)\n"                                                                                  \
  "  .elseif ((\\p) & 7) == 3\n    ds_read_b128 v[232 + ((\\p) %% 6) * 4 : 235 + ((\\p) %% 6) * 4], %[r3] "      \
  "offset:(((\\p) >> 3) * 256)\n"                                                                                  \
  "  .elseif ((\\p) & 7) == 4\n    ds_read_b128 v[232 + ((\\p) %% 6) * 4 : 235 + ((\\p) %% 6) * 4], %[r4] "      \
  "offset:(((\\p) >> 3) * 256)\n"                                                                                  \
  "  .elseif ((\\p) & 7) == 5\n    ds_read_b128 v[232 + ((\\p) %% 6) * 4 : 235 + ((\\p) %% 6) * 4], %[r5] "      \
  "offset:(((\\p) >> 3) * 256)\n"                                                                                  \
  "  .elseif ((\\p) & 7) == 6\n    ds_read_b128 v[232 + ((\\p) %% 6) * 4 : 235 + ((\\p) %% 6) * 4], %[r6] "      \
  "offset:(((\\p) >> 3) * 256)\n"                                                                                  \
  "  .else\n    ds_read_b128 v[232 + ((\\p) %% 6) * 4 : 235 + ((\\p) %% 6) * 4], %[r7] "                         \
  "offset:(((\\p) >> 3) * 256)\n"                                                                                  \
  "  .endif\n"                                                                                                     \
  ".endm\n"                                                                                                        \
  /* dV/dK fragment (query chunk cc, local d block i, dv: dO^T, else Q^T) into buffer p mod 6 (two reads) */      \
  ".macro KS_TR2 ra, rb, off, p\n"                                                                                 \
  "  ds_read_b64_tr_b16 v[232 + ((\\p) %% 6) * 4 : 233 + ((\\p) %% 6) * 4], \\ra offset:(\\off)\n"               \
  "  ds_read_b64_tr_b16 v[234 + ((\\p) %% 6) * 4 : 235 + ((\\p) %% 6) * 4], \\rb offset:(\\off)\n"               \
  ".endm\n"                                                                                                        \
  ".macro KS_TX cc, i, dv, p\n"                                                                                    \
  "  .if (\\i) == 0\n    KS_TR2 %[ta0], %[tb0], ((\\cc) * 8192 + (\\dv) * 16384), (\\p)\n"                         \
  "  .elseif (\\i) == 1\n    KS_TR2 %[ta1], %[tb1], ((\\cc) * 8192 + (\\dv) * 16384), (\\p)\n"                     \
  "  .elseif (\\i) == 2\n    KS_TR2 %[ta2], %[tb2], ((\\cc) * 8192 + (\\dv) * 16384), (\\p)\n"                     \
  "  .else\n    KS_TR2 %[ta3], %[tb3], ((\\cc) * 8192 + (\\dv) * 16384), (\\p)\n  .endif\n"                       \
  ".endm\n"                                                                                                        \
  /* stream position p: S/dP fragments, then with kv the dV fragments (cc outer, block inner), then dK's */       \
  ".macro KS_RD p, nsx, kv\n"                                                                                      \
  "  .if (\\p) < (\\nsx)\n"                                                                                        \
  "    KS_RX (\\p)\n"                                                                                              \
  "  .elseif (\\kv) && ((\\p) < (\\nsx) + 2 * %[nb])\n"                                                            \
  "    KS_TX (((\\p) - (\\nsx)) / %[nb]), (((\\p) - (\\nsx)) %% %[nb]), 1, (\\p)\n"                               \
  "  .elseif (\\kv) && ((\\p) < (\\nsx) + 4 * %[nb])\n"                                                            \
  "    KS_TX (((\\p) - (\\nsx) - 2 * %[nb]) / %[nb]), (((\\p) - (\\nsx) - 2 * %[nb]) %% %[nb]), 0, (\\p)\n"       \
  "  .endif\n"                                                                                                     \
  ".endm\n"                                                                                                        \
  ".macro KS_RD6 nsx, kv\n"                                                                                        \
  "  KS_RD 0, \\nsx, \\kv\n  KS_RD 1, \\nsx, \\kv\n  KS_RD 2, \\nsx, \\kv\n"                                      \
  "  KS_RD 3, \\nsx, \\kv\n  KS_RD 4, \\nsx, \\kv\n  KS_RD 5, \\nsx, \\kv\n"                                      \
  ".endm\n"                                                                                                        \
  /* wait until at most the reads of stream positions a..b-1 (one each before nsx, two after) plus x remain */   \
  ".macro KS_WT2 a, b, nsx, x\n"                                                                                   \
  "  .if (\\b) <= (\\nsx)\n    KS_WAIT ((\\b) - (\\a) + (\\x))\n"                                                  \
  "  .elseif (\\a) >= (\\nsx)\n    KS_WAIT (2 * ((\\b) - (\\a)) + (\\x))\n"                                        \
  "  .else\n    KS_WAIT (((\\nsx) - (\\a)) + 2 * ((\\b) - (\\nsx)) + (\\x))\n  .endif\n"                           \
  ".endm\n"                                                                                                        \
  ".macro KS_WT3 m, nsx, kv, x\n"                                                                                  \
  "  .if (\\m) + 6 <= (\\nsx) + 4 * %[nb] * (\\kv)\n    KS_WT2 ((\\m) + 1), ((\\m) + 6), (\\nsx), (\\x)\n"      \
  "  .else\n    KS_WT2 ((\\m) + 1), ((\\nsx) + 4 * %[nb] * (\\kv)), (\\nsx), (\\x)\n  .endif\n"                   \
  ".endm\n"                                                                                                        \
  /* before the MFMA of position m: its fragment landed.  Positions m+1..m+5 may be in flight, and also */       \
  /* the lr L reads issued after position 5 (m < 6) and the two dS reads issued after the middle barrier, */     \
  /* which follows the MFMA of position bs and the read of position bs + 6 (bs < m <= bs + 6) */                  \
  ".macro KS_WT m, nsx, kv, lr, bs\n"                                                                              \
  "  .if ((\\m) > (\\bs)) && ((\\m) <= (\\bs) + 6)\n"                                                              \
  "    .if (\\m) < 6\n      KS_WT3 (\\m), (\\nsx), (\\kv), ((\\lr) + 2)\n"                                         \
  "    .else\n      KS_WT3 (\\m), (\\nsx), (\\kv), 2\n    .endif\n"                                                  \
  "  .else\n"                                                                                                      \
  "    .if (\\m) < 6\n      KS_WT3 (\\m), (\\nsx), (\\kv), (\\lr)\n"                                               \
  "    .else\n      KS_WT3 (\\m), (\\nsx), (\\kv), 0\n    .endif\n"                                                  \
  "  .endif\n"                                                                                                     \
  ".endm\n"                                                                                                        \
  /* dS half-step h of pair k = h/2 (elements 2k, 2k+1; P word k): unpack and dP - delta, then product and pack */ \
  ".macro KS_DS1 h\n"                                                                                              \
  "  .if ((\\h) & 1) == 0\n"                                                                                       \
  "    v_lshlrev_b32 v148, 16, v[184 + ((\\h) >> 1)]\n"                                                            \
  "    v_and_b32 v149, 0xffff0000, v[184 + ((\\h) >> 1)]\n"                                                        \
  "    v_sub_f32 v[192 + (\\h)], v[192 + (\\h)], v[208 + (\\h)]\n"                                                 \
  "    v_sub_f32 v[193 + (\\h)], v[193 + (\\h)], v[209 + (\\h)]\n"                                                 \
  "  .else\n"                                                                                                      \
  "    v_mul_f32 v148, v148, v[191 + (\\h)]\n"                                                                     \
  "    v_mul_f32 v149, v149, v[192 + (\\h)]\n"                                                                     \
  "    v_cvt_pk_bf16_f32 v[224 + ((\\h) >> 1)], v148, v149\n"                                                      \
  "  .endif\n"                                                                                                     \
  ".endm\n"                                                                                                        \
  ".macro KS_DSR lo, hi\n"                                                                                         \
  KS_DSCHK(0) KS_DSCHK(1) KS_DSCHK(2) KS_DSCHK(3) KS_DSCHK(4) KS_DSCHK(5) KS_DSCHK(6) KS_DSCHK(7)                  \
  KS_DSCHK(8) KS_DSCHK(9) KS_DSCHK(10) KS_DSCHK(11) KS_DSCHK(12) KS_DSCHK(13) KS_DSCHK(14) KS_DSCHK(15)            \
  ".endm\n"                                                                                                        \
  /* exponential slot s (S wave): element s's exponent, element s-1's exp2, pair (s-3)/2's pack -- an */        \
  /* exp2 result is read no sooner than one instruction later */                                                  \
  ".macro KS_EX1 s\n"                                                                                              \
  "  .if %[dh] == 0\n"                                                                                             \
  "    .if (\\s) < 16\n"                                                                                           \
  "      v_mul_f32 v[168 + (\\s)], 0xbfb8aa3b, v[168 + (\\s)]\n"                                                   \
  "      v_fma_f32 v[152 + (\\s)], v[152 + (\\s)], %[c], v[168 + (\\s)]\n"                                         \
  "    .endif\n"                                                                                                   \
  "    .if ((\\s) >= 1) && ((\\s) <= 16)\n"                                                                        \
  "      v_exp_f32 v[151 + (\\s)], v[151 + (\\s)]\n"                                                               \
  "    .endif\n"                                                                                                   \
  "    .if (\\s) == 17\n      s_nop 0\n    .endif\n"                                                             \
  "    .if ((\\s) >= 3) && (((\\s) & 1) == 1)\n"                                                                   \
  "      v_cvt_pk_bf16_f32 v[168 + ((\\s) - 3) / 2], v[149 + (\\s)], v[150 + (\\s)]\n"                             \
  "    .endif\n"                                                                                                   \
  "  .endif\n"                                                                                                     \
  ".endm\n"                                                                                                        \
  ".macro KS_EXR lo, hi\n"                                                                                         \
  KS_EXCHK(0) KS_EXCHK(1) KS_EXCHK(2) KS_EXCHK(3) KS_EXCHK(4) KS_EXCHK(5) KS_EXCHK(6) KS_EXCHK(7)                  \
  KS_EXCHK(8) KS_EXCHK(9) KS_EXCHK(10) KS_EXCHK(11) KS_EXCHK(12) KS_EXCHK(13) KS_EXCHK(14) KS_EXCHK(15)            \
  KS_EXCHK(16) KS_EXCHK(17)                                                                                        \
  ".endm\n"                                                                                                        \
  /* tile t's P (S wave) or dP (dP wave) to the exchange */                                                       \
  ".macro KS_ST\n"                                                                                                 \
  "  s_nop 1\n"                                                                                                    \
  "  .if %[dh] == 0\n"                                                                                             \
  "    ds_write_b128 %[xpw], v[168:171]\n    ds_write_b128 %[xpw], v[172:175] offset:1024\n"                       \
  "  .else\n"                                                                                                      \
  "    ds_write_b128 %[xpw], v[152:155] offset:2048\n    ds_write_b128 %[xpw], v[156:159] offset:3072\n"           \
  "    ds_write_b128 %[xpw], v[160:163] offset:4096\n    ds_write_b128 %[xpw], v[164:167] offset:5120\n"           \
  "  .endif\n"                                                                                                     \
  ".endm\n"                                                                                                        \
  /* the middle barrier; with kv the dP wave publishes tile t-1's dS before it and the S wave reads it after */  \
  ".macro KS_MB kv\n"                                                                                              \
  "  .if %[dh] == 1\n"                                                                                             \
  "    .if (\\kv)\n"                                                                                               \
  "      s_nop 1\n"                                                                                                \
  "      ds_write_b128 %[xpr], v[224:227] offset:6144\n      ds_write_b128 %[xpr], v[228:231] offset:7168\n"       \
  "      s_waitcnt lgkmcnt(0)\n"                                                                                   \
  "    .endif\n"                                                                                                   \
  "    s_barrier\n"                                                                                                \
  "  .else\n"                                                                                                      \
  "    s_barrier\n"                                                                                                \
  "    .if (\\kv)\n"                                                                                               \
  "      ds_read_b128 v[224:227], %[xpr] offset:6144\n      ds_read_b128 v[228:231], %[xpr] offset:7168\n"         \
  "    .endif\n"                                                                                                   \
  "  .endif\n"                                                                                                     \
  ".endm\n"                                                                                                        \
  /* S/dP MFMA m, the read of position m+6, copy load m (m < 8), dS half-steps (dP wave, with ds), and */        \
  /* the middle barrier after position bp */                                                                      \
  ".macro KS_SM m, nsx, kv, ds, lr, bs, bp\n"                                                                      \
  "  .if (\\m) < (\\nsx)\n"                                                                                        \
  "    KS_WT (\\m), (\\nsx), (\\kv), (\\lr), (\\bs)\n"                                                             \
  "    .if (\\m) == 0\n"                                                                                           \
  "      v_mfma_f32_32x32x16_bf16 v[152:167], v[232 + ((\\m) %% 6) * 4 : 235 + ((\\m) %% 6) * 4], "                \
  "a[(\\m) * 4 : (\\m) * 4 + 3], 0\n"                                                                             \
  "    .else\n"                                                                                                    \
  "      v_mfma_f32_32x32x16_bf16 v[152:167], v[232 + ((\\m) %% 6) * 4 : 235 + ((\\m) %% 6) * 4], "                \
  "a[(\\m) * 4 : (\\m) * 4 + 3], v[152:167]\n"                                                                     \
  "    .endif\n"                                                                                                   \
  "    .if (\\m) < 8\n      KC_M0 (\\m)\n    .endif\n"                                                           \
  "    KS_RD ((\\m) + 6), (\\nsx), (\\kv)\n"                                                                       \
  "    .if (\\m) < 8\n      KC_LD (\\m)\n    .endif\n"                                                           \
  "    .if (\\ds) && (%[dh] == 1)\n"                                                                               \
  "      KS_DSR (((\\m) * 16) / ((\\nsx) - 1)), ((((\\m) + 1) * 16) / ((\\nsx) - 1))\n"                            \
  "    .endif\n"                                                                                                   \
  "    .if (\\m) == (\\bp)\n      KS_MB (\\kv)\n    .endif\n"                                                      \
  "  .endif\n"                                                                                                     \
  ".endm\n"                                                                                                        \
  /* one dV (dv) or dK MFMA of query chunk cc, local block i, fragment buffer p mod 6 */                           \
  ".macro KS_MF acc, p, vb\n"                                                                                      \
  "  v_mfma_f32_32x32x16_bf16 \\acc, v[232 + ((\\p) %% 6) * 4 : 235 + ((\\p) %% 6) * 4], v[\\vb : (\\vb) + 3], "  \
  "\\acc\n"                                                                                                        \
  ".endm\n"                                                                                                        \
  ".macro KS_KV cc, i, dv, p\n"                                                                                    \
  "  .if (\\dv) && ((\\i) == 0)\n    KS_MF %[dv0], (\\p), (184 + 4 * (\\cc))\n"                                     \
  "  .elseif (\\dv) && ((\\i) == 1)\n    KS_MF %[dv1], (\\p), (184 + 4 * (\\cc))\n"                                 \
  "  .elseif (\\dv) && ((\\i) == 2)\n    KS_MF %[dv2], (\\p), (184 + 4 * (\\cc))\n"                                 \
  "  .elseif (\\dv)\n    KS_MF %[dv3], (\\p), (184 + 4 * (\\cc))\n"                                                  \
  "  .elseif (\\i) == 0\n    KS_MF %[dk0], (\\p), (224 + 4 * (\\cc))\n"                                               \
  "  .elseif (\\i) == 1\n    KS_MF %[dk1], (\\p), (224 + 4 * (\\cc))\n"                                               \
  "  .elseif (\\i) == 2\n    KS_MF %[dk2], (\\p), (224 + 4 * (\\cc))\n"                                               \
  "  .else\n    KS_MF %[dk3], (\\p), (224 + 4 * (\\cc))\n  .endif\n"                                                 \
  ".endm\n"                                                                                                        \
  /* dV/dK MFMA f (position nsx + f; dV for f < 2 nb), the read 6 ahead, the exponential slots (S wave, */       \
  /* with ex), and the middle barrier after position bp */                                                        \
  ".macro KS_KM f, nsx, ex, bs, bp\n"                                                                              \
  "  .if (\\f) < 4 * %[nb]\n"                                                                                      \
  "    KS_WT ((\\nsx) + (\\f)), (\\nsx), 1, 0, (\\bs)\n"                                                           \
  "    .if (\\f) < 2 * %[nb]\n"                                                                                    \
  "      KS_KV ((\\f) / %[nb]), ((\\f) %% %[nb]), 1, ((\\nsx) + (\\f))\n"                                          \
  "    .else\n"                                                                                                    \
  "      KS_KV (((\\f) - 2 * %[nb]) / %[nb]), (((\\f) - 2 * %[nb]) %% %[nb]), 0, ((\\nsx) + (\\f))\n"              \
  "    .endif\n"                                                                                                   \
  "    KS_RD ((\\nsx) + (\\f) + 6), (\\nsx), 1\n"                                                                  \
  "    .if (\\ex) && (%[dh] == 0)\n"                                                                               \
  "      .if (\\f) == 0\n        s_nop 7\n        s_nop 7\n        s_nop 7\n      .endif\n"                        \
  "      KS_EXR (((\\f) * 18) / (4 * %[nb])), ((((\\f) + 1) * 18) / (4 * %[nb]))\n"                                \
  "    .endif\n"                                                                                                   \
  "    .if ((\\nsx) + (\\f)) == (\\bp)\n      KS_MB 1\n    .endif\n"                                             \
  "  .endif\n"                                                                                                     \
  ".endm\n"                                                                                                        \
  ".macro KS_SMS nsx, kv, ds, lr, bs, bp\n"                                                                        \
  KS_SMC(0) KS_SMC(1) KS_SMC(2) KS_SMC(3) KS_SMC(4) KS_SMC(5) KS_SMC(6) KS_SMC(7)                                  \
  KS_SMC(8) KS_SMC(9) KS_SMC(10) KS_SMC(11) KS_SMC(12) KS_SMC(13) KS_SMC(14) KS_SMC(15)                            \
  ".endm\n"                                                                                                        \
  ".macro KS_KMS nsx, ex, bs, bp\n"                                                                                \
  KS_KMC(0) KS_KMC(1) KS_KMC(2) KS_KMC(3) KS_KMC(4) KS_KMC(5) KS_KMC(6) KS_KMC(7)                                  \
  KS_KMC(8) KS_KMC(9) KS_KMC(10) KS_KMC(11) KS_KMC(12) KS_KMC(13) KS_KMC(14) KS_KMC(15)                            \
  ".endm\n"                                                                                                        \
  /* the middle barrier's position with both chains: after the S wave's first 2 nb - 6 dV MFMAs (so that */     \
  /* every dK fragment is read after dS), after the dP chain for the dP wave */                                   \
  ".set ks_bp, (%[ns] - 1 + (1 - %[dh]) * (2 * %[nb] - 6))\n"                                                      \
  ".set ks_bs, (ks_bp - 1000 * %[dh])\n"                                                                           \
  "s_cmp_eq_u32 %[mode], 7\ns_cbranch_scc1 L_full_%=\n"                                                            \
  "s_cmp_eq_u32 %[mode], 3\ns_cbranch_scc1 L_p12_%=\n"                                                             \
  "s_cmp_eq_u32 %[mode], 5\ns_cbranch_scc1 L_p1e_%=\n"                                                             \
  "s_cmp_eq_u32 %[mode], 1\ns_cbranch_scc1 L_p1_%=\n"                                                              \
  "s_cmp_eq_u32 %[mode], 2\ns_cbranch_scc1 L_p2_%=\n"                                                              \
  "s_barrier\n"                                                                                                    \
  "s_branch L_end_%=\n"                                                                                            \
  "L_full_%=:\n"                                                                                                   \
  "KS_XR\nKS_RD6 %[ns], 1\nKS_LR\nKS_SMS %[ns], 1, 1, (4 - 4 * %[dh]), ks_bs, ks_bp\n"                             \
  "KS_KMS %[ns], 1, ks_bs, ks_bp\nKS_ST\n"                                                                         \
  "s_branch L_end_%=\n"                                                                                            \
  "L_p12_%=:\n"                                                                                                    \
  "KS_XR\nKS_RD6 %[ns], 1\nKS_SMS %[ns], 1, 1, 0, ks_bs, ks_bp\nKS_KMS %[ns], 0, ks_bs, ks_bp\n"                   \
  "s_branch L_end_%=\n"                                                                                            \
  "L_p1e_%=:\n"                                                                                                    \
  "KS_RD6 %[ns], 0\nKS_LR\nKS_SMS %[ns], 0, 0, (4 - 4 * %[dh]), -1000, (%[ns] - 1)\n"                              \
  "s_nop 7\ns_nop 7\ns_nop 7\n"                                                                                    \
  "KS_EXR 0, 18\nKS_ST\n"                                                                                          \
  "s_branch L_end_%=\n"                                                                                            \
  "L_p1_%=:\n"                                                                                                     \
  "KS_RD6 %[ns], 0\nKS_SMS %[ns], 0, 0, 0, -1000, (%[ns] - 1)\n"                                                   \
  "s_nop 7\ns_nop 7\ns_nop 7\n" /* S may be read by vector instructions next */                                  \
  "s_branch L_end_%=\n"                                                                                            \
  "L_p2_%=:\n"                                                                                                     \
  "KS_XR\n"                                                                                                        \
  ".if %[dh] == 1\n  s_waitcnt lgkmcnt(0)\n  KS_DSR 0, 16\n.endif\n"                                               \
  "KS_MB 1\nKS_RD6 0, 1\nKS_KMS 0, 0, -1000, -1000\n"                                                              \
  "L_end_%=:\n"                                                                                                    \
  ".purgem KS_WAIT\n.purgem KC_M0\n.purgem KC_LD\n.purgem KS_XR\n.purgem KS_LR\n.purgem KS_RX\n.purgem KS_TR2\n"                  \
  ".purgem KS_TX\n.purgem KS_RD\n.purgem KS_RD6\n.purgem KS_WT2\n.purgem KS_WT3\n.purgem KS_WT\n"                  \
  ".purgem KS_DS1\n.purgem KS_DSR\n.purgem KS_EX1\n.purgem KS_EXR\n.purgem KS_ST\n.purgem KS_MB\n"                 \
  ".purgem KS_SM\n.purgem KS_MF\n.purgem KS_KV\n.purgem KS_KM\n.purgem KS_SMS\n.purgem KS_KMS\n"
#define KV_STEP_IN                                                                                                 \
  [ns] "i"(NS), [nb] "i"(NB), [dh] "i"(DH), [mode] "s"(mode), [r0] "v"(r[0]), [r1] "v"(r[1]), \
                 [r2] "v"(r[2]), [r3] "v"(r[3]), [r4] "v"(r[4]), [r5] "v"(r[5]), [r6] "v"(r[6]), [r7] "v"(r[7]), \
                 [ta0] "v"(ta[0]), [ta1] "v"(ta[1]), [ta2] "v"(ta[2]), [ta3] "v"(ta[3]), [tb0] "v"(tb[0]), \
                 [tb1] "v"(tb[1]), [tb2] "v"(tb[2]), [tb3] "v"(tb[3]), [xpr] "v"(xpr), [xpw] "v"(xpw), [dlr] "v"(dlr), \
                 [llr] "v"(llr), [c] "v"(c), [qg] "s"(cp.qg), [og] "s"(cp.og), [lq] "s"(cp.lq), [lo] "s"(cp.lo), \
                 [o0] "v"(cp.off[0]), [o1] "v"(cp.off[1]), [o2] "v"(cp.off[2]), \
                 [o3] "v"(cp.off[3]), "{a[0:15]}"(kvg[0]), "{a[16:31]}"(kvg[1]), "{a[32:47]}"(kvg[2]), \
                 "{a[48:63]}"(kvg[3])
#define KV_STEP_CLOB                                                                                               \
  "memory", "scc", "m0", "v148", "v149", "v168", "v169", "v170", "v171", "v172", "v173", "v174", \
                 "v175", "v176", "v177", "v178", "v179", "v180", "v181", "v182", "v183", "v184", "v185", "v186", "v187", \
                 "v188", "v189", "v190", "v191", "v192", "v193", "v194", "v195", "v196", "v197", "v198", "v199", "v200", \
                 "v201", "v202", "v203", "v204", "v205", "v206", "v207", "v208", "v209", "v210", "v211", "v212", "v213", \
                 "v214", "v215", "v216", "v217", "v218", "v219", "v220", "v221", "v222", "v223", "v224", "v225", "v226", \
                 "v227", "v228", "v229", "v230", "v231", "v232", "v233", "v234", "v235", "v236", "v237", "v238", "v239", \
                 "v240", "v241", "v242", "v243", "v244", "v245", "v246", "v247", "v248", "v249", "v250", "v251", "v252", \
                 "v253", "v254", "v255"

// acc[i]: dV block i, acc[4 + i]: dK block i (i < NB; the rest unused, and
// their operand names taken by immediates that the assembler never sees)
template <int NS, int NB, int DH>
__device__ __forceinline__ void kv_step(int mode, const int (&r)[8], const int (&ta)[4], const int (&tb)[4], int xpr,
                                        int xpw, int dlr, int llr, float c, const KvCopy& cp, const f32x16 (&kvg)[4],
                                        f32x16& mine, f32x16 (&acc)[8]) {
  static_assert(NS >= 8 && NS <= 16 && NB >= 2 && NB <= 4, "shape");
  if constexpr (NB == 4)
    asm volatile(KV_STEP_TEXT
                 : "=&{v[152:167]}"(mine), [dv0] "+a"(acc[0]), [dv1] "+a"(acc[1]), [dv2] "+a"(acc[2]),
                   [dv3] "+a"(acc[3]), [dk0] "+a"(acc[4]), [dk1] "+a"(acc[5]), [dk2] "+a"(acc[6]), [dk3] "+a"(acc[7])
                 : KV_STEP_IN
                 : KV_STEP_CLOB);
  else if constexpr (NB == 3)
    asm volatile(KV_STEP_TEXT
                 : "=&{v[152:167]}"(mine), [dv0] "+a"(acc[0]), [dv1] "+a"(acc[1]), [dv2] "+a"(acc[2]),
                   [dk0] "+a"(acc[4]), [dk1] "+a"(acc[5]), [dk2] "+a"(acc[6])
                 : KV_STEP_IN, [dv3] "i"(0), [dk3] "i"(0)
                 : KV_STEP_CLOB);
  else
    asm volatile(KV_STEP_TEXT
                 : "=&{v[152:167]}"(mine), [dv0] "+a"(acc[0]), [dv1] "+a"(acc[1]), [dk0] "+a"(acc[4]),
                   [dk1] "+a"(acc[5])
                 : KV_STEP_IN, [dv2] "i"(0), [dv3] "i"(0), [dk2] "i"(0), [dk3] "i"(0)
                 : KV_STEP_CLOB);
}
#undef KV_STEP_TEXT
#undef KV_STEP_IN
#undef KV_STEP_CLOB
#undef KS_DSCHK
#undef KS_EXCHK
#undef KS_SMC
#undef KS_KMC
#undef KS_LGK

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
  auto lds_addr = [](const lds_char* p) { return (int)(uint32_t)(uintptr_t)p; };

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
  // exchange of tile t in buffer t % 3: [key group][P (bf16x8 [cc][lane]),
  // dP (fp32x4 [r/4][lane]: each lane's 16 values as four 16-byte runs),
  // dS (as P)]; the lane's entry of buffer xb
  auto xp = [&](int xb) {
    return (bf16x8 __attribute__((address_space(3)))*)(smem + 3 * C::kSlotBytes + xb * C::kXBytes +
                                                         kgrp * C::kXGroupBytes) + lane;
  };
  auto xlane = [&](int xb) { return lds_addr((const lds_char*)xp(xb)); };

  // query-tile copies: scalar base and loop-invariant per-lane offsets for
  // whole tiles, rows clamped onto N-1 for a ragged last tile
  RowTileCopier<D, DP, C::kQTile, W> cp;
  cp.init(wave, lane);
  auto load_rows = [&](int t) {  // Q and dO rows of tile t
    const int sl = t % 3, row0 = t * C::kQTile;
    if (row0 + C::kQTile <= N) {
      cp.copy_at(Q, (uint32_t)row0 * (D * 2), qbuf(sl));
      cp.copy_at(dO, (uint32_t)row0 * (D * 2), obuf(sl));
    } else {
      cp.copy_clamped(Q, N, row0, qbuf(sl));
      cp.copy_clamped(dO, N, row0, obuf(sl));
    }
  };
  auto load_stats = [&](int t) {  // L and delta of tile t (wave 0)
    const int sl = t % 3;
    if (wave == 0) {
      int r = t * C::kQTile + lane;
      r = r < N ? r : N - 1;
      load_lds4(Lg + r, lbuf(sl));
      load_lds4(Dg + r, dbuf(sl));
    }
  };
  load_rows(t_begin);
  load_stats(t_begin);

  const float c = a.scale_log2;
  // the lane's byte offsets of fragments 0..7 of a row-major tile row l32
  int roff[8];
#pragma unroll
  for (int ds = 0; ds < 8; ++ds) roff[ds] = lds_off_bytes<DP>(l32, ds * 2 + half);

  // The two output halves run separate instances of the loop, each with one
  // step site, so that the accumulators stay in their registers throughout.
  auto run = [&](auto dhc) {
    constexpr int DH = decltype(dhc)::value;
    constexpr int HB = DH * kHalfBlocks;                             // first d block of this half
    constexpr int NB = DH == 0 ? kHalfBlocks : C::kDBlocks - kHalfBlocks;  // its blocks
    // K (S-forming wave) or V (dP-forming wave) of this wave's keys as B
    // operands: key column l32, d = ds*16 + half*8 + 0..7, fragment ds at
    // registers 4*(ds mod 4) of group ds/4.  Past D (D = 160) the step reads
    // no fragment; those registers take a copy of an earlier one, since
    // registers partly set from constants were rebuilt on every step.
    f32x16 kvg[4];
    {
      const __bf16* __restrict__ src = DH == 0 ? K : V;
      const int crow = key < N ? key : N - 1;
#pragma unroll
      for (int ds = 0; ds < 16; ++ds) {
        const int dsl = ds < kDSteps ? ds : ds - 8;
        const bf16x8 f = *(const bf16x8*)(src + (size_t)crow * D + dsl * 16 + half * 8);
        const f32x4 f4 = __builtin_bit_cast(f32x4, f);
#pragma unroll
        for (int i = 0; i < 4; ++i) kvg[ds >> 2][(ds & 3) * 4 + i] = f4[i];
      }
    }
    // the lane's byte offsets of the two transposed reads of d block HB + i
    // (queries 0..15 of a tile: rows r1 and r1 + 8)
    int troff[4], trd2;
    {
      const int g = lane >> 4, j16 = lane & 15;
      const int r1 = half * 4 + (j16 >> 2);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int dcol = (HB + i) * 32 + (g & 1) * 16 + (j16 & 3) * 4;
        troff[i] = lds_off_bytes<DP>(r1, dcol >> 3) + (dcol & 7) * 2;
      }
      // the same for every block: the row swizzles of r1 and r1 + 8 differ in
      // one bit, which meets the same bit of every block's chunk index
      const int dcol0 = HB * 32 + (g & 1) * 16 + (j16 & 3) * 4;
      trd2 = lds_off_bytes<DP>(r1 + 8, dcol0 >> 3) - lds_off_bytes<DP>(r1, dcol0 >> 3);
    }
    // the LDS addresses of a step, fixed per ring slot (the loop runs the
    // slots as three step sites): the row fragments of tile t in slot sl, the
    // transposed reads, delta and exchange entry of tile t-1 in slot (sl+2)%3
    int ra[3][8], ta[3][4], tb[3][4], xa[3], dla[3], lla[3];
#pragma unroll
    for (int sl = 0; sl < 3; ++sl) {
      const int rbase = lds_addr(DH == 0 ? qbuf(sl) : obuf(sl)), tbase = lds_addr(qbuf(sl));
#pragma unroll
      for (int ds = 0; ds < 8; ++ds) ra[sl][ds] = rbase + roff[ds];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ta[sl][i] = tbase + troff[i];
        tb[sl][i] = ta[sl][i] + trd2;
      }
      xa[sl] = xlane(sl);
      dla[sl] = lds_addr(dbuf(sl)) + 16 * half;
      lla[sl] = lds_addr(lbuf(sl)) + 16 * half;
    }
    // (through an empty asm, so that they are kept rather than rebuilt from
    // the offsets on every step)
#pragma unroll
    for (int sl = 0; sl < 3; ++sl) {
#pragma unroll
      for (int ds = 0; ds < 8; ++ds) asm volatile("" : "+v"(ra[sl][ds]));
#pragma unroll
      for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(ta[sl][i]), "+v"(tb[sl][i]));
      asm volatile("" : "+v"(xa[sl]), "+v"(dla[sl]), "+v"(lla[sl]));
    }
    // the step's work as thresholds on t: tile t is this key group's from
    // tile tw0 on (its first key's row under causal masking); P needs the mask
    // on the causal tile tw0 and from the ragged tile nfull on
    const int tw0 = !group_active ? n_qtiles + 1 : CAUSAL ? wk0 / C::kQTile : 0;
    const int nfull = N / C::kQTile;
    // this wave's half of dV^T (acc[0..NB-1]) and dK^T (acc[4..4+NB-1])
    f32x16 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

    // step t (tile t in slot SL = t % 3): S or dP of tile t, dS/dV/dK of tile
    // t-1; steps outside t_begin .. n_qtiles only pass the barriers
    auto step = [&](int t, auto slc) {
      constexpr int SL = decltype(slc)::value, SP = (SL + 2) % 3, SN = (SL + 1) % 3;
      // publishes tile t (loaded last step) and the exchange of tile t-1; the
      // step's own LDS stores may still be in flight here
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      const bool part1 = t >= tw0 && t < n_qtiles;
      const bool part2 = t > tw0 && t <= n_qtiles;
      // tile t+1 into the slot of tile t-2, finished last step: its Q and dO
      // rows from inside the step's first chain (when it has one), else here.
      // From inside the chain a tile reaching past row N-1 takes rows clamped
      // onto it, and a step with no next tile copies such rows into the free
      // slot.
      const int row1 = (t + 1) * C::kQTile;
      KvCopy kc = {(uint64_t)(uintptr_t)(Q + (size_t)row1 * D), (uint64_t)(uintptr_t)(dO + (size_t)row1 * D),
                   (uint32_t)(uintptr_t)qbuf(SN) + cp.lds_wave, (uint32_t)(uintptr_t)obuf(SN) + cp.lds_wave,
                   {cp.off[0], cp.off[1], cp.off[2], cp.off[3]}};
      if (part1) {
        if (row1 + C::kQTile > N) {
          kc.qg = (uint64_t)(uintptr_t)Q;
          kc.og = (uint64_t)(uintptr_t)dO;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int rc = min(row1 + cp.rowi[i], N - 1);
            kc.off[i] = cp.off[i] + (uint32_t)((rc - cp.rowi[i]) * (D * 2));
          }
        }
      } else if (t >= t_begin && t + 1 < n_qtiles) {
        load_rows(t + 1);
      }
      if (t >= t_begin && t + 1 < n_qtiles) load_stats(t + 1);
      const int tq0 = t * C::kQTile;
      // P of a tile that crosses the diagonal or the end of the sequence
      // needs the mask: computed after the step from the returned S
      const bool masked = DH == 0 && ((CAUSAL && t == tw0) || t >= nfull);
      const int mode =
          __builtin_amdgcn_readfirstlane((part1 ? 1 : 0) | (part2 ? 2 : 0) | (part1 && !masked ? 4 : 0));
      f32x16 mine;
      kv_step<kDSteps, NB, DH>(mode, ra[SL], ta[SP], tb[SP], xa[SP], xa[SL], dla[SP], lla[SL], c, kc, kvg, mine, acc);
      if (DH == 0 && part1 && masked) {
        // P = exp(S - L) with the mask; queries of register r: (r/4)*8 + half*4 + r%4
        float lq[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 l4 = *(const f32x4 __attribute__((address_space(3)))*)(lbuf(SL) + 4 * (g * 8 + half * 4));
#pragma unroll
          for (int i = 0; i < 4; ++i) lq[g * 4 + i] = l4[i];
        }
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int qr = (rr >> 2) * 8 + half * 4 + (rr & 3);
          float x = __builtin_fmaf(mine[rr], c, -lq[rr] * kLog2e);
          bool keep = tq0 + qr < N;
          if constexpr (CAUSAL) keep = keep && key <= tq0 + qr;
          mine[rr] = fast_exp2(keep ? x : -__builtin_inff());
        }
        // P rounded to bf16 once; both waves form dS from this rounded P
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          bf16x2 pp[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) pp[i] = pack_bf16(mine[cc * 8 + 2 * i], mine[cc * 8 + 2 * i + 1]);
          xp(SL)[cc * 64] = join8(pp[0], pp[1], pp[2], pp[3]);
        }
      }
    };
    // (t0 through an empty asm: a first step told apart from the rest by the
    // compiler was peeled off the loop, and with more step sites the
    // accumulators were moved out of their registers and back every step)
    for (int t0 = t_begin - t_begin % 3; t0 <= n_qtiles; t0 += 3) {
      int tt = t0;
      asm volatile("" : "+s"(tt));
      step(tt, std::integral_constant<int, 0>());
      step(tt + 1, std::integral_constant<int, 1>());
      step(tt + 2, std::integral_constant<int, 2>());
    }

    // the last MFMAs' results are read next
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    wait_vmcnt<0>();  // no direct-to-LDS copy may outlive the workgroup
    if (!group_active || key >= N) return;
    __bf16* __restrict__ dK = (__bf16*)a.dk + head_off;
    __bf16* __restrict__ dV = (__bf16*)a.dv + head_off;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const size_t off = (size_t)key * D + (HB + i) * 32 + g4 * 8 + half * 4;
        const f32x16& k4 = acc[4 + i];
        const f32x16& v4 = acc[i];
        u32x2 wk = {pack_bf16_u32(k4[g4 * 4 + 0] * a.scale, k4[g4 * 4 + 1] * a.scale),
                    pack_bf16_u32(k4[g4 * 4 + 2] * a.scale, k4[g4 * 4 + 3] * a.scale)};
        u32x2 wv = {pack_bf16_u32(v4[g4 * 4 + 0], v4[g4 * 4 + 1]), pack_bf16_u32(v4[g4 * 4 + 2], v4[g4 * 4 + 3])};
        *(u32x2*)(dK + off) = wk;
        *(u32x2*)(dV + off) = wv;
      }
    }
  };
  if (dh == 0)
    run(std::integral_constant<int, 0>());
  else
    run(std::integral_constant<int, 1>());
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
