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

// ------------------------------------------ pipelined dQ step (DP = 256)
//
// At D = 160 and 256 a wave's work per key tile is 2 NS + 2 NB MFMAs
// (S^T, dP^T, then dQ^T) whose A operands all come from LDS.  One asm
// block per tile j runs S^T/dP^T of tile j, in their shadow dS^T of tile
// j-1 from the S and dP the previous block left, then dQ^T += K_{j-1}^T
// dS^T; its LDS reads run ten fragments ahead of their MFMA across both
// parts.  The block is entered every step with a wave-uniform mode, so
// that the dQ accumulators pass through the loop in place:
//   0  nothing;
//   1  S^T/dP^T only (the first tile);
//   2  the full step;
//   3  dQ^T only, with dS^T given by the caller (a wave's last tile, where
//      the key mask may apply; the in-block dS is the unmasked one).
// At D = 256 every mode also issues this wave's share of the next tile's
// copy (16 global-to-LDS loads of 1 KB), spread between its MFMAs: issued
// in one burst the loads stalled the wave for about a thousand cycles per
// tile while the vector memory path drained them, with the matrix core
// idle.  The full step issues them one per MFMA from its first, which
// leaves them most of the step to land before the next step's wait (spread
// over the whole step they left a wait of about 300 cycles).
// Per element the in-block dS is the plain loop's arithmetic, instruction
// for instruction: x = fma(S, c, -L), p = exp2(x), (dP - delta) p, pairs
// packed to bf16.
//
// Fixed registers: Q^T fragment of k-step ds in a[4 ds : 4 ds + 3], dO^T
// in a[64 + 4 ds : ...]; dQ^T block db in a[128 + 16 db : +15]; S and dP
// of the two alternating sets in v[142:173] and v[174:205] (S in the first
// 16 of a set); dS^T pairs in v[206:213] (elements 2k, 2k+1 in
// v[206 + k]); read and copy addresses formed in v214, v215; ten fragment
// buffers in v[216:255].
//
// Read addresses: a tile row is 512 bytes and 512-aligned in LDS, and the
// swizzle only permutes 16-byte chunks inside each 256-byte half, so the
// lane's address of chunk c ^ swz equals its address of chunk swz with
// the chunk bits flipped by c: one XOR with a constant per read.  rb, rv:
// the lane's chunk-0 address of its K and V row in tile j's slots (k-step
// ds at ^ 32 (ds mod 8), +256 bytes for ds >= 8); t1, t2: its addresses of
// the two transposed reads of tile j-1's block 0 (block db at ^ 64 (db mod
// 4), +256 bytes for db >= 4, second 16 keys +8192).
#define DQ_STEP_TEXT                                                                                               \
  /* s_waitcnt lgkmcnt(n), n an assemble-time expression, at most 15 */                                             \
  ".macro FQ_WAIT n\n"                                                                                             \
  "  .if (\\n) <= 0\n    s_waitcnt lgkmcnt(0)\n"                                                                   \
  "  .elseif (\\n) == 1\n    s_waitcnt lgkmcnt(1)\n"                                                               \
  "  .elseif (\\n) == 2\n    s_waitcnt lgkmcnt(2)\n"                                                               \
  "  .elseif (\\n) == 3\n    s_waitcnt lgkmcnt(3)\n"                                                               \
  "  .elseif (\\n) == 4\n    s_waitcnt lgkmcnt(4)\n"                                                               \
  "  .elseif (\\n) == 5\n    s_waitcnt lgkmcnt(5)\n"                                                               \
  "  .elseif (\\n) == 6\n    s_waitcnt lgkmcnt(6)\n"                                                               \
  "  .elseif (\\n) == 7\n    s_waitcnt lgkmcnt(7)\n"                                                               \
  "  .elseif (\\n) == 8\n    s_waitcnt lgkmcnt(8)\n"                                                               \
  "  .elseif (\\n) == 9\n    s_waitcnt lgkmcnt(9)\n"                                                               \
  "  .elseif (\\n) == 10\n    s_waitcnt lgkmcnt(10)\n"                                                             \
  "  .elseif (\\n) == 11\n    s_waitcnt lgkmcnt(11)\n"          \
  "  .elseif (\\n) == 12\n    s_waitcnt lgkmcnt(12)\n"          \
  "  .elseif (\\n) == 13\n    s_waitcnt lgkmcnt(13)\n"          \
  "  .elseif (\\n) == 14\n    s_waitcnt lgkmcnt(14)\n"          \
  "  .else\n    s_waitcnt lgkmcnt(15)\n"          \
  "  .endif\n"                                                                                                     \
  ".endm\n"                                                                                                        \
  /* row read of stream position p (k-step p/2) from base, address formed in tmp */                              \
  ".macro FQ_RX p, base, tmp\n"                                                                                    \
  "  .if (((\\p) >> 1) & 7) == 0\n"                                                                                \
  "    ds_read_b128 v[216 + ((\\p) %% 10) * 4 : 219 + ((\\p) %% 10) * 4], \\base offset:((((\\p) >> 4) & 1) * 256)\n" \
  "  .else\n"                                                                                                      \
  "    v_xor_b32 \\tmp, 32 * (((\\p) >> 1) & 7), \\base\n"                                                        \
  "    ds_read_b128 v[216 + ((\\p) %% 10) * 4 : 219 + ((\\p) %% 10) * 4], \\tmp offset:((((\\p) >> 4) & 1) * 256)\n"  \
  "  .endif\n"                                                                                                     \
  ".endm\n"                                                                                                        \
  /* the two transposed reads of block db, chunk offset co, into the buffer of stream position p */              \
  ".macro FQ_TX db, co, p\n"                                                                                       \
  "  .if ((\\db) & 3) == 0\n"                                                                                      \
  "    ds_read_b64_tr_b16 v[216 + ((\\p) %% 10) * 4 : 217 + ((\\p) %% 10) * 4], %[t1] "                            \
  "offset:((\\co) + ((\\db) >> 2) * 256)\n"                                                                        \
  "    ds_read_b64_tr_b16 v[218 + ((\\p) %% 10) * 4 : 219 + ((\\p) %% 10) * 4], %[t2] "                            \
  "offset:((\\co) + ((\\db) >> 2) * 256)\n"                                                                        \
  "  .else\n"                                                                                                      \
  "    v_xor_b32 v214, 64 * ((\\db) & 3), %[t1]\n"                                                                \
  "    v_xor_b32 v215, 64 * ((\\db) & 3), %[t2]\n"                                                                \
  "    ds_read_b64_tr_b16 v[216 + ((\\p) %% 10) * 4 : 217 + ((\\p) %% 10) * 4], v214 "                             \
  "offset:((\\co) + ((\\db) >> 2) * 256)\n"                                                                        \
  "    ds_read_b64_tr_b16 v[218 + ((\\p) %% 10) * 4 : 219 + ((\\p) %% 10) * 4], v215 "                             \
  "offset:((\\co) + ((\\db) >> 2) * 256)\n"                                                                        \
  "  .endif\n"                                                                                                     \
  ".endm\n"                                                                                                        \
  /* a stream: nsx S/dP fragments (one LDS instruction each), then, if dq, 2 NB dQ */                            \
  /* fragments (blocks of the first 16 keys, then of the second; two instructions each) */                       \
  ".macro FQ_RD p, nsx, dq\n"                                                                                      \
  "  .if (\\p) < (\\nsx)\n"                                                                                        \
  "    .if ((\\p) & 1) == 0\n"                                                                                     \
  "      FQ_RX (\\p), %[rb], v214\n"                                                                               \
  "    .else\n"                                                                                                    \
  "      FQ_RX (\\p), %[rv], v215\n"                                                                               \
  "    .endif\n"                                                                                                   \
  "  .elseif (\\dq) && ((\\p) < (\\nsx) + %[nb])\n"                                                                \
  "    FQ_TX ((\\p) - (\\nsx)), 0, (\\p)\n"                                                                        \
  "  .elseif (\\dq) && ((\\p) < (\\nsx) + 2 * %[nb])\n"                                                            \
  "    FQ_TX ((\\p) - (\\nsx) - %[nb]), 8192, (\\p)\n"                                                             \
  "  .endif\n"                                                                                                     \
  ".endm\n"                                                                                                        \
  /* wait for the fragments before position a with those before b issued */                                     \
  ".macro FQ_WT2 a, b, nsx\n"                                                                                      \
  "  .if (\\b) <= (\\nsx)\n"                                                                                       \
  "    FQ_WAIT ((\\b) - (\\a))\n"                                                                                  \
  "  .elseif (\\a) >= (\\nsx)\n"                                                                                   \
  "    FQ_WAIT (2 * ((\\b) - (\\a)))\n"                                                                            \
  "  .else\n"                                                                                                      \
  "    FQ_WAIT (((\\nsx) - (\\a)) + 2 * ((\\b) - (\\nsx)))\n"                                                      \
  "  .endif\n"                                                                                                     \
  ".endm\n"                                                                                                        \
  ".macro FQ_WT m, nsx, dq\n"                                                                                      \
  "  .if (\\m) + 10 <= (\\nsx) + 2 * %[nb] * (\\dq)\n"                                                              \
  "    FQ_WT2 ((\\m) + 1), ((\\m) + 10), (\\nsx)\n"                                                                 \
  "  .else\n"                                                                                                      \
  "    FQ_WT2 ((\\m) + 1), ((\\nsx) + 2 * %[nb] * (\\dq)), (\\nsx)\n"                                              \
  "  .endif\n"                                                                                                     \
  ".endm\n"                                                                                                        \
  /* next tile's copy, load n (0..7 K rows, 8..15 V rows) of this wave's share: global */                      \
  /* offset (co + 1024 i) ^ (k_i << 4), k_i = 8 (i & 1) + i / 2, into LDS at M0 */                             \
  ".macro FQ_CP n\n"                                                                                              \
  "  v_add_u32 v214, ((\\n) & 7) * 1024, %[co]\n"                                                                \
  "  .if ((((\\n) & 1) << 3) | (((\\n) & 7) >> 1)) != 0\n"                                                       \
  "    v_xor_b32 v214, ((((\\n) & 1) << 3) | (((\\n) & 7) >> 1)) << 4, v214\n"                                      \
  "  .endif\n"                                                                                                     \
  "  .if ((\\n) >> 3) == 0\n"                                                                                     \
  "    s_add_u32 m0, %[lk], ((\\n) & 7) * 1024\n"                                                                 \
  "  .else\n"                                                                                                      \
  "    s_add_u32 m0, %[lv], ((\\n) & 7) * 1024\n"                                                                 \
  "  .endif\n"                                                                                                     \
  "  s_mov_b64 exec, %[cx]\n"                                                                                      \
  "  .if ((\\n) >> 3) == 0\n"                                                                                     \
  "    global_load_lds_dwordx4 v214, %[kg]\n"                                                                      \
  "  .else\n"                                                                                                      \
  "    global_load_lds_dwordx4 v214, %[vg]\n"                                                                      \
  "  .endif\n"                                                                                                     \
  "  s_mov_b64 exec, -1\n"                                                                                         \
  ".endm\n"                                                                                                        \
  /* after the MFMA at stream position m: copy load m / cps when m mod cps = cps - 1 */                           \
  ".macro FQ_CPAT m, cps\n"                                                                                        \
  "  .if %[cpon] && (((\\m) %% (\\cps)) == ((\\cps) - 1)) && (((\\m) / (\\cps)) < 16)\n"                         \
  "    FQ_CP ((\\m) / (\\cps))\n"                                                                                  \
  "  .endif\n"                                                                                                     \
  ".endm\n"                                                                                                        \
  /* dS work in the shadow of S/dP MFMA m: element m's fma and subtraction, element */                           \
  /* m-1's exp, element m-2's product, pair (m-3)/2's pack */                                                    \
  ".macro FQ_V m\n"                                                                                                \
  "  .if (\\m) < 16\n"                                                                                             \
  "    v_fma_f32 v[%[sp] + (\\m)], v[%[sp] + (\\m)], %[c], %[nl]\n"                                                \
  "    v_sub_f32 v[%[sp] + 16 + (\\m)], v[%[sp] + 16 + (\\m)], %[dl]\n"                                            \
  "  .endif\n"                                                                                                     \
  "  .if ((\\m) >= 1) && ((\\m) <= 16)\n"                                                                          \
  "    v_exp_f32 v[%[sp] + (\\m) - 1], v[%[sp] + (\\m) - 1]\n"                                                     \
  "  .endif\n"                                                                                                     \
  "  .if ((\\m) >= 2) && ((\\m) <= 17)\n"                                                                          \
  "    v_mul_f32 v[%[sp] + (\\m) - 2], v[%[sp] + (\\m) - 2], v[%[sp] + 16 + (\\m) - 2]\n"                          \
  "  .endif\n"                                                                                                     \
  "  .if ((\\m) >= 3) && ((\\m) <= 17) && (((\\m) & 1) == 1)\n"                                                     \
  "    v_cvt_pk_bf16_f32 v[206 + ((\\m) - 3) / 2], v[%[sp] + (\\m) - 3], v[%[sp] + (\\m) - 2]\n"                    \
  "  .endif\n"                                                                                                     \
  ".endm\n"                                                                                                        \
  /* S/dP MFMA m (S for even m, dP for odd, k-step m/2), then the read 10 ahead and, if v, dS work */             \
  ".macro FQ_SM m, nsx, dq, v, cps\n"                                                                                   \
  "  .if (\\m) < (\\nsx)\n"                                                                                        \
  "    FQ_WT (\\m), (\\nsx), (\\dq)\n"                                                                             \
  "    .if ((\\m) >> 1) == 0\n"                                                                                    \
  "      v_mfma_f32_32x32x16_bf16 v[%[sn] + ((\\m) & 1) * 16 : %[sn] + ((\\m) & 1) * 16 + 15], "                  \
  "v[216 + ((\\m) %% 10) * 4 : 219 + ((\\m) %% 10) * 4], "                                                          \
  "a[((\\m) & 1) * 64 + ((\\m) >> 1) * 4 : ((\\m) & 1) * 64 + ((\\m) >> 1) * 4 + 3], 0\n"                          \
  "    .else\n"                                                                                                    \
  "      v_mfma_f32_32x32x16_bf16 v[%[sn] + ((\\m) & 1) * 16 : %[sn] + ((\\m) & 1) * 16 + 15], "                  \
  "v[216 + ((\\m) %% 10) * 4 : 219 + ((\\m) %% 10) * 4], "                                                          \
  "a[((\\m) & 1) * 64 + ((\\m) >> 1) * 4 : ((\\m) & 1) * 64 + ((\\m) >> 1) * 4 + 3], "                            \
  "v[%[sn] + ((\\m) & 1) * 16 : %[sn] + ((\\m) & 1) * 16 + 15]\n"                                                 \
  "    .endif\n"                                                                                                   \
  "    FQ_RD ((\\m) + 10), (\\nsx), (\\dq)\n"                                                                       \
  "    .if (\\v)\n"                                                                                                \
  "      FQ_V (\\m)\n"                                                                                             \
  "    .endif\n"                                                                                                   \
  "    FQ_CPAT (\\m), (\\cps)\n"                                                                                  \
  "  .endif\n"                                                                                                     \
  ".endm\n"                                                                                                        \
  /* dQ MFMA of dQ fragment f (stream position nsx + f) into block a[128 + 16 db], B operand b */                \
  ".macro FQ_DM f, lim, db, b, nsx, cps\n"                                                                              \
  "  .if (\\f) < (\\lim)\n"                                                                                        \
  "    FQ_WT ((\\nsx) + (\\f)), (\\nsx), 1\n"                                                                      \
  "    v_mfma_f32_32x32x16_bf16 a[128 + 16 * (\\db) : 143 + 16 * (\\db)], "                                        \
  "v[216 + (((\\nsx) + (\\f)) %% 10) * 4 : 219 + (((\\nsx) + (\\f)) %% 10) * 4], \\b, "                              \
  "a[128 + 16 * (\\db) : 143 + 16 * (\\db)]\n"                                                                     \
  "    FQ_RD ((\\nsx) + (\\f) + 10), (\\nsx), 1\n"                                                                  \
  "    FQ_CPAT ((\\nsx) + (\\f)), (\\cps)\n"                                                                     \
  "  .endif\n"                                                                                                     \
  ".endm\n"                                                                                                        \
  ".macro FQ_SMS nsx, dq, v, cps\n"                                                                                     \
  "  FQ_SM 0, \\nsx, \\dq, \\v, \\cps\n  FQ_SM 1, \\nsx, \\dq, \\v, \\cps\n  FQ_SM 2, \\nsx, \\dq, \\v, \\cps\n"                          \
  "  FQ_SM 3, \\nsx, \\dq, \\v, \\cps\n  FQ_SM 4, \\nsx, \\dq, \\v, \\cps\n  FQ_SM 5, \\nsx, \\dq, \\v, \\cps\n"                          \
  "  FQ_SM 6, \\nsx, \\dq, \\v, \\cps\n  FQ_SM 7, \\nsx, \\dq, \\v, \\cps\n  FQ_SM 8, \\nsx, \\dq, \\v, \\cps\n"                          \
  "  FQ_SM 9, \\nsx, \\dq, \\v, \\cps\n  FQ_SM 10, \\nsx, \\dq, \\v, \\cps\n  FQ_SM 11, \\nsx, \\dq, \\v, \\cps\n"                        \
  "  FQ_SM 12, \\nsx, \\dq, \\v, \\cps\n  FQ_SM 13, \\nsx, \\dq, \\v, \\cps\n  FQ_SM 14, \\nsx, \\dq, \\v, \\cps\n"                       \
  "  FQ_SM 15, \\nsx, \\dq, \\v, \\cps\n  FQ_SM 16, \\nsx, \\dq, \\v, \\cps\n  FQ_SM 17, \\nsx, \\dq, \\v, \\cps\n"                       \
  "  FQ_SM 18, \\nsx, \\dq, \\v, \\cps\n  FQ_SM 19, \\nsx, \\dq, \\v, \\cps\n  FQ_SM 20, \\nsx, \\dq, \\v, \\cps\n"                       \
  "  FQ_SM 21, \\nsx, \\dq, \\v, \\cps\n  FQ_SM 22, \\nsx, \\dq, \\v, \\cps\n  FQ_SM 23, \\nsx, \\dq, \\v, \\cps\n"                       \
  "  FQ_SM 24, \\nsx, \\dq, \\v, \\cps\n  FQ_SM 25, \\nsx, \\dq, \\v, \\cps\n  FQ_SM 26, \\nsx, \\dq, \\v, \\cps\n"                       \
  "  FQ_SM 27, \\nsx, \\dq, \\v, \\cps\n  FQ_SM 28, \\nsx, \\dq, \\v, \\cps\n  FQ_SM 29, \\nsx, \\dq, \\v, \\cps\n"                       \
  "  FQ_SM 30, \\nsx, \\dq, \\v, \\cps\n  FQ_SM 31, \\nsx, \\dq, \\v, \\cps\n"                                                    \
  ".endm\n"                                                                                                        \
  ".macro FQ_DMS b0, b1, nsx, cps\n"                                                                                    \
  "  FQ_DM 0, %[nb], 0, \\b0, \\nsx, \\cps\n  FQ_DM 1, %[nb], 1, \\b0, \\nsx, \\cps\n  FQ_DM 2, %[nb], 2, \\b0, \\nsx, \\cps\n"            \
  "  FQ_DM 3, %[nb], 3, \\b0, \\nsx, \\cps\n  FQ_DM 4, %[nb], 4, \\b0, \\nsx, \\cps\n  FQ_DM 5, %[nb], 5, \\b0, \\nsx, \\cps\n"            \
  "  FQ_DM 6, %[nb], 6, \\b0, \\nsx, \\cps\n  FQ_DM 7, %[nb], 7, \\b0, \\nsx, \\cps\n"                                             \
  "  FQ_DM %[nb]+0, 2*%[nb], 0, \\b1, \\nsx, \\cps\n  FQ_DM %[nb]+1, 2*%[nb], 1, \\b1, \\nsx, \\cps\n"                              \
  "  FQ_DM %[nb]+2, 2*%[nb], 2, \\b1, \\nsx, \\cps\n  FQ_DM %[nb]+3, 2*%[nb], 3, \\b1, \\nsx, \\cps\n"                              \
  "  FQ_DM %[nb]+4, 2*%[nb], 4, \\b1, \\nsx, \\cps\n  FQ_DM %[nb]+5, 2*%[nb], 5, \\b1, \\nsx, \\cps\n"                              \
  "  FQ_DM %[nb]+6, 2*%[nb], 6, \\b1, \\nsx, \\cps\n  FQ_DM %[nb]+7, 2*%[nb], 7, \\b1, \\nsx, \\cps\n"                              \
  ".endm\n"                                                                                                        \
  "s_cmp_eq_u32 %[mode], 2\n"                                                                                      \
  "s_cbranch_scc1 L_full_%=\n"                                                                                     \
  "s_cmp_eq_u32 %[mode], 1\n"                                                                                      \
  "s_cbranch_scc1 L_first_%=\n"                                                                                    \
  "s_cmp_eq_u32 %[mode], 3\n"                                                                                      \
  "s_cbranch_scc1 L_dq_%=\n"                                                                                       \
  ".if %[cpon]\n"                                                                                                 \
  "  FQ_CP 0\n  FQ_CP 1\n  FQ_CP 2\n  FQ_CP 3\n  FQ_CP 4\n  FQ_CP 5\n  FQ_CP 6\n  FQ_CP 7\n"                        \
  "  FQ_CP 8\n  FQ_CP 9\n  FQ_CP 10\n  FQ_CP 11\n  FQ_CP 12\n  FQ_CP 13\n  FQ_CP 14\n  FQ_CP 15\n"                  \
  ".endif\n"                                                                                                       \
  "s_branch L_end_%=\n"                                                                                            \
  "L_full_%=:\n"                                                                                                   \
  "FQ_RD 0, 2 * %[ns], 1\nFQ_RD 1, 2 * %[ns], 1\nFQ_RD 2, 2 * %[ns], 1\nFQ_RD 3, 2 * %[ns], 1\nFQ_RD 4, 2 * %[ns], 1\n"      \
  "FQ_RD 5, 2 * %[ns], 1\nFQ_RD 6, 2 * %[ns], 1\nFQ_RD 7, 2 * %[ns], 1\nFQ_RD 8, 2 * %[ns], 1\nFQ_RD 9, 2 * %[ns], 1\n"      \
  "FQ_SMS (2 * %[ns]), 1, 1, 1\n"                                                                                  \
  "FQ_DMS v[206:209], v[210:213], (2 * %[ns]), 1\n"                                                                \
  "s_branch L_end_%=\n"                                                                                            \
  "L_first_%=:\n"                                                                                                  \
  "FQ_RD 0, 2 * %[ns], 0\nFQ_RD 1, 2 * %[ns], 0\nFQ_RD 2, 2 * %[ns], 0\nFQ_RD 3, 2 * %[ns], 0\nFQ_RD 4, 2 * %[ns], 0\n"      \
  "FQ_RD 5, 2 * %[ns], 0\nFQ_RD 6, 2 * %[ns], 0\nFQ_RD 7, 2 * %[ns], 0\nFQ_RD 8, 2 * %[ns], 0\nFQ_RD 9, 2 * %[ns], 0\n"      \
  "FQ_SMS (2 * %[ns]), 0, 0, 2\n"                                                                                  \
  "s_branch L_end_%=\n"                                                                                            \
  "L_dq_%=:\n"                                                                                                     \
  "FQ_RD 0, 0, 1\nFQ_RD 1, 0, 1\nFQ_RD 2, 0, 1\nFQ_RD 3, 0, 1\nFQ_RD 4, 0, 1\n"      \
  "FQ_RD 5, 0, 1\nFQ_RD 6, 0, 1\nFQ_RD 7, 0, 1\nFQ_RD 8, 0, 1\nFQ_RD 9, 0, 1\n"      \
  "FQ_DMS %[d0], %[d1], 0, 1\n"                                                                                    \
  "L_end_%=:\n"                                                                                                    \
  "s_nop 7\ns_nop 7\ns_nop 7\n" /* MFMA results may be read by vector instructions next */                         \
  ".purgem FQ_WAIT\n.purgem FQ_RX\n.purgem FQ_TX\n.purgem FQ_RD\n.purgem FQ_WT2\n.purgem FQ_WT\n"                \
  ".purgem FQ_V\n.purgem FQ_SM\n.purgem FQ_DM\n.purgem FQ_SMS\n.purgem FQ_DMS\n.purgem FQ_CP\n.purgem FQ_CPAT\n"

#define DQ_STEP_INPUTS                                                                                                 \
  [ns] "i"(NS), [nb] "i"(NB), [cpon] "i"(NS == 16 ? 1 : 0), [mode] "s"(mode), [rb] "v"(rb), [rv] "v"(rv),         \
      [t1] "v"(t1), [t2] "v"(t2), [c] "v"(c), [kg] "s"(cp.kg), [vg] "s"(cp.vg), [lk] "s"(cp.lk), [lv] "s"(cp.lv),   \
      [cx] "s"(cp.exec), [co] "v"(cp.co),                                                                       \
      [nl] "v"(nl), [dl] "v"(dl), [d0] "v"(d0), [d1] "v"(d1), "{a[0:15]}"(qo[0]), "{a[16:31]}"(qo[1]),             \
      "{a[32:47]}"(qo[2]), "{a[48:63]}"(qo[3]), "{a[64:79]}"(qo[4]), "{a[80:95]}"(qo[5]), "{a[96:111]}"(qo[6]),    \
      "{a[112:127]}"(qo[7])
#define DQ_STEP_ACC                                                                                          \
  "+{a[128:143]}"(q[0]), "+{a[144:159]}"(q[1]), "+{a[160:175]}"(q[2]), "+{a[176:191]}"(q[3]),               \
      "+{a[192:207]}"(q[4]), "+{a[208:223]}"(q[5]), "+{a[224:239]}"(q[6]), "+{a[240:255]}"(q[7])
#define DQ_STEP_CLOBBERS                                                                                          \
  "memory", "scc", "m0", "exec", "v206", "v207", "v208", "v209", "v210", "v211", "v212", "v213", "v214", "v215", \
      "v216", "v217", "v218", "v219", "v220", "v221", "v222", "v223", "v224", "v225", "v226", "v227", "v228", \
      "v229", "v230", "v231", "v232", "v233", "v234", "v235", "v236", "v237", "v238", "v239", "v240", "v241", \
      "v242", "v243", "v244", "v245", "v246", "v247", "v248", "v249", "v250", "v251", "v252", "v253", "v254", \
      "v255"

// The next tile's copy as the step issues it: this wave's loads i = 0..7
// of K rows then of V rows, from global tile bases kg, vg (whole tiles) to
// LDS lk, lv (this wave's share of the slots) + 1024 i, at lane offsets
// (co + 1024 i) ^ (k_i << 4) with k_i = 8 (i mod 2) + i / 2 -- the
// swizzled row copy's offsets, which differ from one load to the next only
// in those bits.  exec = 0 leaves the loads out.
struct DqStepCopy {
  uint64_t kg, vg;
  uint32_t lk, lv;
  uint64_t exec;
  int co;
};

// PAR 0: the new S/dP go to v[142:173] (set A), the previous ones are in
// v[174:205] (set B); PAR 1 the other way round.  Both sets are in-out
// operands in every mode, so that they too stay in place.
template <int NS, int NB, int PAR>
__device__ __forceinline__ void dq_step(int mode, int rb, int rv, int t1, int t2, float c, float nl, float dl,
                                        const bf16x8& d0, const bf16x8& d1, const DqStepCopy& cp,
                                        const f32x16 (&qo)[8], f32x16& sa, f32x16& da, f32x16& sb, f32x16& db,
                                        f32x16 (&q)[8]) {
  static_assert(NS >= 9 && NS <= 16 && NB >= 4 && NB <= 8, "shape");  // in-block dS ends at MFMA 17
  if constexpr (PAR == 0) {
    asm volatile(DQ_STEP_TEXT
                 : "+{v[142:157]}"(sa), "+{v[158:173]}"(da), "+{v[174:189]}"(sb), "+{v[190:205]}"(db), DQ_STEP_ACC
                 : [sn] "i"(142), [sp] "i"(174), DQ_STEP_INPUTS
                 : DQ_STEP_CLOBBERS);
  } else {
    asm volatile(DQ_STEP_TEXT
                 : "+{v[142:157]}"(sa), "+{v[158:173]}"(da), "+{v[174:189]}"(sb), "+{v[190:205]}"(db), DQ_STEP_ACC
                 : [sn] "i"(174), [sp] "i"(142), DQ_STEP_INPUTS
                 : DQ_STEP_CLOBBERS);
  }
}
#undef DQ_STEP_TEXT
#undef DQ_STEP_INPUTS
#undef DQ_STEP_ACC
#undef DQ_STEP_CLOBBERS

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
  // 256-wide rows run the pipelined asm step (one 32-key block per wave)
  constexpr bool kChains = DP == 256;
  static_assert(!kChains || (KB == 1 && kTileBytes == 32768), "chain layout");
  // ring: with the pipelined step K tiles j-1, j and V tile j are read while
  // tile j+1 loads, in three K slots (tile t in slot t mod 3) and two V
  // slots (slot 3 + t mod 2), 160 KB; otherwise K0 K1 V0 V1
  constexpr int kSlots = kChains ? 5 : 4;
  __shared__ __attribute__((aligned(1024))) char smem_raw[kSlots * kTileBytes];
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
  auto copy_tile = [&](int t, lds_char* kd, lds_char* vd) {
    const int row0 = t * kKeyTile;
    if (row0 + kKeyTile <= N) {
      cp.copy_at(K, (uint32_t)row0 * (D * 2), kd);
      cp.copy_at(V, (uint32_t)row0 * (D * 2), vd);
    } else {
      cp.copy_clamped(K, N, row0, kd);
      cp.copy_clamped(V, N, row0, vd);
    }
  };
  if constexpr (kChains)
    copy_tile(0, smem, smem + 3 * kTileBytes);
  else
    copy_tile(0, kbuf[0], vbuf[0]);

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

  if constexpr (kChains) {
    auto kslot = [&](int k) { return (int)(uint32_t)(uintptr_t)(smem + k * kTileBytes); };
    const float nl = -lse2;
    f32x16 sA, dA, sB, dB;  // S^T and dP^T of the last two tiles, tile t in set A for even t
    // dS^T of tile jt (this wave's last, after its step) from its S and dP,
    // masked where the tile needs it
    auto last_ds = [&](int jt, const f32x16& st, const f32x16& dt, bf16x8& d0, bf16x8& d1) {
      const bool masked = (CAUSAL && jt == wave_last) || (jt == n_ktiles_all - 1 && (N % kKeyTile) != 0);
      auto make_ds = [&](auto mask_tag) {
        constexpr bool kMask = decltype(mask_tag)::value;
        asm volatile("" ::: "memory");  // keeps the two variants from being merged into selects
        bf16x8 dsk[2];
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          bf16x2 pr[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float e[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              const int r = cc * 8 + 2 * i + t;
              float x = __builtin_fmaf(st[r], c, nl);
              if constexpr (kMask) {
                const int key = jt * kKeyTile + kpart * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
                bool keep = key < N;
                if constexpr (CAUSAL) keep = keep && key <= row;
                x = keep ? x : -__builtin_inff();
              }
              e[t] = fast_exp2(x) * (dt[r] - delta);
            }
            pr[i] = pack_bf16(e[0], e[1]);
          }
          dsk[cc] = join8(pr[0], pr[1], pr[2], pr[3]);
        }
        d0 = dsk[0];
        d1 = dsk[1];
      };
      if (masked)
        make_ds(std::true_type{});
      else
        make_ds(std::false_type{});
    };
    // this wave's copy offsets: the row copy's (co + 1024 i) ^ (k_i << 4) at D = 256
    constexpr bool kAsmCopy = D == 256;
    const int co = (wave * 16 + half) * 512 + ((l32 ^ (half << 2)) << 4);
    const uint32_t smem_u = (uint32_t)(uintptr_t)smem;
    int ks = 0;  // K slot of tile j
    // step j (j may be nt, a step with nothing to do): publishes tile j,
    // starts loading j+1, then S/dP of tile j with dS and dQ of tile j-1
    // (mode 1 at j = 0, 2 after); a wave one past its last tile finishes
    // that tile (mode 3)
    auto step = [&](int j, auto par_tag) {
      constexpr int P = decltype(par_tag)::value;  // j mod 2: S/dP of tile j go to set A (0) or B (1)
      wait_vmcnt<0>();
      __syncthreads();
      const int ks_next = ks == 2 ? 0 : ks + 1, ks_prev = ks == 0 ? 2 : ks - 1;
      DqStepCopy cpy = {0, 0, 0, 0, 0, co};
      if (j + 1 < nt) {
        const int vs_next = 3 + ((j + 1) & 1);
        if (kAsmCopy && (j + 2) * kKeyTile <= N) {  // a whole tile: the step issues it
          const size_t off = (size_t)(j + 1) * kKeyTile * D;
          cpy.kg = (uint64_t)(uintptr_t)(K + off);
          cpy.vg = (uint64_t)(uintptr_t)(V + off);
          cpy.lk = smem_u + ks_next * kTileBytes + wave * 8192;
          cpy.lv = smem_u + vs_next * kTileBytes + wave * 8192;
          cpy.exec = ~0ull;
        } else {
          copy_tile(j + 1, smem + ks_next * kTileBytes, smem + vs_next * kTileBytes);
        }
      }
      int mode = 0;
      bf16x8 d0 = {}, d1 = {};
      if (wave_active) {
        if (j <= wave_last) {
          mode = j == 0 ? 1 : 2;
        } else if (CAUSAL && j == wave_last + 1 && j < nt) {  // (unmasked, a wave's last tile is nt-1)
          mode = 3;
          if constexpr (P == 1)
            last_ds(j - 1, sA, dA, d0, d1);
          else
            last_ds(j - 1, sB, dB, d0, d1);
        }
      }
      const int kb = kslot(ks), vb = kslot(3 + P), pb = kslot(ks_prev);
      dq_step<kDSteps, kDBlocks, P>(__builtin_amdgcn_readfirstlane(mode), kb + rofs, vb + rofs, pb + tofs1,
                                    pb + tofs2, c, nl, delta, d0, d1, cpy, qo, sA, dA, sB, dB, dq);
      ks = ks_next;
    };
    for (int j = 0; j < nt; j += 2) {
      step(j, std::integral_constant<int, 0>{});
      step(j + 1, std::integral_constant<int, 1>{});
    }
    // the workgroup's last tile nt-1, if it is this wave's last, in its K
    // slot (nt-1) mod 3
    {
      int mode = 0;
      bf16x8 d0 = {}, d1 = {};
      if (wave_active && wave_last == nt - 1) {
        mode = 3;
        if ((nt - 1) & 1)
          last_ds(nt - 1, sB, dB, d0, d1);
        else
          last_ds(nt - 1, sA, dA, d0, d1);
      }
      const int pb = kslot((nt - 1) % 3);
      const DqStepCopy none = {0, 0, 0, 0, 0, co};
      dq_step<kDSteps, kDBlocks, 0>(__builtin_amdgcn_readfirstlane(mode), 0, 0, pb + tofs1, pb + tofs2, c, nl, delta,
                                    d0, d1, none, qo, sA, dA, sB, dB, dq);
    }
  } else {
    for (int j = 0; j < nt; ++j) {
      wait_vmcnt<0>();
      __syncthreads();
      if (j + 1 < nt) copy_tile(j + 1, kbuf[(j + 1) & 1], vbuf[(j + 1) & 1]);
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
  }

  if constexpr (DqCfg<D>::kSplit == 2) {
    // add the second key half's dQ partial sums (lane-major through LDS)
    float __attribute__((address_space(3)))* x =
        (float __attribute__((address_space(3)))*)smem + qblk * 64 * kDBlocks * 16 + lane;
    static_assert(kQBlocks * 64 * kDBlocks * 16 * 4 <= kSlots * kTileBytes, "merge buffer exceeds the ring");
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
