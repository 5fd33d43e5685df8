// fa_fwd_d128.hip -- square exact-attention forward at head dimension 128,
// bf16 in and out: one wave per SIMD, 64 query rows per wave, key loop in
// hand-scheduled gfx950 assembly.
//
// The method is the one of the generic forward kernel (fa_fwd_bf16.h) and of
// the pages ("Learning Metal with FlashAttention", section FlashAttention;
// "Flash Attention" page, kernel anatomy; metal-flash-attention README,
// "Quantifying performance", forward pseudocode): Q rows resident, K and V
// streamed in tiles of 64 keys through a 4-slot LDS ring, scores S^T = K Q^T
// on 32x32x16 bf16 MFMA, an online softmax in the exp2 domain against a
// running reference max, O^T += V^T P^T with P straight from the score
// accumulators, causal tiles above the diagonal never visited.
//
// What differs is the register plan and the schedule.  Each wave owns 64
// query rows (two 32-row blocks), so every K or V fragment read from LDS
// feeds two MFMAs: half the LDS bytes per FLOP of 32-row waves.  That needs
// more than the 256 architectural VGPRs: the O accumulators (128 registers)
// and the Q fragments (64) live in AGPRs, which the MFMA reads and writes
// directly; scores, P and fragment buffers are VGPRs.  The compiler does not
// keep such a split without copies, so the key loop is one block of inline
// assembly over fixed registers with the instruction order written out.
//
// The loop is a three-stage pipeline over key tiles.  Step p issues 72
// MFMAs -- the 32 P V products of tile p, 8 row-sum products over P of tile
// p+1 and the 32 score products of tile p+2 -- and between them, one small
// group of vector instructions per MFMA, the softmax of tile p+1: one
// exponential (an FMA to the exp2 domain against the running max and a
// v_exp_f32, in place) and, every other position, the bf16 pack of a pair
// into P.  No group is longer than an MFMA, so the vector work hides under
// the matrix work; a pack into P waits until the P V products of tile p have
// read the old P block it overwrites.  The row sums of the rounded P are
// MFMAs too, on the half-cost 16x16x32 shape (a 0/1 selector times P):
// plain VALU adds of the rounded values would need an unpack per value, and
// v_dot2 executes in the matrix pipe.  Ring refills go into MFMA positions
// with light vector work; a V refill reads the tile its K refill read one
// step before, so its address is that address moved to the V tensor.  After
// the MFMAs the tile's row sums are checked:
// a share above 2^16 (or not finite) takes an out-of-line path that
// recomputes the tile's scores, raises the running max, rescales
// O and l and redoes the exponentials.  The prologue (Q rows, scores of
// tiles 0 and 1, their masks, the running max, P of tile 0) and the
// epilogue (O / l, L) are ordinary C++.
//
// Register map inside the loop (v = VGPR, a = AGPR):
//   v[0:63], v[64:127]   score sets: tile q in set q mod 2, block (kb, qb)
//                        at set*64 + (kb*2 + qb)*16; exponentials in place
//   v[128:159]           P (bf16 pairs), (qb, kb, cc) at 128 + ((qb*2 + kb)*2 + cc)*4
//   v[160:175]           4 K-fragment buffers
//   v[176:191]           4 V-fragment buffers; temporaries of the masks and
//                        of the out-of-line path, which run while they idle
//   v192, v193; v194, v195  running max m; row sum l (per 32-row block)
//   v196, v197           this tile's row sums;  v198, v199  -m*c per block
//   v[200:207]           per-lane K fragment LDS addresses (one per k-step)
//   v[208:215]           per-lane V fragment LDS addresses (two per d block)
//   v[216:219]           per-lane global offsets of this lane's ring copies
//   v220, v221, v222     causal bound per block, half*4 (masks);  v223 -inf
//   v[224:227]           0/1 selector (the row-sum MFMAs' A operand)
//   a[0:127]             O^T accumulators, block (qb, db) at (qb*4 + db)*16
//   a[128:191]           Q^T fragments, (qb, ds) at 128 + (qb*8 + ds)*4
//   a[192:199]           row-sum accumulators, block qb at 192 + qb*4
//   s[70:71]             K of the head;  s74 position p;  s75 tiles;
//   s76 masked tiles R;  s77 first masked tile;  s78 last tile byte offset;
//   s79 scale*log2(e);  s80 LDS ring base + this wave's copy offset;  s81 wave;
//   s82..s85 scalar temporaries;  s86 p+2;  s87 2^16 (the bound on a
//   tile's exponentials);  s[88:89] this step's V refill address;
//   s[90:91], s94, s95 the next block's K, R and first masked tile;
//   s[92:93] the distance from the K tensor to the V tensor;  s97 the ring
//   slot the block starts in;  s[98:99] the address of the last K refill
#include "fa_device.h"
#include "fa_kernels.h"
#include "fa_sched.h"

namespace fa {
namespace d128 {

constexpr int D = 128;
constexpr int kWaves = 4;
constexpr int kRows = 64 * kWaves;       // query rows per workgroup
constexpr int kBlockN = 64;              // keys per tile
constexpr int kTileBytes = kBlockN * D * 2;
constexpr int kNB = 4;                   // ring slots per tensor
constexpr int kRingBytes = 2 * kNB * kTileBytes;
constexpr int kStageBytes = kWaves * 32 * D * 2;  // epilogue staging, 32 rows per wave
constexpr float kMaxFloor = 1.0e30f;     // the running max starts at -kMaxFloor

typedef __attribute__((ext_vector_type(32))) float f32x32;
typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;

// The key loop.  Macros of the GNU assembler syntax the LLVM integrated
// assembler accepts; register numbers are assembler expressions.  %= makes
// the labels unique per instance of the statement.  Pair n of a score tile
// (0..31, in the order the P blocks are freed) is key block kb = n/16,
// chunk cc = (n/8) mod 2, query block qb = (n/4) mod 2, word w = n mod 4:
// scores (kb, qb) elements cc*8 + 2w, +1.
#define FA_D128_LOOP_ASM R"ASM(
  // register of element e (0, 1) of pair n of score set c
  // exponential of element e of pair n of score set c, in place
  .macro FA_E n, e, c
    v_fma_f32 v[(\c)*64+((((\n)>>4)*2+(((\n)>>2)&1))*16)+((((\n)>>3)&1)*8)+((\n)&3)*2+(\e)], v[(\c)*64+((((\n)>>4)*2+(((\n)>>2)&1))*16)+((((\n)>>3)&1)*8)+((\n)&3)*2+(\e)], s79, v[198+(((\n)>>2)&1)]
    v_exp_f32 v[(\c)*64+((((\n)>>4)*2+(((\n)>>2)&1))*16)+((((\n)>>3)&1)*8)+((\n)&3)*2+(\e)], v[(\c)*64+((((\n)>>4)*2+(((\n)>>2)&1))*16)+((((\n)>>3)&1)*8)+((\n)&3)*2+(\e)]
  .endm
  // bf16 pack of pair n of score set c into P
  .macro FA_C n, c
    v_cvt_pk_bf16_f32 v[128+((((\n)>>2)&1)*2+((\n)>>4))*8+(((\n)>>3)&1)*4+((\n)&3)], v[(\c)*64+((((\n)>>4)*2+(((\n)>>2)&1))*16)+((((\n)>>3)&1)*8)+((\n)&3)*2], v[(\c)*64+((((\n)>>4)*2+(((\n)>>2)&1))*16)+((((\n)>>3)&1)*8)+((\n)&3)*2+1]
  .endm
  // vector work of MFMA position t of a step (softmax of score set c): the
  // exponential of one score, and the pack of pair n at position
  // max(2n+2, n+8) -- after both its exponentials, and after the P V
  // products of tile p have read the old P block it overwrites
  .macro FA_VPOS t, c
    .if (\t) < 64
      FA_E ((\t)>>1), ((\t)&1), \c
    .endif
    .if ((\t) >= 8) && ((\t) <= 14)
      FA_C ((\t)-8), \c
    .elseif ((\t) >= 16) && ((\t) <= 64) && (((\t)&1) == 0)
      FA_C (((\t)-2)>>1), \c
    .endif
  .endm
  // score MFMA k (group i = k/2: k-step ds = i/2, key block kb = i mod 2;
  // query block qb = k mod 2) into set n
  .macro FA_SMFMA k, n
    .if (((\k)>>2) == 0)
      v_mfma_f32_32x32x16_bf16 v[(\n)*64+((((\k)>>1)&1)*2+((\k)&1))*16:(\n)*64+((((\k)>>1)&1)*2+((\k)&1))*16+15], v[160+(((\k)>>1)&3)*4:163+(((\k)>>1)&3)*4], a[128+(((\k)&1)*8+((\k)>>2))*4:131+(((\k)&1)*8+((\k)>>2))*4], 0
    .else
      v_mfma_f32_32x32x16_bf16 v[(\n)*64+((((\k)>>1)&1)*2+((\k)&1))*16:(\n)*64+((((\k)>>1)&1)*2+((\k)&1))*16+15], v[160+(((\k)>>1)&3)*4:163+(((\k)>>1)&3)*4], a[128+(((\k)&1)*8+((\k)>>2))*4:131+(((\k)&1)*8+((\k)>>2))*4], v[(\n)*64+((((\k)>>1)&1)*2+((\k)&1))*16:(\n)*64+((((\k)>>1)&1)*2+((\k)&1))*16+15]
    .endif
  .endm
  // P V MFMA of V fragment j (16-key chunk kc = j/4, d block db = j mod 4)
  // for query block qb: O(qb, db) += V^T P^T
  .macro FA_PMFMA j, qb
    v_mfma_f32_32x32x16_bf16 a[(\qb)*64+((\j)&3)*16:(\qb)*64+((\j)&3)*16+15], v[176+((\j)&3)*4:179+((\j)&3)*4], v[128+(\qb)*16+((((\j)>>3)&1)*2+(((\j)>>2)&1))*4:131+(\qb)*16+((((\j)>>3)&1)*2+(((\j)>>2)&1))*4], a[(\qb)*64+((\j)&3)*16:(\qb)*64+((\j)&3)*16+15]
  .endm
  // row-sum MFMA of P block b = 2 kb + cc of query block qb (16 keys), on
  // the 16x16x32 shape: B = the P block as it stands (lane group g = lane/16
  // holds query (lane mod 16) + 16 (g mod 2), keys 8 (g/2) .. +7); A = the
  // 0/1 selector v[224:227] (row i sums the groups g with g mod 2 = (i/4)
  // mod 2), so each lane's four accumulators a[192 + qb*4 : +3] all get its
  // own query's sum over the block, accumulated over the 4 blocks
  .macro FA_RSMFMA b, qb
    .if (\b) == 0
      v_mfma_f32_16x16x32_bf16 a[192+(\qb)*4:195+(\qb)*4], v[224:227], v[128+(\qb)*16+(\b)*4:131+(\qb)*16+(\b)*4], 0
    .else
      v_mfma_f32_16x16x32_bf16 a[192+(\qb)*4:195+(\qb)*4], v[224:227], v[128+(\qb)*16+(\b)*4:131+(\qb)*16+(\b)*4], a[192+(\qb)*4:195+(\qb)*4]
    .endif
  .endm
  // K fragment i (k-step i/2, key block i mod 2) of ring slot b
  .macro FA_KREAD i, b
    ds_read_b128 v[160+((\i)&3)*4:163+((\i)&3)*4], v[200+((\i)>>1)] offset:(\b)*16384+((\i)&1)*8192
  .endm
  // V fragment j of ring slot b
  .macro FA_VREAD j, b
    ds_read_b64_tr_b16 v[176+((\j)&3)*4:177+((\j)&3)*4], v[208+((\j)&3)*2] offset:(\b)*16384+((((\j)>>3)&1)*32+(((\j)>>2)&1)*16)*256
    ds_read_b64_tr_b16 v[178+((\j)&3)*4:179+((\j)&3)*4], v[209+((\j)&3)*2] offset:(\b)*16384+((((\j)>>3)&1)*32+(((\j)>>2)&1)*16)*256
  .endm
  // byte offset of the tile at sequence position s82 -> s82: masked tiles
  // (positions < R) are tiles first_masked.., the rest tiles 0..; a ragged
  // last tile is loaded shifted back to end at key N
  .macro FA_TILE_BYTES
    s_add_u32 s83, s82, s77
    s_sub_u32 s84, s82, s76
    s_cmp_lt_u32 s82, s76
    s_cselect_b32 s82, s83, s84
    s_lshl_b32 s82, s82, 14
    s_min_u32 s82, s82, s78
  .endm
  // ring refill piece r of step p (slot j = p mod 4): 0 = address of V(p+3),
  // which is the address K(p+3) was copied from one step before moved by
  // the distance between the K and V tensors (s[92:93]: heads sit at the
  // same offset in both), and M0 of its first copy; 1..4 = its four copies
  // into V slot (j+3) mod 4; 5 = address of K(p+4) into s[98:99]; 6..9 =
  // its copies into slot j.  M0 is written one piece before the copy that
  // reads it.  A position past the block's last tile is the next block's
  // tile (position minus nt), computed out of line; the last block's "next
  // block" is itself, so every copy reads a valid tile (those past the end
  // land in ring slots no step reads again).
  .macro FA_REFILL r, j, uid
    .if (\r) == 0
      s_add_u32 s88, s98, s92
      s_addc_u32 s89, s99, s93
      s_add_u32 m0, s80, 65536+((((\j)+3)&3)*16384)
    .elseif (\r) <= 3
      global_load_lds_dwordx4 v[216+(\r)-1], s[88:89]
      s_add_u32 m0, s80, 65536+((((\j)+3)&3)*16384)+(\r)*1024
    .elseif (\r) == 4
      global_load_lds_dwordx4 v219, s[88:89]
      s_add_u32 m0, s80, (\j)*16384
    .elseif (\r) == 5
      s_add_u32 s82, s74, 4
      s_cmp_lt_u32 s82, s75
      s_cbranch_scc0 L_kn_\j\()_\uid
      FA_TILE_BYTES
      s_add_u32 s98, s70, s82
      s_addc_u32 s99, s71, 0
    L_kr_\j\()_\uid:
    .elseif (\r) <= 8
      global_load_lds_dwordx4 v[216+(\r)-6], s[98:99]
      s_add_u32 m0, s80, (\j)*16384+((\r)-5)*1024
    .else
      global_load_lds_dwordx4 v219, s[98:99]
    .endif
  .endm
  // out of line: the K address of the next block's tile at position
  // s82 - nt (its masked tiles first, as for every block)
  .macro FA_RNEXT j, uid
  L_kn_\j\()_\uid:
    s_sub_u32 s82, s82, s75
    s_add_u32 s83, s82, s95
    s_sub_u32 s84, s82, s94
    s_cmp_lt_u32 s82, s94
    s_cselect_b32 s82, s83, s84
    s_lshl_b32 s82, s82, 14
    s_min_u32 s82, s82, s78
    s_add_u32 s98, s90, s82
    s_addc_u32 s99, s91, 0
    s_branch L_kr_\j\()_\uid
  .endm
  // the score-half MFMA at step position t (32..71): row-sum MFMAs at 32..35,
  // 42, 50, 58, 66 (after the packs they read), score MFMAs k = 0..31 at the
  // others; K fragments waited for before each even k and read three ahead
  .macro FA_SK k, j
    .if ((\k)&1) == 0
      .if ((\k)>>1) <= 13
        s_waitcnt lgkmcnt(2)
      .elseif ((\k)>>1) == 14
        s_waitcnt lgkmcnt(1)
      .else
        s_waitcnt lgkmcnt(2)
      .endif
    .endif
    FA_SMFMA \k, ((\j)&1)
    .if (((\k)&1) == 1) && (((\k)>>1) <= 12)
      FA_KREAD (((\k)>>1)+3), (((\j)+2)&3)
    .endif
  .endm
  .macro FA_SPOS t, j
    .if (\t) <= 35
      FA_RSMFMA (((\t)-32)>>1), (((\t)-32)&1)
    .elseif (\t) <= 41
      FA_SK ((\t)-36), \j
    .elseif (\t) == 42
      FA_RSMFMA 2, 0
    .elseif (\t) <= 49
      FA_SK ((\t)-37), \j
    .elseif (\t) == 50
      FA_RSMFMA 2, 1
    .elseif (\t) <= 57
      FA_SK ((\t)-38), \j
    .elseif (\t) == 58
      FA_RSMFMA 3, 0
    .elseif (\t) <= 65
      FA_SK ((\t)-39), \j
    .elseif (\t) == 66
      FA_RSMFMA 3, 1
    .else
      FA_SK ((\t)-40), \j
    .endif
  .endm
  // -inf where a key of the tile at position p + q (score set c) is
  // invisible: above the causal bound, past N, or (ragged last tile, loaded
  // shifted back) below the tile's first new key.  Temporaries: the V
  // fragment buffers (idle at the end of a step).
  .macro FA_MASKSET c, q
    s_nop 7
    s_nop 7
    v_mov_b32 v223, 0xff800000
    s_add_u32 s82, s74, s77
    s_add_u32 s82, s82, \q
    s_lshl_b32 s83, s82, 6
    s_lshr_b32 s84, s78, 8
    s_min_u32 s84, s83, s84
    v_add_u32 v228, s84, v222
    v_sub_u32 v229, s83, v228
    v_sub_u32 v230, v220, v228
    v_sub_u32 v231, v221, v228
    v_sub_u32 v230, v230, v229
    v_max_i32 v230, 0, v230
    v_sub_u32 v231, v231, v229
    v_max_i32 v231, 0, v231
    .irp kb, 0, 1
      .irp r, 0,1,2,3,4,5,6,7,8,9,10,11,12,13,14,15
        v_sub_u32 v232, (\kb)*32+((\r)>>2)*8+((\r)&3), v229
        v_cmp_gt_u32 vcc, v230, v232
        v_cndmask_b32 v[(\c)*64+(\kb)*32+(\r)], v223, v[(\c)*64+(\kb)*32+(\r)], vcc
        v_cmp_gt_u32 vcc, v231, v232
        v_cndmask_b32 v[(\c)*64+(\kb)*32+16+(\r)], v223, v[(\c)*64+(\kb)*32+16+(\r)], vcc
      .endr
    .endr
  .endm

  // ---- step p (s74), unrolled over the ring: j = p mod 4.  Scores of tile
  // p+1 are in set (j+1) mod 2 (masked), P of tile p in v[128:159].
  .macro FA_STEP j, uid
    s_waitcnt vmcnt(8)
    s_barrier
    s_add_u32 s86, s74, 2
    // a causal diagonal tile past this wave's rows (p < R, p > wave): its P
    // is zero, the variant without P V products
    s_cmp_lt_u32 s74, s76
    s_cbranch_scc1 L_pvd_\j\()_\uid
  L_pvfull_\j\()_\uid:
    // P V half: positions 0..31 (each position's LDS reads go out before its
    // vector work, which then covers part of their latency)
    .irp t, 0,1,2,3,4,5,6,7,8,9,10,11,12,13,14,15,16,17,18,19,20,21,22,23,24,25,26,27,28,29,30,31
      .if ((\t)&1) == 0
        .if ((\t)>>1) <= 13
          s_waitcnt lgkmcnt(4)
        .elseif ((\t)>>1) == 14
          s_waitcnt lgkmcnt(3)
        .else
          s_waitcnt lgkmcnt(2)
        .endif
      .endif
      FA_PMFMA ((\t)>>1), ((\t)&1)
      .if (((\t)&1) == 1) && (((\t)>>1) <= 12)
        FA_VREAD (((\t)>>1)+3), (\j)
      .endif
      .if ((\t) == 27) || ((\t) == 29) || ((\t) == 31)
        FA_KREAD (((\t)-27)>>1), (((\j)+2)&3)
      .endif
      FA_VPOS \t, (((\j)+1)&1)
    .endr
  L_pvret_\j\()_\uid:
    // score half: positions 32..71 (32 score MFMAs of tile p+2, 8 row sums);
    // past the block's last tile (p+2 >= nt) the variant without scores
    s_cmp_ge_u32 s86, s75
    s_cbranch_scc1 L_ns_\j\()_\uid
    s_cmp_lt_u32 s86, s76
    s_cbranch_scc1 L_diag_\j\()_\uid
  L_sfull_\j\()_\uid:
    .irp t, 32,33,34,35,36,37,38,39,40,41,42,43,44,45,46,47,48,49,50,51,52,53,54,55,56,57,58,59,60,61,62,63,64,65,66,67,68,69,70,71
      FA_SPOS \t, \j
      .if (\t) >= 62
        FA_REFILL ((\t)-62), \j, \uid
      .endif
      .if (\t) >= 69
        FA_VREAD ((\t)-69), (((\j)+1)&3)
      .endif
      FA_VPOS \t, (((\j)+1)&1)
    .endr
  L_nsret_\j\()_\uid:
    v_accvgpr_read_b32 v196, a192
    v_accvgpr_read_b32 v197, a196
    // tile p+1 exists (p+2 <= nt): check its exponentials against 2^16
    // (s87), add its row sums
    s_cmp_le_u32 s86, s75
    s_cbranch_scc0 L_nochk_\j\()_\uid
    v_cmp_nle_f32_e64 s[84:85], v196, s87
    v_cmp_nle_f32_e64 vcc, v197, s87
    s_or_b64 vcc, vcc, s[84:85]
    s_cbranch_vccnz L_rare_\j\()_\uid
  L_rret_\j\()_\uid:
    v_add_f32 v194, v194, v196
    v_add_f32 v195, v195, v197
  L_nochk_\j\()_\uid:
    // tile p+2 needs the elementwise mask if p+2 < R
    s_cmp_lt_u32 s86, s76
    s_cbranch_scc1 L_mask_\j\()_\uid
  L_mret_\j\()_\uid:
    s_add_u32 s74, s74, 1
    s_cmp_ge_u32 s74, s75
    s_cbranch_scc1 L_done_\uid
  .endm

  // ---- out of line: the scores of tile p+1 (set (j+1) mod 2) recomputed
  // from K slot (j+1) mod 4 and masked, the running max raised to their row
  // max where it grew by more than 2^8 (exp2 domain) with O and l rescaled,
  // exponentials, P and row sums redone.  Temporaries: the V fragment
  // buffers v[176:191].
  .macro FA_RARE j, uid
  L_rare_\j\()_\uid:
    .irp k, 0,1,2,3,4,5,6,7,8,9,10,11,12,13,14,15,16,17,18,19,20,21,22,23,24,25,26,27,28,29,30,31
      .if ((\k)&1) == 0
        FA_KREAD ((\k)>>1), (((\j)+1)&3)
        s_waitcnt lgkmcnt(0)
      .endif
      FA_SMFMA \k, (((\j)+1)&1)
    .endr
    s_add_u32 s82, s74, 1
    s_cmp_lt_u32 s82, s76
    s_cbranch_scc0 L_rnomask_\j\()_\uid
    FA_MASKSET (((\j)+1)&1), 1
  L_rnomask_\j\()_\uid:
    s_nop 7
    s_nop 7
    .irp qb, 0, 1
      v_max3_f32 v228, v[(((\j)+1)&1)*64+(\qb)*16], v[(((\j)+1)&1)*64+(\qb)*16+1], v[(((\j)+1)&1)*64+(\qb)*16+2]
      .irp r, 3, 5, 7, 9, 11, 13
        v_max3_f32 v228, v228, v[(((\j)+1)&1)*64+(\qb)*16+(\r)], v[(((\j)+1)&1)*64+(\qb)*16+(\r)+1]
      .endr
      v_max_f32 v228, v228, v[(((\j)+1)&1)*64+(\qb)*16+15]
      .irp r, 0, 2, 4, 6, 8, 10, 12, 14
        v_max3_f32 v228, v228, v[(((\j)+1)&1)*64+32+(\qb)*16+(\r)], v[(((\j)+1)&1)*64+32+(\qb)*16+(\r)+1]
      .endr
      v_mov_b32 v229, v228
      s_nop 1
      v_permlane32_swap_b32 v228, v229
      s_nop 1
      v_max_f32 v[233+(\qb)], v228, v229
    .endr
    .irp qb, 0, 1
      v_max_f32 v235, v[192+(\qb)], v[233+(\qb)]
      v_sub_f32 v236, v235, v[192+(\qb)]
      v_mul_f32 v236, s79, v236
      v_cmp_lt_f32 vcc, 0x41000000, v236
      s_and_b64 vcc, exec, vcc
      s_cbranch_vccz L_keep_\j\()_\uid\()_\qb
      v_sub_f32 v236, v[192+(\qb)], v235
      v_mul_f32 v236, s79, v236
      v_exp_f32 v236, v236
      s_nop 1
      .irp r, 0,4,8,12,16,20,24,28,32,36,40,44,48,52,56,60
        v_accvgpr_read_b32 v228, a[(\qb)*64+(\r)]
        v_accvgpr_read_b32 v229, a[(\qb)*64+(\r)+1]
        v_accvgpr_read_b32 v230, a[(\qb)*64+(\r)+2]
        v_accvgpr_read_b32 v231, a[(\qb)*64+(\r)+3]
        v_mul_f32 v228, v228, v236
        v_mul_f32 v229, v229, v236
        v_mul_f32 v230, v230, v236
        v_mul_f32 v231, v231, v236
        v_accvgpr_write_b32 a[(\qb)*64+(\r)], v228
        v_accvgpr_write_b32 a[(\qb)*64+(\r)+1], v229
        v_accvgpr_write_b32 a[(\qb)*64+(\r)+2], v230
        v_accvgpr_write_b32 a[(\qb)*64+(\r)+3], v231
      .endr
      v_mul_f32 v[194+(\qb)], v[194+(\qb)], v236
      v_mov_b32 v[192+(\qb)], v235
    L_keep_\j\()_\uid\()_\qb:
    .endr
    v_mul_f32_e64 v198, -v192, s79
    v_mul_f32_e64 v199, -v193, s79
    .irp n, 0,1,2,3,4,5,6,7,8,9,10,11,12,13,14,15,16,17,18,19,20,21,22,23,24,25,26,27,28,29,30,31
      FA_E \n, 0, (((\j)+1)&1)
      FA_E \n, 1, (((\j)+1)&1)
    .endr
    s_nop 2
    .irp n, 0,1,2,3,4,5,6,7,8,9,10,11,12,13,14,15,16,17,18,19,20,21,22,23,24,25,26,27,28,29,30,31
      FA_C \n, (((\j)+1)&1)
    .endr
    s_nop 4
    .irp b, 0, 1, 2, 3
      FA_RSMFMA \b, 0
      FA_RSMFMA \b, 1
    .endr
    s_nop 7
    s_nop 7
    s_nop 7
    v_accvgpr_read_b32 v196, a192
    v_accvgpr_read_b32 v197, a196
    s_nop 4
    s_branch L_rret_\j\()_\uid
  .endm

  // ---- out of line: the P V half of a step whose tile p is a causal
  // diagonal tile past this wave's rows: its P is zero, so no P V products
  // and no V reads (V fragments 0..2, read at the end of the last step, are
  // waited for with the K fragments in the score half); the softmax of tile
  // p+1 and the first K reads of tile p+2 as in the full half
  .macro FA_PVD j, uid
  L_pvd_\j\()_\uid:
    s_cmp_gt_u32 s74, s81
    s_cbranch_scc0 L_pvfull_\j\()_\uid
    .irp t, 0,1,2,3,4,5,6,7,8,9,10,11,12,13,14,15,16,17,18,19,20,21,22,23,24,25,26,27,28,29,30,31
      .if ((\t) == 27) || ((\t) == 29) || ((\t) == 31)
        FA_KREAD (((\t)-27)>>1), (((\j)+2)&3)
      .endif
      FA_VPOS \t, (((\j)+1)&1)
    .endr
    s_branch L_pvret_\j\()_\uid
  .endm

  .macro FA_MASK j, uid
  L_mask_\j\()_\uid:
    FA_MASKSET ((\j)&1), 2
    s_branch L_mret_\j\()_\uid
  .endm

  // ---- out of line: the score half of the block's last two steps, whose
  // score tiles p+2 lie past its end: the same row sums, softmax, ring
  // refills and V reads, without the score MFMAs (nops keep the hazard
  // distances the score MFMAs gave)
  .macro FA_NS j, uid
    // a masked tile p+2: without the causal mask's diagonal tiles past
    // this wave's rows (position > wave), whose scores the mask turns
    // into -inf whatever they hold
  L_diag_\j\()_\uid:
    s_cmp_gt_u32 s86, s81
    s_cbranch_scc0 L_sfull_\j\()_\uid
  L_ns_\j\()_\uid:
    .irp t, 32,33,34,35,36,37,38,39,40,41,42,43,44,45,46,47,48,49,50,51,52,53,54,55,56,57,58,59,60,61,62,63,64,65,66,67,68,69,70,71
      .if ((\t) <= 35) || ((\t) == 42) || ((\t) == 50) || ((\t) == 58) || ((\t) == 66)
        s_nop 4
        FA_SPOS \t, \j
      .endif
      .if (\t) >= 62
        FA_REFILL ((\t)-62), \j, \uid\()n
      .endif
      .if (\t) >= 69
        FA_VREAD ((\t)-69), (((\j)+1)&3)
      .endif
      FA_VPOS \t, (((\j)+1)&1)
    .endr
    s_nop 7
    s_nop 7
    s_nop 7
    s_branch L_nsret_\j\()_\uid
  .endm

  // score sets swapped on entry at an odd ring slot: tile 1's scores belong
  // in set 0
  .macro FA_SWAPSETS
    .irp r, 0,1,2,3,4,5,6,7,8,9,10,11,12,13,14,15,16,17,18,19,20,21,22,23,24,25,26,27,28,29,30,31,32,33,34,35,36,37,38,39,40,41,42,43,44,45,46,47,48,49,50,51,52,53,54,55,56,57,58,59,60,61,62,63
      v_mov_b32 v[\r], v[64+(\r)]
    .endr
  .endm

  s_waitcnt lgkmcnt(0)
  .irp r, 0,1,2,3,4,5,6,7,8,9,10,11,12,13,14,15,16,17,18,19,20,21,22,23,24,25,26,27,28,29,30,31,32,33,34,35,36,37,38,39,40,41,42,43,44,45,46,47,48,49,50,51,52,53,54,55,56,57,58,59,60,61,62,63
    v_accvgpr_write_b32 a[\r], 0
    v_accvgpr_write_b32 a[64+(\r)], 0
  .endr
  v_mul_f32_e64 v198, -v192, s79
  v_mul_f32_e64 v199, -v193, s79
  s_mov_b32 s87, 0x47800000
  s_waitcnt vmcnt(16)
  s_barrier
  // enter the unrolled ring at the block's first slot (s97)
  s_cmp_eq_u32 s97, 1
  s_cbranch_scc1 L_e1_%=
  s_cmp_eq_u32 s97, 2
  s_cbranch_scc1 L_e2_%=
  s_cmp_eq_u32 s97, 3
  s_cbranch_scc1 L_e3_%=
  FA_VREAD 0, 0
  FA_VREAD 1, 0
  FA_VREAD 2, 0
  s_branch L_s0_%=
L_e1_%=:
  FA_SWAPSETS
  FA_VREAD 0, 1
  FA_VREAD 1, 1
  FA_VREAD 2, 1
  s_branch L_s1_%=
L_e2_%=:
  FA_VREAD 0, 2
  FA_VREAD 1, 2
  FA_VREAD 2, 2
  s_branch L_s2_%=
L_e3_%=:
  FA_SWAPSETS
  FA_VREAD 0, 3
  FA_VREAD 1, 3
  FA_VREAD 2, 3
  s_branch L_s3_%=
L_s0_%=:
  FA_STEP 0, %=
L_s1_%=:
  FA_STEP 1, %=
L_s2_%=:
  FA_STEP 2, %=
L_s3_%=:
  FA_STEP 3, %=
  s_branch L_s0_%=
  FA_RARE 0, %=
  FA_RARE 1, %=
  FA_RARE 2, %=
  FA_RARE 3, %=
  FA_MASK 0, %=
  FA_MASK 1, %=
  FA_MASK 2, %=
  FA_MASK 3, %=
  FA_PVD 0, %=
  FA_PVD 1, %=
  FA_PVD 2, %=
  FA_PVD 3, %=
  .irp jj, 0, 1, 2, 3
    FA_NS \jj, %=
    FA_RNEXT \jj, %=
    FA_RNEXT \jj, %=n
  .endr
L_done_%=:
  s_waitcnt lgkmcnt(0)
  s_nop 7
  s_nop 7
  s_nop 7
  .purgem FA_E
  .purgem FA_C
  .purgem FA_VPOS
  .purgem FA_SMFMA
  .purgem FA_PMFMA
  .purgem FA_RSMFMA
  .purgem FA_KREAD
  .purgem FA_VREAD
  .purgem FA_TILE_BYTES
  .purgem FA_REFILL
  .purgem FA_SK
  .purgem FA_SPOS
  .purgem FA_MASKSET
  .purgem FA_STEP
  .purgem FA_RARE
  .purgem FA_MASK
  .purgem FA_PVD
  .purgem FA_SWAPSETS
  .purgem FA_RNEXT
  .purgem FA_NS
)ASM"

// One work item: a block of kRows query rows of one (batch, head), its key
// tiles in processing order -- the R tiles that need the elementwise mask
// (the causal diagonal region, or a ragged last tile) first, then tiles 0..
struct Block {
  int qtile, bh;
  int nt;  // key tiles visited
  int fm;  // first masked tile
  int R;   // masked tiles
};

template <bool CAUSAL>
__device__ __forceinline__ Block make_block(const TileSched& sched, int hw, int N) {
  Block k;
  sched_item(sched, hw, k.qtile, k.bh);
  const int q0 = k.qtile * kRows;
  const int n_ktiles = (N + kBlockN - 1) / kBlockN;
  k.nt = n_ktiles;
  if constexpr (CAUSAL) k.nt = min(q0 + kRows - 1, N - 1) / kBlockN + 1;
  k.fm = k.nt;
  if (CAUSAL) k.fm = q0 / kBlockN;
  else if (N % kBlockN != 0) k.fm = n_ktiles - 1;
  k.R = k.nt - k.fm;
  return k;
}

// The blocks of workgroup w.  With one block per workgroup (cont == 0) that
// is block w.  Persistent (cont != 0, gridDim.x a multiple of 8): round r
// gives workgroup w = 8u + x the block 8 * (u, or U-1-u in odd rounds) + x of
// the r-th run of gridDim.x blocks in scheduler order (U = gridDim.x / 8), so
// a workgroup keeps to the heads of its XCD (x = w mod 8, where the
// dispatcher places it) and, since the scheduler orders a causal grid
// heaviest first, alternate rounds pair heavy blocks with light ones.
__device__ __forceinline__ int block_of(int w, int round, int n_blocks, int cont) {
  if (!cont) return round == 0 ? w : -1;
  const int G = (int)gridDim.x, U = G >> 3, x = w & 7, u = w >> 3;
  const int hw = round * G + 8 * ((round & 1) ? U - 1 - u : u) + x;
  return hw < n_blocks ? hw : -1;
}

template <bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kWaves, 64 * kWaves), amdgpu_waves_per_eu(1, 1))) void
fwd_d128_kernel(FwdArgs a, TileSched sched, int n_blocks, int cont) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[kRingBytes + kStageBytes];
  lds_char* smem = (lds_char*)smem_raw;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, half = lane >> 5;
  const int N = a.N;
  const uint32_t last_tile_bytes = (uint32_t)(N - kBlockN) * (D * 2);
  const int w = (int)blockIdx.x;

  // ring copies: K slots at [0, 64 KB), V slots at [64 KB, 128 KB)
  RowTileCopier<D, D, kBlockN, kWaves> cp;
  cp.init(wave, lane);
  // per-lane LDS addresses of the K and V fragments (ring base included)
  const uint32_t ring = (uint32_t)(uintptr_t)smem;
  i32x8 koff, voff;
#pragma unroll
  for (int ds = 0; ds < 8; ++ds) koff[ds] = (int)ring + lds_off_bytes<D>(l32, ds * 2 + half);
  {
    const int g = lane >> 4, j16 = lane & 15;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int dcol = db * 32 + (g & 1) * 16 + (j16 & 3) * 4;
      const int r1 = half * 4 + (j16 >> 2);
#pragma unroll
      for (int t = 0; t < 2; ++t)
        voff[db * 2 + t] = (int)ring + kNB * kTileBytes + lds_off_bytes<D>(r1 + 8 * t, dcol >> 3) + (dcol & 7) * 2;
    }
  }
  const i32x4 cpoff = {(int)cp.off[0], (int)cp.off[1], (int)cp.off[2], (int)cp.off[3]};
  const int half4 = half * 4;
  // A operand of the row-sum MFMAs: bf16 ones where ((lane mod 16) / 4) mod 2
  // equals (lane / 16) mod 2, zeros elsewhere
  const int rsel1 = (((lane & 15) >> 2) & 1) == ((lane >> 4) & 1) ? 0x3f803f80 : 0;
  const i32x4 rsel = {rsel1, rsel1, rsel1, rsel1};
  const float c = a.scale_log2;

  auto head = [&](const __bf16* t, int bh) { return t + (size_t)bh * N * D; };
  auto tile_bytes = [&](const Block& k, int p) {
    const int t = p < k.R ? k.fm + p : p - k.R;
    return min((uint32_t)t * (uint32_t)kTileBytes, last_tile_bytes);
  };
  // Q^T fragments of a block: query column l32 of each 32-row group, d = ds*16 + half*8 .. +7
  bf16x8 qf[2][8];
  auto load_q = [&](const Block& k) {
    const __bf16* __restrict__ Q = head((const __bf16*)a.q, k.bh);
    const int wq0 = k.qtile * kRows + wave * 64;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int row = min(wq0 + qb * 32 + l32, N - 1);
#pragma unroll
      for (int ds = 0; ds < 8; ++ds) qf[qb][ds] = *(const bf16x8*)(Q + (size_t)row * D + ds * 16 + half * 8);
    }
  };

  int round = 0;
  Block cur = make_block<CAUSAL>(sched, block_of(w, 0, n_blocks, cont), N);
  // the first block: its Q rows, then its prologue copies in the order the
  // first steps need them, K0 K1 V0 K2 V1 K3 V2 (positions past its last
  // tile load a valid tile that is never read).  Later blocks find theirs
  // in the ring, copied by the steps of the block before.
  load_q(cur);
  {
    const __bf16* K = head((const __bf16*)a.k, cur.bh);
    const __bf16* V = head((const __bf16*)a.v, cur.bh);
    auto issue_k = [&](int p) { cp.copy_at(K, tile_bytes(cur, p), smem + p * kTileBytes); };
    auto issue_v = [&](int p) { cp.copy_at(V, tile_bytes(cur, p), smem + (kNB + p) * kTileBytes); };
    issue_k(0);
    issue_k(1);
    issue_v(0);
    issue_k(2);
    issue_v(1);
    issue_k(3);
    issue_v(2);
  }
  wait_vmcnt<5 * RowTileCopier<D, D, kBlockN, kWaves>::kLoads>();  // Q, K0 and K1 landed
  int r0 = 0;  // ring slot of the block's first tile

  for (;;) {
    const int hw_next = block_of(w, round + 1, n_blocks, cont);
    const bool has_next = hw_next >= 0;
    const Block nxt = has_next ? make_block<CAUSAL>(sched, hw_next, N) : cur;
    const int wq0 = cur.qtile * kRows + wave * 64;
    // causal bound of each query block: keys < bound are visible
    int bound0 = N, bound1 = N;
    if constexpr (CAUSAL) {
      bound0 = min(N, wq0 + l32 + 1);
      bound1 = min(N, wq0 + 32 + l32 + 1);
    }

    // scores of the tile at position p from K ring slot b, masked when p < R
    auto scores = [&](int b, int p, f32x16 (&s)[2][2]) {
      if (CAUSAL && p < cur.R && p > wave) {  // a diagonal tile past this wave's rows
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][qb][r] = -__builtin_inff();
        return;
      }
#pragma unroll
      for (int ds = 0; ds < 8; ++ds)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 kf =
              *(const bf16x8 __attribute__((address_space(3)))*)(smem + b * kTileBytes + koff[ds] - ring + kb * 32 * D * 2);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) s[kb][qb] = mfma32(kf, qf[qb][ds], ds == 0 ? f32x16{} : s[kb][qb]);
        }
      if (p < cur.R) {
        // -inf where a key is invisible (the loop's mask rule)
        const int t = cur.fm + p;
        const int row0 = min(t * kBlockN, N - kBlockN);
        int base = row0 + half4;
        // (kept opaque: hoisted out of the block loop, the 64 comparisons
        // would each hold an SGPR pair for the kernel's whole life)
        asm volatile("" : "+v"(base));
        const int lo = t * kBlockN - base;
        const int hi[2] = {bound0 - base, bound1 - base};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int off = kb * 32 + (r >> 2) * 8 + (r & 3);
              s[kb][qb][r] = (off >= lo && off < hi[qb]) ? s[kb][qb][r] : -__builtin_inff();
            }
      }
    };

    // tile 0: scores, the running max (its row max; a finite floor where a
    // row sees none of its keys), P and the row sums over the rounded P.
    // Every wave's copies of tiles 0 and 1 have landed (waited for above,
    // or at the start of the previous block's last step).
    __syncthreads();
    f32x16 s0[2][2], s1[2][2];
    scores(r0, 0, s0);
    float m[2], l[2];
    bf16x8 p0[2][2][2];  // [qb][kb][cc]
    const bf16x8 rsel_bf = __builtin_bit_cast(bf16x8, rsel);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float t = -kMaxFloor;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) t = __builtin_fmaxf(t, s0[kb][qb][r]);
      m[qb] = max_halves(t);
      const float nmc = -m[qb] * c;
      // row sums over the rounded P on the loop's row-sum MFMAs (selector x P)
      f32x4 rs = {};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          bf16x2 pr[4];
#pragma unroll
          for (int w4 = 0; w4 < 4; ++w4)
            pr[w4] = pack_bf16(fast_exp2(__builtin_fmaf(s0[kb][qb][cc * 8 + 2 * w4], c, nmc)),
                               fast_exp2(__builtin_fmaf(s0[kb][qb][cc * 8 + 2 * w4 + 1], c, nmc)));
          p0[qb][kb][cc] = join8(pr[0], pr[1], pr[2], pr[3]);
          rs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rsel_bf, p0[qb][kb][cc], rs, 0, 0, 0);
        }
      l[qb] = rs[0];  // every lane holds its row's whole sum
    }
    // the scores of tile 1
    scores((r0 + 1) & 3, 1, s1);

    f32x32 o0, o1, o2, o3;  // O^T: a[0:31] (qb 0, db 0-1) .. a[96:127] (qb 1, db 2-3)
    f32x32 junk0, junk1;    // registers the loop uses internally
    f32x16 junk2, junk3;
    f32x4 junk4;
    f32x8 junk5;
    // scalar operands of the loop, pinned to SGPRs (all are wave-uniform)
    auto sgpr = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
    auto sgpr_ptr = [](const __bf16* x) {
      const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)x);
      const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uintptr_t)x >> 32));
      return (const __bf16*)(((uint64_t)hi << 32) | (uint64_t)lo);
    };
    int p = sgpr(0);
    const int ring_wave = sgpr((int)ring + (int)cp.lds_wave);
    const float cs = __builtin_bit_cast(float, sgpr(__builtin_bit_cast(int, c)));
    const __bf16* Ks = sgpr_ptr(head((const __bf16*)a.k, cur.bh));
    const __bf16* Kn = sgpr_ptr(head((const __bf16*)a.k, nxt.bh));
    // the address K(3) was copied from (the first V refill reads the same
    // tile of V), and the distance from the K tensor to the V tensor
    const __bf16* k_addr =
        sgpr_ptr((const __bf16*)((const char*)head((const __bf16*)a.k, cur.bh) + tile_bytes(cur, 3)));
    const int64_t kv_dist = (int64_t)((const char*)a.v - (const char*)a.k);
    const int64_t kv_s = ((int64_t)sgpr((int)(uint32_t)((uint64_t)kv_dist >> 32)) << 32) |
                         (int64_t)(uint32_t)sgpr((int)(uint32_t)(uint64_t)kv_dist);
    const int nt_s = sgpr(cur.nt), R_s = sgpr(cur.R), fm_s = sgpr(cur.fm);
    // the diagonal tile at position i (i < R under causal masking) is fully
    // masked for the rows of waves below i
    const int wave_s = sgpr(CAUSAL ? wave : 1 << 30);
    const int ltb_s = sgpr((int)last_tile_bytes);
    const int Rn_s = sgpr(nxt.R), fmn_s = sgpr(nxt.fm), r0_s = sgpr(r0);
    asm volatile(FA_D128_LOOP_ASM
                 : "={a[0:31]}"(o0), "={a[32:63]}"(o1), "={a[64:95]}"(o2), "={a[96:127]}"(o3),
                   "=&{v[0:31]}"(junk0), "+{v[64:79]}"(s1[0][0]), "+{v[80:95]}"(s1[0][1]), "+{v[96:111]}"(s1[1][0]),
                   "+{v[112:127]}"(s1[1][1]), "+{v[128:131]}"(p0[0][0][0]), "+{v[132:135]}"(p0[0][0][1]),
                   "+{v[136:139]}"(p0[0][1][0]), "+{v[140:143]}"(p0[0][1][1]), "+{v[144:147]}"(p0[1][0][0]),
                   "+{v[148:151]}"(p0[1][0][1]), "+{v[152:155]}"(p0[1][1][0]), "+{v[156:159]}"(p0[1][1][1]),
                   "+{v192}"(m[0]), "+{v193}"(m[1]), "+{v194}"(l[0]), "+{v195}"(l[1]), "+{s74}"(p), "+{s[98:99]}"(k_addr),
                   "=&{v[32:63]}"(junk1), "=&{v[160:175]}"(junk2), "=&{v[176:191]}"(junk3), "=&{v[196:199]}"(junk4),
                   "=&{a[192:199]}"(junk5)
                 : "{a[128:131]}"(qf[0][0]), "{a[132:135]}"(qf[0][1]), "{a[136:139]}"(qf[0][2]), "{a[140:143]}"(qf[0][3]),
                   "{a[144:147]}"(qf[0][4]), "{a[148:151]}"(qf[0][5]), "{a[152:155]}"(qf[0][6]), "{a[156:159]}"(qf[0][7]),
                   "{a[160:163]}"(qf[1][0]), "{a[164:167]}"(qf[1][1]), "{a[168:171]}"(qf[1][2]), "{a[172:175]}"(qf[1][3]),
                   "{a[176:179]}"(qf[1][4]), "{a[180:183]}"(qf[1][5]), "{a[184:187]}"(qf[1][6]), "{a[188:191]}"(qf[1][7]),
                   "{v[200:207]}"(koff), "{v[208:215]}"(voff), "{v[216:219]}"(cpoff), "{v220}"(bound0), "{v221}"(bound1),
                   "{v222}"(half4), "{v[224:227]}"(rsel), "{s[70:71]}"(Ks), "{s75}"(nt_s), "{s76}"(R_s),
                   "{s77}"(fm_s), "{s78}"(ltb_s), "{s79}"(cs), "{s80}"(ring_wave), "{s81}"(wave_s), "{s[90:91]}"(Kn),
                   "{s[92:93]}"(kv_s), "{s94}"(Rn_s), "{s95}"(fmn_s), "{s97}"(r0_s)
                 : "v223", "v228", "v229", "v230", "v231", "v232", "v233", "v234", "v235", "v236", "s82", "s83", "s84",
                   "s85", "s86", "s87", "s88", "s89", "m0", "vcc", "exec", "scc", "memory");
    // The next block's tiles 0 and 1 have landed (its ring copies were issued
    // from four and three steps before the end); its Q rows load during this
    // block's epilogue.
    const Block done = cur;
    if (has_next) load_q(nxt);

    // ---- epilogue: O = acc / l, L = m*scale + ln l.  Each wave stages its
    // 64 x 128 bf16 block of O, 32 rows at a time, in its own 8 KB past the
    // ring (256-byte rows, 16-byte chunks XOR-swizzled by row) and stores it
    // in whole rows: a lane's fragment holds 8 bytes of 32 different rows,
    // which stored directly would split every store into 32 row pieces.
    __bf16* __restrict__ O = (__bf16*)a.o + (size_t)done.bh * N * D;
    float* __restrict__ Lse = a.lse + (size_t)done.bh * N;
    lds_char* ostage = smem + kRingBytes + wave * (32 * D * 2);
    const f32x32 ob[2][2] = {{o0, o1}, {o2, o3}};
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float lt = l[qb];
      const float inv = 1.0f / lt;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x32& x = ob[qb][db >> 1];
          const int e = (db & 1) * 16 + g4 * 4;
          const u32x2 v2 = {pack_bf16_u32(x[e + 0] * inv, x[e + 1] * inv), pack_bf16_u32(x[e + 2] * inv, x[e + 3] * inv)};
          const int chunk = db * 4 + g4;
          *(u32x2 __attribute__((address_space(3)))*)(ostage + l32 * (D * 2) + ((chunk ^ (l32 & 15)) << 4) + half * 8) = v2;
        }
      const int row = wq0 + qb * 32 + l32;
      if (row < N && half == 0) Lse[row] = m[qb] * a.scale + fast_log2(lt) * kLn2;
      // back in rows: lanes 16k .. 16k+15 hold one 256-byte row
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int r = k * 4 + (lane >> 4), ch = lane & 15;
        const u32x4 v4 = *(const u32x4 __attribute__((address_space(3)))*)(ostage + r * (D * 2) + ((ch ^ (r & 15)) << 4));
        const int orow = wq0 + qb * 32 + r;
        if (orow < N) *(u32x4*)(O + (size_t)orow * D + ch * 8) = v4;
      }
    }
    if (!has_next) break;
    r0 = (r0 + done.nt) & 3;
    cur = nxt;
    ++round;
  }
  wait_vmcnt<0>();  // no direct-to-LDS copy may outlive the workgroup
}

}  // namespace d128

// Square forward at D = 128 for N >= 64 (callers route shorter tensors to
// the generic kernel).  From N = 256 on (every block then visits at least
// four key tiles) a grid larger than the device runs persistently: one
// workgroup per compute unit, each working through its blocks with the ring
// carried from one block into the next.
int launch_fwd_d128(const FwdArgs& a, hipStream_t stream) {
  if (a.D != 128 || a.N < d128::kBlockN) return -2;
  const int n_qtiles = (a.N + d128::kRows - 1) / d128::kRows;
  TileSched sched = make_sched(n_qtiles, a.B * a.H, a.causal != 0);
  const long n_blocks = (long)n_qtiles * a.B * a.H;
  long grid = n_blocks;
  int cont = 0;
  const int cus = device_cus();
  if (a.N >= 4 * d128::kBlockN && cus >= 8 && n_blocks > cus) {
    grid = cus & ~7;
    cont = 1;
    sched.head_major = 1;
  }
  if (a.causal)
    hipLaunchKernelGGL(d128::fwd_d128_kernel<true>, dim3((unsigned)grid), dim3(64 * d128::kWaves), 0, stream, a, sched,
                       (int)n_blocks, cont);
  else
    hipLaunchKernelGGL(d128::fwd_d128_kernel<false>, dim3((unsigned)grid), dim3(64 * d128::kWaves), 0, stream, a, sched,
                       (int)n_blocks, cont);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace fa
