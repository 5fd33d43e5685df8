// fa_fwd_d256.hip -- square exact-attention forward at head dimension 256,
// bf16 in and out, without causal masking: 32 query rows per wave, the key
// loop in hand-scheduled gfx950 assembly.
//
// The method is the one of the other forward kernels and of the pages
// ("Learning Metal with FlashAttention", section FlashAttention; "Flash
// Attention" page, kernel anatomy; metal-flash-attention README,
// "Quantifying performance", forward pseudocode): Q rows resident, K and V
// streamed in tiles of 64 keys through LDS, S^T = K Q^T on 32x32x16 bf16
// MFMA, an online softmax in the exp2 domain against a running reference
// max, O^T += V^T P^T with P straight from the score accumulators.
//
// A workgroup owns 64 query rows (two 32-row blocks) and four waves; waves
// w and w+2 hold the same rows and take the two 32-key halves of every
// tile, and merge their partial results (m, l, O) through LDS at the end.
// One wave per SIMD: the 256 O accumulators of 64 rows would not fit beside
// the rest, and c5-sized grids (B*H*N/64 workgroups) just fill the chip.
// A wave keeps its Q rows (64 registers) and O accumulators (128) in AGPRs,
// which the MFMAs read and write directly, so Q is read from memory once and
// LDS holds only the K ring (2 tiles of 32 KB) and the V ring (3).
//
// Step p issues 32 MFMAs -- the 16 score products of tile p+1, carrying the
// softmax of tile p in their shadow (per score an FMA to the exp2 domain
// and a v_exp_f32 into a temporary, the bf16 packs into P and their row
// sums by v_dot2 against ones, software-pipelined so that no exp2 result is
// read by the next instruction), then the 16 P V products of tile p -- and
// between them, one fragment read per MFMA six positions ahead of its use
// and one of the 16 copies (1 KB each) of tile p+2.  A step waits for its
// copies of the step before (K) and of two steps before (V) and passes one
// barrier.  The running max is a reference point, as in the other kernels:
// when a lane's share of a tile's row sum exceeds 2^16 (or is not finite) an
// out-of-line path raises it to the tile's row max, rescales O and l and
// redoes the tile's softmax from the kept scores.  The loop is unrolled six
// times (K slot p mod 2, V slot p mod 3) so that every LDS offset is a
// constant.  The prologue (Q rows, the copies of tiles 0 and 1, the scores
// and row max of tile 0) and the merge and epilogue are ordinary C++.
//
// Register map inside the loop (v = VGPR, a = AGPR):
//   v[0:15], v[16:31]    score sets: tile q in set q mod 2 (a key per
//                        register r: (r/4)*8 + half*4 + r%4; a query per lane)
//   v[32:39]             P (bf16 pairs): chunk kc of 16 keys at 32 + 4 kc
//   v[40:63]             6 fragment buffers
//   v[64:79]             exponentials of the tile in hand (temporaries)
//   v80, v81, v82, v83   running max m, -m*c, row sum l, the tile's row sum
//   v84, v85             bf16 ones (row sums), the ragged-tile mask bound
//   v86, v87             temporaries
//   v[88:95]             per-lane K fragment addresses (k-step mod 8; K slot 0)
//   v[96:111]            per-lane V^T fragment addresses (d block mod 4 x 2
//                        reads; V slots 0 and 1, then slot 2)
//   v[112:119]           per-lane global offsets of this lane's copies
//   a[0:127]             O^T accumulators, d block db at 16 db
//   a[128:191]           Q^T fragments, k-step ds at 128 + 4 ds
//   s[70:71], s[72:73]   K and V of the head;  s74 position p;  s75 tiles
//   s76 last tile byte offset;  s77, s78 this wave's copy base in the K and V
//   rings;  s79 scale*log2(e);  s80 tiles - 1;  s81 the ragged last tile
//   (or none);  s82..s91 scalar temporaries
#include "fa_device.h"
#include "fa_kernels.h"
#include "fa_sched.h"

namespace fa {
namespace d256 {

constexpr int D = 256;
constexpr int kWaves = 4;
constexpr int kRows = 64;                       // query rows per workgroup
constexpr int kBlockN = 64;                     // keys per tile (32 per wave)
constexpr int kTileBytes = kBlockN * D * 2;     // 32 KB
constexpr int kKSlots = 2, kVSlots = 3;
constexpr int kVRing = kKSlots * kTileBytes;    // byte offset of the V ring
constexpr int kLdsBytes = (kKSlots + kVSlots) * kTileBytes;
static_assert(kLdsBytes <= 160 * 1024, "LDS of one workgroup");
static_assert(2 * 64 * 130 * 4 + 2 * 32 * D * 2 <= kLdsBytes, "the merge and the output staging reuse the ring");

typedef __attribute__((ext_vector_type(32))) float f32x32;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(16))) int i32x16;

// The key loop.  Macros of the GNU assembler syntax the LLVM integrated
// assembler accepts; register numbers are assembler expressions.
#define FD_LOOP_ASM R"ASM(
  .macro FD_WAIT n
    .if (\n) <= 0
      s_waitcnt lgkmcnt(0)
    .elseif (\n) < 15
      s_waitcnt lgkmcnt(\n)
    .endif
  .endm
  // K fragment p (k-step p) of ring slot ks into buffer p mod 6
  .macro FD_RX p, ks
    ds_read_b128 v[40+((\p)%%6)*4:43+((\p)%%6)*4], v[88+((\p)&7)] offset:((\ks)*32768+((\p)>>3)*256)
  .endm
  // V^T fragment f (16-key chunk f/8, d block f mod 8) of V ring slot vs
  // into buffer p mod 6: two transposed reads, rows r and r + 8
  .macro FD_TX f, vs, p
    .if (\vs) == 2
      ds_read_b64_tr_b16 v[40+((\p)%%6)*4:41+((\p)%%6)*4], v[104+2*((\f)&3)] offset:(((\f)>>3)*8192+(((\f)>>2)&1)*256)
      ds_read_b64_tr_b16 v[42+((\p)%%6)*4:43+((\p)%%6)*4], v[105+2*((\f)&3)] offset:(((\f)>>3)*8192+(((\f)>>2)&1)*256)
    .else
      ds_read_b64_tr_b16 v[40+((\p)%%6)*4:41+((\p)%%6)*4], v[96+2*((\f)&3)] offset:((\vs)*32768+((\f)>>3)*8192+(((\f)>>2)&1)*256)
      ds_read_b64_tr_b16 v[42+((\p)%%6)*4:43+((\p)%%6)*4], v[97+2*((\f)&3)] offset:((\vs)*32768+((\f)>>3)*8192+(((\f)>>2)&1)*256)
    .endif
  .endm
  // stream position p: K fragments before nsx (one read each), then the 16
  // V fragments (two reads each)
  .macro FD_RD p, nsx, ks, vs
    .if (\p) < (\nsx)
      FD_RX (\p), (\ks)
    .elseif (\p) < (\nsx) + 16
      FD_TX ((\p)-(\nsx)), (\vs), (\p)
    .endif
  .endm
  .macro FD_RD6 nsx, ks, vs
    FD_RD 0, \nsx, \ks, \vs
    FD_RD 1, \nsx, \ks, \vs
    FD_RD 2, \nsx, \ks, \vs
    FD_RD 3, \nsx, \ks, \vs
    FD_RD 4, \nsx, \ks, \vs
    FD_RD 5, \nsx, \ks, \vs
  .endm
  // wait until at most the reads of positions a..b-1 remain
  .macro FD_WT2 a, b, nsx
    .if (\b) <= (\nsx)
      FD_WAIT ((\b)-(\a))
    .elseif (\a) >= (\nsx)
      FD_WAIT (2*((\b)-(\a)))
    .else
      FD_WAIT (((\nsx)-(\a))+2*((\b)-(\nsx)))
    .endif
  .endm
  // before the MFMA of position m: its fragment landed (the next five may
  // still be in flight)
  .macro FD_WT m, nsx
    .if (\m)+6 <= (\nsx)+16
      FD_WT2 ((\m)+1), ((\m)+6), (\nsx)
    .else
      FD_WT2 ((\m)+1), ((\nsx)+16), (\nsx)
    .endif
  .endm
  // softmax slot s (0..18) of the tile in score set sj: element s's
  // exponent (into temporary s), element s-1's exp2, pair (s-3)/2's pack
  // into P and pair (s-4)/2's row-sum dot product; an exp2 result is read
  // no sooner than one instruction later
  .macro FD_EX s, sj
    .if (\s) == 0
      v_mov_b32 v83, 0
    .endif
    .if (\s) < 16
      v_fma_f32 v[64+(\s)], v[16*(\sj)+(\s)], s79, v81
    .endif
    .if ((\s) >= 1) && ((\s) <= 16)
      v_exp_f32 v[63+(\s)], v[63+(\s)]
    .endif
    .if (\s) == 17
      s_nop 0
    .endif
    .if ((\s) >= 3) && ((\s) <= 17) && (((\s)&1) == 1)
      v_cvt_pk_bf16_f32 v[32+((\s)-3)/2], v[61+(\s)], v[62+(\s)]
    .endif
    .if ((\s) >= 4) && ((\s) <= 18) && (((\s)&1) == 0)
      v_dot2_f32_bf16 v83, v[32+((\s)-4)/2], v84, v83
    .endif
  .endm
  .macro FD_EXR lo, hi, sj
    .irp s, 0,1,2,3,4,5,6,7,8,9,10,11,12,13,14,15,16,17,18
      .if ((\s) >= (\lo)) && ((\s) < (\hi))
        FD_EX \s, \sj
      .endif
    .endr
  .endm
  // score MFMA m of the tile in K slot ks into score set sd (B: Q^T from
  // AGPRs), the read six positions ahead, copy m of the tile two ahead (K
  // into K slot ks^1 for m < 8, then V into V slot vd: the step after waits
  // for the K copies only), and the softmax slots of the tile in set se
  .macro FD_SM m, sd, se, ks, vs, vd
    FD_WT (\m), 16
    .if (\m) == 0
      v_mfma_f32_32x32x16_bf16 v[16*(\sd):16*(\sd)+15], v[40+((\m)%%6)*4:43+((\m)%%6)*4], a[128+4*(\m):131+4*(\m)], 0
    .else
      v_mfma_f32_32x32x16_bf16 v[16*(\sd):16*(\sd)+15], v[40+((\m)%%6)*4:43+((\m)%%6)*4], a[128+4*(\m):131+4*(\m)], v[16*(\sd):16*(\sd)+15]
    .endif
    .if (\m) < 8
      s_add_u32 m0, s77, ((\ks)^1)*32768+(\m)*1024
    .else
      s_add_u32 m0, s78, (\vd)*32768+((\m)-8)*1024
    .endif
    FD_RD ((\m)+6), 16, (\ks), (\vs)
    .if (\m) < 8
      global_load_lds_dwordx4 v[112+(\m)], s[86:87]
    .else
      global_load_lds_dwordx4 v[112+(\m)-8], s[88:89]
    .endif
    FD_EXR (((\m)*19)/16), ((((\m)+1)*19)/16), (\se)
  .endm
  // P V MFMA f (position nsx + f): O^T block f mod 8 += V^T (chunk f/8) P^T,
  // the read six ahead and, with cp, V copy f of the tile two ahead (into V
  // slot vd)
  .macro FD_PM f, nsx, vs, vd, cp
    FD_WT ((\nsx)+(\f)), (\nsx)
    v_mfma_f32_32x32x16_bf16 a[16*((\f)&7):16*((\f)&7)+15], v[40+(((\nsx)+(\f))%%6)*4:43+(((\nsx)+(\f))%%6)*4], v[32+4*((\f)>>3):35+4*((\f)>>3)], a[16*((\f)&7):16*((\f)&7)+15]
    .if (\cp) && ((\f) < 8)
      s_add_u32 m0, s78, (\vd)*32768+(\f)*1024
    .endif
    FD_RD ((\nsx)+(\f)+6), (\nsx), 0, (\vs)
    .if (\cp) && ((\f) < 8)
      global_load_lds_dwordx4 v[112+(\f)], s[88:89]
    .endif
  .endm
  // the row-sum shares of the tile's P: above 2^16 (or not finite) in any
  // lane -> the rare path, which returns to label ret
  .macro FD_CHECK j, ret, uid
    s_mov_b32 s82, 0x47800000
    v_cmp_nle_f32_e64 s[84:85], v83, s82
    s_and_b64 vcc, exec, s[84:85]
    s_getpc_b64 s[90:91]
  L_pc\ret\()_\uid:
    s_add_u32 s90, s90, (L_\ret\()_\uid - L_pc\ret\()_\uid)
    s_addc_u32 s91, s91, 0
    s_cbranch_vccnz L_rare\j\()_\uid
  L_\ret\()_\uid:
  .endm

  // ---- step p (s74) with p = j mod 2 = u mod 3: the scores of tile p+1
  // (K slot j^1) into set j^1 carrying the softmax of tile p (set j), then
  // O += V(p) P(p) (V slot u); copies of tile p+2 into K slot j and V slot
  // (u+2) mod 3.  The block's last tile takes the tail variant.
  .macro FD_STEP j, u, uid
    s_add_u32 s82, s74, 1
    s_cmp_ge_u32 s82, s75
    s_cbranch_scc1 L_t\j\u\()_\uid
    s_waitcnt vmcnt(8)
    s_barrier
    // copy sources: tile min(p+2, nt-1), a ragged last tile shifted back
    s_add_u32 s82, s74, 2
    s_min_u32 s82, s82, s80
    s_lshl_b32 s82, s82, 15
    s_min_u32 s82, s82, s76
    s_add_u32 s86, s70, s82
    s_addc_u32 s87, s71, 0
    s_add_u32 s88, s72, s82
    s_addc_u32 s89, s73, 0
    FD_RD6 16, ((\j)^1), \u
    .irp m, 0,1,2,3,4,5,6,7,8,9,10,11,12,13,14,15
      FD_SM \m, ((\j)^1), \j, ((\j)^1), \u, (((\u)+2)%%3)
    .endr
    FD_CHECK \j, r\j\u, \uid
    v_add_f32 v82, v82, v83
    .irp f, 0,1,2,3,4,5,6,7,8,9,10,11,12,13,14,15
      FD_PM \f, 16, \u, 0, 0
    .endr
    // tile p+1 is the ragged last tile: its scores take the mask
    s_add_u32 s82, s74, 1
    s_cmp_eq_u32 s82, s81
    s_cbranch_scc1 L_mk\j\u\()_\uid
  L_mr\j\u\()_\uid:
    s_add_u32 s74, s74, 1
  .endm
  // ---- the block's last tile: softmax, then O += V P, no scores and no copies
  .macro FD_TAIL j, u, uid
  L_t\j\u\()_\uid:
    s_waitcnt vmcnt(8)
    s_barrier
    FD_RD6 0, 0, \u
    .irp s, 0,1,2,3,4,5,6,7,8,9,10,11,12,13,14,15,16,17,18
      FD_EX \s, \j
    .endr
    FD_CHECK \j, q\j\u, \uid
    v_add_f32 v82, v82, v83
    .irp f, 0,1,2,3,4,5,6,7,8,9,10,11,12,13,14,15
      FD_PM \f, 0, \u, 0, 0
    .endr
    s_branch L_done_\uid
  .endm
  // ---- out of line: keys of the ragged last tile (loaded shifted back to end
  // at key N-1) that an earlier tile already held -> -inf in score set j^1
  .macro FD_MASK j, u, uid
  L_mk\j\u\()_\uid:
    s_nop 7
    s_nop 7
    v_mov_b32 v87, 0xff800000
    .irp r, 0,1,2,3,4,5,6,7,8,9,10,11,12,13,14,15
      v_cmp_lt_i32 vcc, (((\r)>>2)*8+((\r)&3)), v85
      v_cndmask_b32 v[16*((\j)^1)+(\r)], v[16*((\j)^1)+(\r)], v87, vcc
    .endr
    s_branch L_mr\j\u\()_\uid
  .endm
  // ---- out of line: the running max raised to the tile's row max where it
  // grew by more than 2^8 (exp2 domain), O and l rescaled, the softmax of the
  // tile (set j, kept) redone; returns through s[90:91]
  .macro FD_RARE j, uid
  L_rare\j\()_\uid:
    v_max3_f32 v86, v[16*(\j)+0], v[16*(\j)+1], v[16*(\j)+2]
    .irp r, 3, 5, 7, 9, 11, 13
      v_max3_f32 v86, v86, v[16*(\j)+(\r)], v[16*(\j)+(\r)+1]
    .endr
    v_max_f32 v86, v86, v[16*(\j)+15]
    v_mov_b32 v87, v86
    s_nop 1
    v_permlane32_swap_b32 v86, v87
    s_nop 1
    v_max_f32 v86, v86, v87
    v_max_f32 v86, v80, v86
    v_sub_f32 v87, v86, v80
    v_mul_f32 v87, s79, v87
    v_cmp_lt_f32 vcc, 0x41000000, v87
    v_cndmask_b32 v86, v80, v86, vcc
    v_sub_f32 v87, v80, v86
    v_mul_f32 v87, s79, v87
    v_exp_f32 v87, v87
    v_mov_b32 v80, v86
    v_mul_f32_e64 v81, -v80, s79
    s_nop 1
    v_mul_f32 v82, v82, v87
    .irp r, 0,4,8,12,16,20,24,28,32,36,40,44,48,52,56,60,64,68,72,76,80,84,88,92,96,100,104,108,112,116,120,124
      v_accvgpr_read_b32 v64, a[\r]
      v_accvgpr_read_b32 v65, a[(\r)+1]
      v_accvgpr_read_b32 v66, a[(\r)+2]
      v_accvgpr_read_b32 v67, a[(\r)+3]
      v_mul_f32 v64, v64, v87
      v_mul_f32 v65, v65, v87
      v_mul_f32 v66, v66, v87
      v_mul_f32 v67, v67, v87
      v_accvgpr_write_b32 a[\r], v64
      v_accvgpr_write_b32 a[(\r)+1], v65
      v_accvgpr_write_b32 a[(\r)+2], v66
      v_accvgpr_write_b32 a[(\r)+3], v67
    .endr
    .irp s, 0,1,2,3,4,5,6,7,8,9,10,11,12,13,14,15,16,17,18
      FD_EX \s, \j
    .endr
    s_nop 7
    s_nop 7
    s_setpc_b64 s[90:91]
  .endm

  .irp r, 0,1,2,3,4,5,6,7,8,9,10,11,12,13,14,15,16,17,18,19,20,21,22,23,24,25,26,27,28,29,30,31,32,33,34,35,36,37,38,39,40,41,42,43,44,45,46,47,48,49,50,51,52,53,54,55,56,57,58,59,60,61,62,63
    v_accvgpr_write_b32 a[\r], 0
    v_accvgpr_write_b32 a[64+(\r)], 0
  .endr
  v_mul_f32_e64 v81, -v80, s79
  v_mov_b32 v82, 0
  s_mov_b32 s74, 0
L_loop_%=:
  FD_STEP 0, 0, %=
  FD_STEP 1, 1, %=
  FD_STEP 0, 2, %=
  FD_STEP 1, 0, %=
  FD_STEP 0, 1, %=
  FD_STEP 1, 2, %=
  s_branch L_loop_%=
  FD_TAIL 0, 0, %=
  FD_TAIL 1, 1, %=
  FD_TAIL 0, 2, %=
  FD_TAIL 1, 0, %=
  FD_TAIL 0, 1, %=
  FD_TAIL 1, 2, %=
  FD_MASK 0, 0, %=
  FD_MASK 1, 1, %=
  FD_MASK 0, 2, %=
  FD_MASK 1, 0, %=
  FD_MASK 0, 1, %=
  FD_MASK 1, 2, %=
  FD_RARE 0, %=
  FD_RARE 1, %=
L_done_%=:
  s_waitcnt lgkmcnt(0)
  s_nop 7
  s_nop 7
  s_nop 7
  .purgem FD_WAIT
  .purgem FD_RX
  .purgem FD_TX
  .purgem FD_RD
  .purgem FD_RD6
  .purgem FD_WT2
  .purgem FD_WT
  .purgem FD_EX
  .purgem FD_EXR
  .purgem FD_SM
  .purgem FD_PM
  .purgem FD_CHECK
  .purgem FD_STEP
  .purgem FD_TAIL
  .purgem FD_MASK
  .purgem FD_RARE
)ASM"

#define CLOBBERS "v16", "v17", "v18", "v19", "v20", "v21", "v22", "v23", "v24", "v25", "v26", "v27", "v28", "v29", "v30", "v31", "v32", "v33", "v34", "v35", "v36", "v37", "v38", "v39", "v40", "v41", "v42", "v43", "v44", "v45", "v46", "v47", "v48", "v49", "v50", "v51", "v52", "v53", "v54", "v55", "v56", "v57", "v58", "v59", "v60", "v61", "v62", "v63", "v64", "v65", "v66", "v67", "v68", "v69", "v70", "v71", "v72", "v73", "v74", "v75", "v76", "v77", "v78", "v79", "v81", "v83", "v86", "v87"

__global__ __attribute__((amdgpu_flat_work_group_size(64 * kWaves, 64 * kWaves), amdgpu_waves_per_eu(1, 1))) void
fwd_d256_kernel(FwdArgs a, TileSched sched) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[kLdsBytes];
  lds_char* smem = (lds_char*)smem_raw;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, half = lane >> 5;
  const int qb = wave & 1, kh = wave >> 1;  // query block; key half of every tile
  int qtile, bh;
  sched_item(sched, blockIdx.x, qtile, bh);
  const int N = a.N;
  const size_t head_off = (size_t)bh * N * D;
  const __bf16* __restrict__ Q = (const __bf16*)a.q + head_off;
  const __bf16* __restrict__ K = (const __bf16*)a.k + head_off;
  const __bf16* __restrict__ V = (const __bf16*)a.v + head_off;
  const int nt = (N + kBlockN - 1) / kBlockN;
  // a ragged last tile is loaded shifted back to end at key N-1
  const uint32_t last_tile_bytes = (uint32_t)(N - kBlockN) * (D * 2);
  auto tile_bytes = [&](int t) { return min((uint32_t)t * (uint32_t)kTileBytes, last_tile_bytes); };
  const float c = a.scale_log2;

  RowTileCopier<D, D, kBlockN, kWaves> cp;
  cp.init(wave, lane);
  const uint32_t ring = (uint32_t)(uintptr_t)smem;
  // prologue copies, in the order the first step waits for them: K0 K1 V0 V1
  cp.copy_at(K, tile_bytes(0), smem);
  cp.copy_at(K, tile_bytes(min(1, nt - 1)), smem + kTileBytes);
  cp.copy_at(V, tile_bytes(0), smem + kVRing);
  cp.copy_at(V, tile_bytes(min(1, nt - 1)), smem + kVRing + kTileBytes);

  // Q^T fragments of this wave's rows: query column l32, d = ds*16 + half*8 .. +7
  const int q0 = qtile * kRows + qb * 32;
  const int qrow = min(q0 + l32, N - 1);
  bf16x8 qf[16];
#pragma unroll
  for (int ds = 0; ds < 16; ++ds) qf[ds] = *(const bf16x8*)(Q + (size_t)qrow * D + ds * 16 + half * 8);

  // per-lane LDS addresses: K fragments (key row kh*32 + l32) and the two
  // transposed reads of V^T fragments (key rows kh*32 + half*4 + j16/4 and
  // +8; d block db at XOR 64 (db mod 4), +256 bytes for db >= 4)
  i32x8 kaddr;
#pragma unroll
  for (int i = 0; i < 8; ++i) kaddr[i] = (int)ring + lds_off_bytes<D>(kh * 32 + l32, 2 * i + half);
  i32x16 vaddr;
  {
    const int g = lane >> 4, j16 = lane & 15;
    const int r1 = kh * 32 + half * 4 + (j16 >> 2);
    const int dcol0 = (g & 1) * 16 + (j16 & 3) * 4;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int base = (int)ring + kVRing + lds_off_bytes<D>(r1 + 8 * t, dcol0 >> 3) + (dcol0 & 7) * 2;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        vaddr[2 * q + t] = base ^ (64 * q);
        vaddr[8 + 2 * q + t] = (base ^ (64 * q)) + 2 * kTileBytes;
      }
    }
  }
  const i32x8 cpoff = {(int)cp.off[0], (int)cp.off[1], (int)cp.off[2], (int)cp.off[3],
                       (int)cp.off[4], (int)cp.off[5], (int)cp.off[6], (int)cp.off[7]};

  // tile 0: scores (K0 has landed; three tiles of copies follow it) and the
  // running max, its row max over this wave's key half
  wait_vmcnt<3 * RowTileCopier<D, D, kBlockN, kWaves>::kLoads>();
  __syncthreads();
  f32x16 s0 = {};
#pragma unroll
  for (int ds = 0; ds < 16; ++ds) {
    const bf16x8 kf =
        *(const bf16x8 __attribute__((address_space(3)))*)(smem + lds_off_bytes<D>(kh * 32 + l32, ds * 2 + half));
    s0 = mfma32(kf, qf[ds], s0);
  }
  float mx = -__builtin_inff();
#pragma unroll
  for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s0[r]);
  float m = max_halves(mx), l = 0.f;
  // the ragged last tile: its first 64 - N mod 64 keys belong to the tile
  // before; a lane masks its register offsets (r/4)*8 + r%4 below mlo
  const int ragged_tile = (N % kBlockN) ? nt - 1 : (1 << 30);
  const int mlo = (N % kBlockN ? kBlockN - N % kBlockN : 0) - kh * 32 - half * 4;
  const int ones = 0x3f803f80;

  // scalar operands of the loop, pinned to SGPRs (all are wave-uniform)
  auto sgpr = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
  auto sgpr_ptr = [](const __bf16* x) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)x);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uintptr_t)x >> 32));
    return (const __bf16*)(((uint64_t)hi << 32) | (uint64_t)lo);
  };
  const __bf16* Ks = sgpr_ptr(K);
  const __bf16* Vs = sgpr_ptr(V);
  const int nt_s = sgpr(nt), ltb_s = sgpr((int)last_tile_bytes), ntm1_s = sgpr(nt - 1), rag_s = sgpr(ragged_tile);
  const int kl_s = sgpr((int)(ring + cp.lds_wave)), vl_s = sgpr((int)(ring + kVRing + cp.lds_wave));
  const float cs = __builtin_bit_cast(float, sgpr(__builtin_bit_cast(int, c)));
  f32x32 o0, o1, o2, o3;
  int p = 0;
  asm volatile(FD_LOOP_ASM
               : "={a[0:31]}"(o0), "={a[32:63]}"(o1), "={a[64:95]}"(o2), "={a[96:127]}"(o3), "+{v80}"(m), "+{v82}"(l),
                 "+{v[0:15]}"(s0), "={s74}"(p)
               : "{a[128:131]}"(qf[0]), "{a[132:135]}"(qf[1]), "{a[136:139]}"(qf[2]), "{a[140:143]}"(qf[3]),
                 "{a[144:147]}"(qf[4]), "{a[148:151]}"(qf[5]), "{a[152:155]}"(qf[6]), "{a[156:159]}"(qf[7]),
                 "{a[160:163]}"(qf[8]), "{a[164:167]}"(qf[9]), "{a[168:171]}"(qf[10]), "{a[172:175]}"(qf[11]),
                 "{a[176:179]}"(qf[12]), "{a[180:183]}"(qf[13]), "{a[184:187]}"(qf[14]), "{a[188:191]}"(qf[15]),
                 "{v[88:95]}"(kaddr), "{v[96:111]}"(vaddr), "{v[112:119]}"(cpoff), "{v84}"(ones), "{v85}"(mlo),
                 "{s[70:71]}"(Ks), "{s[72:73]}"(Vs), "{s75}"(nt_s), "{s76}"(ltb_s), "{s77}"(kl_s), "{s78}"(vl_s),
                 "{s79}"(cs), "{s80}"(ntm1_s), "{s81}"(rag_s)
               : CLOBBERS, "s82", "s83", "s84", "s85", "s86", "s87", "s88", "s89", "s90", "s91", "m0", "vcc", "scc",
                 "memory");
  wait_vmcnt<0>();  // no direct-to-LDS copy may outlive the workgroup

  // merge of the two key halves: the second-half waves hand their running
  // max, row sums and O accumulators to the first-half wave of the same rows
  // through LDS (lane-major, conflict-free); each pair of partial results is
  // rescaled to the larger max and added
  const f32x32 ob[4] = {o0, o1, o2, o3};
  float __attribute__((address_space(3)))* xo = (float __attribute__((address_space(3)))*)smem + qb * 64 * 130 + lane;
  __syncthreads();  // every wave is done with the ring
  if (kh == 1) {
#pragma unroll
    for (int i = 0; i < 128; ++i) xo[i * 64] = ob[i >> 5][i & 31];
    xo[128 * 64] = m;
    xo[129 * 64] = l;
  }
  __syncthreads();
  if (kh == 1) return;
  const float m2 = xo[128 * 64], l2 = xo[129 * 64];
  const float mn = __builtin_fmaxf(m, m2);
  const float a1 = fast_exp2((m - mn) * c), a2 = fast_exp2((m2 - mn) * c);
  const float lt = sum_halves(l * a1 + l2 * a2);
  const float inv = 1.0f / lt;

  // ---- epilogue: O = acc / l, L = m*scale + ln l.  O^T block db, register
  // r of lane (query l32): d = db*32 + (r/4)*8 + half*4 + r%4.  The wave
  // stages its 32 x 256 bf16 block of O past the merge data (512-byte rows,
  // 16-byte chunks XOR-swizzled by row) and stores it in whole rows: a lane's
  // fragment holds 8 bytes of 32 different rows, which stored directly
  // would split every store into 32 row pieces.
  __bf16* __restrict__ O = (__bf16*)a.o + head_off;
  float* __restrict__ Lse = a.lse + (size_t)bh * N;
  lds_char* ostage = smem + 2 * 64 * 130 * 4 + qb * (32 * D * 2);
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      float v4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = db * 16 + g4 * 4 + e;
        v4[e] = (ob[i >> 5][i & 31] * a1 + xo[i * 64] * a2) * inv;
      }
      const u32x2 w = {pack_bf16_u32(v4[0], v4[1]), pack_bf16_u32(v4[2], v4[3])};
      const int chunk = db * 4 + g4;
      *(u32x2 __attribute__((address_space(3)))*)(ostage + l32 * (D * 2) + ((chunk ^ (l32 & 15)) << 4) + half * 8) = w;
    }
  if (half == 0 && q0 + l32 < N) Lse[q0 + l32] = mn * a.scale + fast_log2(lt) * kLn2;
  // back in rows: lanes 32k .. 32k+31 hold one 512-byte row
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int r = k * 2 + half, ch = l32;
    const u32x4 v4 = *(const u32x4 __attribute__((address_space(3)))*)(ostage + r * (D * 2) + ((ch ^ (r & 15)) << 4));
    const int orow = q0 + r;
    if (orow < N) *(u32x4*)(O + (size_t)orow * D + ch * 8) = v4;
  }
}

}  // namespace d256

// Square forward at D = 256 without causal masking, N >= 64 (the rest runs
// on the generic kernel).
int launch_fwd_d256(const FwdArgs& a, hipStream_t stream) {
  if (a.D != 256 || a.causal || a.N < d256::kBlockN) return -2;
  const int n_qtiles = (a.N + d256::kRows - 1) / d256::kRows;
  const TileSched sched = make_sched(n_qtiles, a.B * a.H, false);
  const long grid = (long)n_qtiles * a.B * a.H;
  hipLaunchKernelGGL(d256::fwd_d256_kernel, dim3((unsigned)grid), dim3(64 * d256::kWaves), 0, stream, a, sched);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace fa
