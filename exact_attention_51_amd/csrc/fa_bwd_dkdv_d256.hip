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

// S = A K^T over d as one accumulator chain of NS (6 <= NS <= 16) MFMAs,
// the A fragments read from LDS 6 ahead of their MFMA (one buffer each).
// The B operands (this wave's K or V rows) are held in a[0:63], fragment ds
// in a[4ds : 4ds+3].  addr[ds] is the lane's LDS byte address of fragment
// ds < 8; fragment ds >= 8 lies 256 bytes further (the swizzle permutes
// chunks within each 16-chunk half of a 512-byte row).  Compiler-scheduled,
// at 256 VGPRs this chain read one fragment at a time and waited for it.
//
// The chain also issues this wave's share of the next query tile's copy
// (cp: 4 loads of Q rows, then 4 of dO rows, from the tiles' global bases
// qg, og to LDS lq, lo + 1024 i at the copier's lane offsets), one after
// each of its first 8 MFMAs; exec = 0 leaves them out.  Issued in one burst after
// the step's barrier, the 8 loads of 1 KB stalled the wave for about 500
// cycles while the vector memory path drained them.
struct KvCopy {
  uint64_t qg, og;
  uint32_t lq, lo;
  uint64_t exec;
  uint32_t off[4];
};

template <int NS>
__device__ __forceinline__ f32x16 kv_chain(const int (&addr)[8], const f32x16& kv0, const f32x16& kv1,
                                           const f32x16& kv2, const f32x16& kv3, const KvCopy& cp) {
  static_assert(NS >= 8 && NS <= 16, "chain length");
  f32x16 acc;
  f32x4 b[6];  // fragment buffers: fragment ds in buffer ds mod 6
  asm volatile(
      // copy load n: Q rows (n < 4) or dO rows, load n mod 4 of the wave's share
      ".macro KC_LD n\n"
      "  .if ((\\n) >> 2) == 0\n"
      "    s_add_u32 m0, %[lq], ((\\n) & 3) * 1024\n"
      "  .else\n"
      "    s_add_u32 m0, %[lo], ((\\n) & 3) * 1024\n"
      "  .endif\n"
      "  s_mov_b64 exec, %[cx]\n"
      "  .if (\\n) == 0\n    global_load_lds_dwordx4 %[o0], %[qg]\n"
      "  .elseif (\\n) == 1\n    global_load_lds_dwordx4 %[o1], %[qg]\n"
      "  .elseif (\\n) == 2\n    global_load_lds_dwordx4 %[o2], %[qg]\n"
      "  .elseif (\\n) == 3\n    global_load_lds_dwordx4 %[o3], %[qg]\n"
      "  .elseif (\\n) == 4\n    global_load_lds_dwordx4 %[o0], %[og]\n"
      "  .elseif (\\n) == 5\n    global_load_lds_dwordx4 %[o1], %[og]\n"
      "  .elseif (\\n) == 6\n    global_load_lds_dwordx4 %[o2], %[og]\n"
      "  .else\n    global_load_lds_dwordx4 %[o3], %[og]\n"
      "  .endif\n"
      "  s_mov_b64 exec, -1\n"
      ".endm\n"
      // after MFMA i: load i of the 8 (the earliest issue leaves them the
      // most time to land before the next step's wait)
      ".macro KC_AT i\n"
      "  .if (\\i) < 8\n"
      "    KC_LD (\\i)\n"
      "  .endif\n"
      ".endm\n"
      "ds_read_b128 %[f0], %[a0]\n"
      "ds_read_b128 %[f1], %[a1]\n"
      "ds_read_b128 %[f2], %[a2]\n"
      "ds_read_b128 %[f3], %[a3]\n"
      "ds_read_b128 %[f4], %[a4]\n"
      "ds_read_b128 %[f5], %[a5]\n"
      ".if 0 < %[ns]\n"
      "  .if 0 + 5 < %[ns]\n    s_waitcnt lgkmcnt(5)\n"
      "  .elseif 0 + 4 < %[ns]\n    s_waitcnt lgkmcnt(4)\n"
      "  .elseif 0 + 3 < %[ns]\n    s_waitcnt lgkmcnt(3)\n"
      "  .elseif 0 + 2 < %[ns]\n    s_waitcnt lgkmcnt(2)\n"
      "  .elseif 0 + 1 < %[ns]\n    s_waitcnt lgkmcnt(1)\n"
      "  .else\n    s_waitcnt lgkmcnt(0)\n  .endif\n"
      "  v_mfma_f32_32x32x16_bf16 %[acc], %[f0], a[0:3], 0\n"
      "  KC_AT 0\n"
      "  .if 6 < %[ns]\n    ds_read_b128 %[f0], %[a6]\n  .endif\n"
      ".endif\n"
      ".if 1 < %[ns]\n"
      "  .if 1 + 5 < %[ns]\n    s_waitcnt lgkmcnt(5)\n"
      "  .elseif 1 + 4 < %[ns]\n    s_waitcnt lgkmcnt(4)\n"
      "  .elseif 1 + 3 < %[ns]\n    s_waitcnt lgkmcnt(3)\n"
      "  .elseif 1 + 2 < %[ns]\n    s_waitcnt lgkmcnt(2)\n"
      "  .elseif 1 + 1 < %[ns]\n    s_waitcnt lgkmcnt(1)\n"
      "  .else\n    s_waitcnt lgkmcnt(0)\n  .endif\n"
      "  v_mfma_f32_32x32x16_bf16 %[acc], %[f1], a[4:7], %[acc]\n"
      "  KC_AT 1\n"
      "  .if 7 < %[ns]\n    ds_read_b128 %[f1], %[a7]\n  .endif\n"
      ".endif\n"
      ".if 2 < %[ns]\n"
      "  .if 2 + 5 < %[ns]\n    s_waitcnt lgkmcnt(5)\n"
      "  .elseif 2 + 4 < %[ns]\n    s_waitcnt lgkmcnt(4)\n"
      "  .elseif 2 + 3 < %[ns]\n    s_waitcnt lgkmcnt(3)\n"
      "  .elseif 2 + 2 < %[ns]\n    s_waitcnt lgkmcnt(2)\n"
      "  .elseif 2 + 1 < %[ns]\n    s_waitcnt lgkmcnt(1)\n"
      "  .else\n    s_waitcnt lgkmcnt(0)\n  .endif\n"
      "  v_mfma_f32_32x32x16_bf16 %[acc], %[f2], a[8:11], %[acc]\n"
      "  KC_AT 2\n"
      "  .if 8 < %[ns]\n    ds_read_b128 %[f2], %[a0] offset:256\n  .endif\n"
      ".endif\n"
      ".if 3 < %[ns]\n"
      "  .if 3 + 5 < %[ns]\n    s_waitcnt lgkmcnt(5)\n"
      "  .elseif 3 + 4 < %[ns]\n    s_waitcnt lgkmcnt(4)\n"
      "  .elseif 3 + 3 < %[ns]\n    s_waitcnt lgkmcnt(3)\n"
      "  .elseif 3 + 2 < %[ns]\n    s_waitcnt lgkmcnt(2)\n"
      "  .elseif 3 + 1 < %[ns]\n    s_waitcnt lgkmcnt(1)\n"
      "  .else\n    s_waitcnt lgkmcnt(0)\n  .endif\n"
      "  v_mfma_f32_32x32x16_bf16 %[acc], %[f3], a[12:15], %[acc]\n"
      "  KC_AT 3\n"
      "  .if 9 < %[ns]\n    ds_read_b128 %[f3], %[a1] offset:256\n  .endif\n"
      ".endif\n"
      ".if 4 < %[ns]\n"
      "  .if 4 + 5 < %[ns]\n    s_waitcnt lgkmcnt(5)\n"
      "  .elseif 4 + 4 < %[ns]\n    s_waitcnt lgkmcnt(4)\n"
      "  .elseif 4 + 3 < %[ns]\n    s_waitcnt lgkmcnt(3)\n"
      "  .elseif 4 + 2 < %[ns]\n    s_waitcnt lgkmcnt(2)\n"
      "  .elseif 4 + 1 < %[ns]\n    s_waitcnt lgkmcnt(1)\n"
      "  .else\n    s_waitcnt lgkmcnt(0)\n  .endif\n"
      "  v_mfma_f32_32x32x16_bf16 %[acc], %[f4], a[16:19], %[acc]\n"
      "  KC_AT 4\n"
      "  .if 10 < %[ns]\n    ds_read_b128 %[f4], %[a2] offset:256\n  .endif\n"
      ".endif\n"
      ".if 5 < %[ns]\n"
      "  .if 5 + 5 < %[ns]\n    s_waitcnt lgkmcnt(5)\n"
      "  .elseif 5 + 4 < %[ns]\n    s_waitcnt lgkmcnt(4)\n"
      "  .elseif 5 + 3 < %[ns]\n    s_waitcnt lgkmcnt(3)\n"
      "  .elseif 5 + 2 < %[ns]\n    s_waitcnt lgkmcnt(2)\n"
      "  .elseif 5 + 1 < %[ns]\n    s_waitcnt lgkmcnt(1)\n"
      "  .else\n    s_waitcnt lgkmcnt(0)\n  .endif\n"
      "  v_mfma_f32_32x32x16_bf16 %[acc], %[f5], a[20:23], %[acc]\n"
      "  KC_AT 5\n"
      "  .if 11 < %[ns]\n    ds_read_b128 %[f5], %[a3] offset:256\n  .endif\n"
      ".endif\n"
      ".if 6 < %[ns]\n"
      "  .if 6 + 5 < %[ns]\n    s_waitcnt lgkmcnt(5)\n"
      "  .elseif 6 + 4 < %[ns]\n    s_waitcnt lgkmcnt(4)\n"
      "  .elseif 6 + 3 < %[ns]\n    s_waitcnt lgkmcnt(3)\n"
      "  .elseif 6 + 2 < %[ns]\n    s_waitcnt lgkmcnt(2)\n"
      "  .elseif 6 + 1 < %[ns]\n    s_waitcnt lgkmcnt(1)\n"
      "  .else\n    s_waitcnt lgkmcnt(0)\n  .endif\n"
      "  v_mfma_f32_32x32x16_bf16 %[acc], %[f0], a[24:27], %[acc]\n"
      "  KC_AT 6\n"
      "  .if 12 < %[ns]\n    ds_read_b128 %[f0], %[a4] offset:256\n  .endif\n"
      ".endif\n"
      ".if 7 < %[ns]\n"
      "  .if 7 + 5 < %[ns]\n    s_waitcnt lgkmcnt(5)\n"
      "  .elseif 7 + 4 < %[ns]\n    s_waitcnt lgkmcnt(4)\n"
      "  .elseif 7 + 3 < %[ns]\n    s_waitcnt lgkmcnt(3)\n"
      "  .elseif 7 + 2 < %[ns]\n    s_waitcnt lgkmcnt(2)\n"
      "  .elseif 7 + 1 < %[ns]\n    s_waitcnt lgkmcnt(1)\n"
      "  .else\n    s_waitcnt lgkmcnt(0)\n  .endif\n"
      "  v_mfma_f32_32x32x16_bf16 %[acc], %[f1], a[28:31], %[acc]\n"
      "  KC_AT 7\n"
      "  .if 13 < %[ns]\n    ds_read_b128 %[f1], %[a5] offset:256\n  .endif\n"
      ".endif\n"
      ".if 8 < %[ns]\n"
      "  .if 8 + 5 < %[ns]\n    s_waitcnt lgkmcnt(5)\n"
      "  .elseif 8 + 4 < %[ns]\n    s_waitcnt lgkmcnt(4)\n"
      "  .elseif 8 + 3 < %[ns]\n    s_waitcnt lgkmcnt(3)\n"
      "  .elseif 8 + 2 < %[ns]\n    s_waitcnt lgkmcnt(2)\n"
      "  .elseif 8 + 1 < %[ns]\n    s_waitcnt lgkmcnt(1)\n"
      "  .else\n    s_waitcnt lgkmcnt(0)\n  .endif\n"
      "  v_mfma_f32_32x32x16_bf16 %[acc], %[f2], a[32:35], %[acc]\n"
      "  KC_AT 8\n"
      "  .if 14 < %[ns]\n    ds_read_b128 %[f2], %[a6] offset:256\n  .endif\n"
      ".endif\n"
      ".if 9 < %[ns]\n"
      "  .if 9 + 5 < %[ns]\n    s_waitcnt lgkmcnt(5)\n"
      "  .elseif 9 + 4 < %[ns]\n    s_waitcnt lgkmcnt(4)\n"
      "  .elseif 9 + 3 < %[ns]\n    s_waitcnt lgkmcnt(3)\n"
      "  .elseif 9 + 2 < %[ns]\n    s_waitcnt lgkmcnt(2)\n"
      "  .elseif 9 + 1 < %[ns]\n    s_waitcnt lgkmcnt(1)\n"
      "  .else\n    s_waitcnt lgkmcnt(0)\n  .endif\n"
      "  v_mfma_f32_32x32x16_bf16 %[acc], %[f3], a[36:39], %[acc]\n"
      "  KC_AT 9\n"
      "  .if 15 < %[ns]\n    ds_read_b128 %[f3], %[a7] offset:256\n  .endif\n"
      ".endif\n"
      ".if 10 < %[ns]\n"
      "  .if 10 + 5 < %[ns]\n    s_waitcnt lgkmcnt(5)\n"
      "  .elseif 10 + 4 < %[ns]\n    s_waitcnt lgkmcnt(4)\n"
      "  .elseif 10 + 3 < %[ns]\n    s_waitcnt lgkmcnt(3)\n"
      "  .elseif 10 + 2 < %[ns]\n    s_waitcnt lgkmcnt(2)\n"
      "  .elseif 10 + 1 < %[ns]\n    s_waitcnt lgkmcnt(1)\n"
      "  .else\n    s_waitcnt lgkmcnt(0)\n  .endif\n"
      "  v_mfma_f32_32x32x16_bf16 %[acc], %[f4], a[40:43], %[acc]\n"
      "  KC_AT 10\n"
      ".endif\n"
      ".if 11 < %[ns]\n"
      "  .if 11 + 5 < %[ns]\n    s_waitcnt lgkmcnt(5)\n"
      "  .elseif 11 + 4 < %[ns]\n    s_waitcnt lgkmcnt(4)\n"
      "  .elseif 11 + 3 < %[ns]\n    s_waitcnt lgkmcnt(3)\n"
      "  .elseif 11 + 2 < %[ns]\n    s_waitcnt lgkmcnt(2)\n"
      "  .elseif 11 + 1 < %[ns]\n    s_waitcnt lgkmcnt(1)\n"
      "  .else\n    s_waitcnt lgkmcnt(0)\n  .endif\n"
      "  v_mfma_f32_32x32x16_bf16 %[acc], %[f5], a[44:47], %[acc]\n"
      "  KC_AT 11\n"
      ".endif\n"
      ".if 12 < %[ns]\n"
      "  .if 12 + 5 < %[ns]\n    s_waitcnt lgkmcnt(5)\n"
      "  .elseif 12 + 4 < %[ns]\n    s_waitcnt lgkmcnt(4)\n"
      "  .elseif 12 + 3 < %[ns]\n    s_waitcnt lgkmcnt(3)\n"
      "  .elseif 12 + 2 < %[ns]\n    s_waitcnt lgkmcnt(2)\n"
      "  .elseif 12 + 1 < %[ns]\n    s_waitcnt lgkmcnt(1)\n"
      "  .else\n    s_waitcnt lgkmcnt(0)\n  .endif\n"
      "  v_mfma_f32_32x32x16_bf16 %[acc], %[f0], a[48:51], %[acc]\n"
      "  KC_AT 12\n"
      ".endif\n"
      ".if 13 < %[ns]\n"
      "  .if 13 + 5 < %[ns]\n    s_waitcnt lgkmcnt(5)\n"
      "  .elseif 13 + 4 < %[ns]\n    s_waitcnt lgkmcnt(4)\n"
      "  .elseif 13 + 3 < %[ns]\n    s_waitcnt lgkmcnt(3)\n"
      "  .elseif 13 + 2 < %[ns]\n    s_waitcnt lgkmcnt(2)\n"
      "  .elseif 13 + 1 < %[ns]\n    s_waitcnt lgkmcnt(1)\n"
      "  .else\n    s_waitcnt lgkmcnt(0)\n  .endif\n"
      "  v_mfma_f32_32x32x16_bf16 %[acc], %[f1], a[52:55], %[acc]\n"
      "  KC_AT 13\n"
      ".endif\n"
      ".if 14 < %[ns]\n"
      "  .if 14 + 5 < %[ns]\n    s_waitcnt lgkmcnt(5)\n"
      "  .elseif 14 + 4 < %[ns]\n    s_waitcnt lgkmcnt(4)\n"
      "  .elseif 14 + 3 < %[ns]\n    s_waitcnt lgkmcnt(3)\n"
      "  .elseif 14 + 2 < %[ns]\n    s_waitcnt lgkmcnt(2)\n"
      "  .elseif 14 + 1 < %[ns]\n    s_waitcnt lgkmcnt(1)\n"
      "  .else\n    s_waitcnt lgkmcnt(0)\n  .endif\n"
      "  v_mfma_f32_32x32x16_bf16 %[acc], %[f2], a[56:59], %[acc]\n"
      "  KC_AT 14\n"
      ".endif\n"
      ".if 15 < %[ns]\n"
      "  .if 15 + 5 < %[ns]\n    s_waitcnt lgkmcnt(5)\n"
      "  .elseif 15 + 4 < %[ns]\n    s_waitcnt lgkmcnt(4)\n"
      "  .elseif 15 + 3 < %[ns]\n    s_waitcnt lgkmcnt(3)\n"
      "  .elseif 15 + 2 < %[ns]\n    s_waitcnt lgkmcnt(2)\n"
      "  .elseif 15 + 1 < %[ns]\n    s_waitcnt lgkmcnt(1)\n"
      "  .else\n    s_waitcnt lgkmcnt(0)\n  .endif\n"
      "  v_mfma_f32_32x32x16_bf16 %[acc], %[f3], a[60:63], %[acc]\n"
      "  KC_AT 15\n"
      ".endif\n"
      "s_nop 7\n"
      "s_nop 7\n"
      "s_nop 7\n"  // the MFMA results may be read by vector instructions right after
      ".purgem KC_LD\n"
      ".purgem KC_AT\n"
      : [acc] "=&v"(acc), [f0] "=&v"(b[0]), [f1] "=&v"(b[1]), [f2] "=&v"(b[2]), [f3] "=&v"(b[3]), [f4] "=&v"(b[4]), [f5] "=&v"(b[5])
      : [a0] "v"(addr[0]), [a1] "v"(addr[1]), [a2] "v"(addr[2]), [a3] "v"(addr[3]), [a4] "v"(addr[4]),
        [a5] "v"(addr[5]), [a6] "v"(addr[6]), [a7] "v"(addr[7]), [ns] "i"(NS), "{a[0:15]}"(kv0), "{a[16:31]}"(kv1),
        "{a[32:47]}"(kv2), "{a[48:63]}"(kv3), [qg] "s"(cp.qg), [og] "s"(cp.og), [lq] "s"(cp.lq), [lo] "s"(cp.lo),
        [cx] "s"(cp.exec), [o0] "v"(cp.off[0]), [o1] "v"(cp.off[1]), [o2] "v"(cp.off[2]), [o3] "v"(cp.off[3])
      : "memory", "m0", "exec", "scc");
  return acc;
}

// dV^T += dO^T P and dK^T += Q^T dS over NB 32-column blocks, the Oᵀ and Qᵀ
// operands read transposed from the query tile 3 fragments ahead of their
// MFMA (fragment buffers v[240:255], second-read addresses in
// v236..v239).  addr[i] is the lane's address of block i's first
// transposed read in the Q tile (cc = 0); the dO tile lies 16384 bytes
// further, the second 16 queries (cc = 1) 8192, the read 8 rows down d2.
template <int NB>
__device__ __forceinline__ void kv_tr_chain(const int (&addr)[4], int d2, const bf16x8& pp0, const bf16x8& pp1,
                                            const bf16x8& ds0, const bf16x8& ds1, f32x16& dv0, f32x16& dv1,
                                            f32x16& dv2, f32x16& dv3, f32x16& dk0, f32x16& dk1, f32x16& dk2,
                                            f32x16& dk3) {
  static_assert(NB >= 1 && NB <= 4, "blocks");
  f32x16 junk;
  f32x4 junk2;
  asm volatile(
      ".if 0 < 4 * %[nb]\n"
      "  ds_read_b64_tr_b16 v[240:241], %[a0] offset:16384\n"
      "  v_add_u32 v236, %[a0], %[d2]\n"
      "  ds_read_b64_tr_b16 v[242:243], v236 offset:16384\n"
      ".endif\n"
      ".if 1 < 4 * %[nb]\n"
      "  ds_read_b64_tr_b16 v[244:245], %[a0] offset:0\n"
      "  v_add_u32 v237, %[a0], %[d2]\n"
      "  ds_read_b64_tr_b16 v[246:247], v237 offset:0\n"
      ".endif\n"
      ".if 2 < 4 * %[nb]\n"
      "  ds_read_b64_tr_b16 v[248:249], %[a0] offset:24576\n"
      "  v_add_u32 v238, %[a0], %[d2]\n"
      "  ds_read_b64_tr_b16 v[250:251], v238 offset:24576\n"
      ".endif\n"
      ".if 3 < 4 * %[nb]\n"
      "  ds_read_b64_tr_b16 v[252:253], %[a0] offset:8192\n"
      "  v_add_u32 v239, %[a0], %[d2]\n"
      "  ds_read_b64_tr_b16 v[254:255], v239 offset:8192\n"
      ".endif\n"
      ".if 0 < 4 * %[nb]\n"
      "  .if 0 + 3 < 4 * %[nb]\n    s_waitcnt lgkmcnt(6)\n"
      "  .elseif 0 + 2 < 4 * %[nb]\n    s_waitcnt lgkmcnt(4)\n"
      "  .elseif 0 + 1 < 4 * %[nb]\n    s_waitcnt lgkmcnt(2)\n"
      "  .else\n    s_waitcnt lgkmcnt(0)\n  .endif\n"
      "  v_mfma_f32_32x32x16_bf16 %[dv0], v[240:243], %[pp0], %[dv0]\n"
      "  .if 4 < 4 * %[nb]\n"
      "    ds_read_b64_tr_b16 v[240:241], %[a1] offset:16384\n"
      "    v_add_u32 v236, %[a1], %[d2]\n"
      "    ds_read_b64_tr_b16 v[242:243], v236 offset:16384\n"
      "  .endif\n"
      ".endif\n"
      ".if 1 < 4 * %[nb]\n"
      "  .if 1 + 3 < 4 * %[nb]\n    s_waitcnt lgkmcnt(6)\n"
      "  .elseif 1 + 2 < 4 * %[nb]\n    s_waitcnt lgkmcnt(4)\n"
      "  .elseif 1 + 1 < 4 * %[nb]\n    s_waitcnt lgkmcnt(2)\n"
      "  .else\n    s_waitcnt lgkmcnt(0)\n  .endif\n"
      "  v_mfma_f32_32x32x16_bf16 %[dk0], v[244:247], %[ds0], %[dk0]\n"
      "  .if 5 < 4 * %[nb]\n"
      "    ds_read_b64_tr_b16 v[244:245], %[a1] offset:0\n"
      "    v_add_u32 v237, %[a1], %[d2]\n"
      "    ds_read_b64_tr_b16 v[246:247], v237 offset:0\n"
      "  .endif\n"
      ".endif\n"
      ".if 2 < 4 * %[nb]\n"
      "  .if 2 + 3 < 4 * %[nb]\n    s_waitcnt lgkmcnt(6)\n"
      "  .elseif 2 + 2 < 4 * %[nb]\n    s_waitcnt lgkmcnt(4)\n"
      "  .elseif 2 + 1 < 4 * %[nb]\n    s_waitcnt lgkmcnt(2)\n"
      "  .else\n    s_waitcnt lgkmcnt(0)\n  .endif\n"
      "  v_mfma_f32_32x32x16_bf16 %[dv0], v[248:251], %[pp1], %[dv0]\n"
      "  .if 6 < 4 * %[nb]\n"
      "    ds_read_b64_tr_b16 v[248:249], %[a1] offset:24576\n"
      "    v_add_u32 v238, %[a1], %[d2]\n"
      "    ds_read_b64_tr_b16 v[250:251], v238 offset:24576\n"
      "  .endif\n"
      ".endif\n"
      ".if 3 < 4 * %[nb]\n"
      "  .if 3 + 3 < 4 * %[nb]\n    s_waitcnt lgkmcnt(6)\n"
      "  .elseif 3 + 2 < 4 * %[nb]\n    s_waitcnt lgkmcnt(4)\n"
      "  .elseif 3 + 1 < 4 * %[nb]\n    s_waitcnt lgkmcnt(2)\n"
      "  .else\n    s_waitcnt lgkmcnt(0)\n  .endif\n"
      "  v_mfma_f32_32x32x16_bf16 %[dk0], v[252:255], %[ds1], %[dk0]\n"
      "  .if 7 < 4 * %[nb]\n"
      "    ds_read_b64_tr_b16 v[252:253], %[a1] offset:8192\n"
      "    v_add_u32 v239, %[a1], %[d2]\n"
      "    ds_read_b64_tr_b16 v[254:255], v239 offset:8192\n"
      "  .endif\n"
      ".endif\n"
      ".if 4 < 4 * %[nb]\n"
      "  .if 4 + 3 < 4 * %[nb]\n    s_waitcnt lgkmcnt(6)\n"
      "  .elseif 4 + 2 < 4 * %[nb]\n    s_waitcnt lgkmcnt(4)\n"
      "  .elseif 4 + 1 < 4 * %[nb]\n    s_waitcnt lgkmcnt(2)\n"
      "  .else\n    s_waitcnt lgkmcnt(0)\n  .endif\n"
      "  v_mfma_f32_32x32x16_bf16 %[dv1], v[240:243], %[pp0], %[dv1]\n"
      "  .if 8 < 4 * %[nb]\n"
      "    ds_read_b64_tr_b16 v[240:241], %[a2] offset:16384\n"
      "    v_add_u32 v236, %[a2], %[d2]\n"
      "    ds_read_b64_tr_b16 v[242:243], v236 offset:16384\n"
      "  .endif\n"
      ".endif\n"
      ".if 5 < 4 * %[nb]\n"
      "  .if 5 + 3 < 4 * %[nb]\n    s_waitcnt lgkmcnt(6)\n"
      "  .elseif 5 + 2 < 4 * %[nb]\n    s_waitcnt lgkmcnt(4)\n"
      "  .elseif 5 + 1 < 4 * %[nb]\n    s_waitcnt lgkmcnt(2)\n"
      "  .else\n    s_waitcnt lgkmcnt(0)\n  .endif\n"
      "  v_mfma_f32_32x32x16_bf16 %[dk1], v[244:247], %[ds0], %[dk1]\n"
      "  .if 9 < 4 * %[nb]\n"
      "    ds_read_b64_tr_b16 v[244:245], %[a2] offset:0\n"
      "    v_add_u32 v237, %[a2], %[d2]\n"
      "    ds_read_b64_tr_b16 v[246:247], v237 offset:0\n"
      "  .endif\n"
      ".endif\n"
      ".if 6 < 4 * %[nb]\n"
      "  .if 6 + 3 < 4 * %[nb]\n    s_waitcnt lgkmcnt(6)\n"
      "  .elseif 6 + 2 < 4 * %[nb]\n    s_waitcnt lgkmcnt(4)\n"
      "  .elseif 6 + 1 < 4 * %[nb]\n    s_waitcnt lgkmcnt(2)\n"
      "  .else\n    s_waitcnt lgkmcnt(0)\n  .endif\n"
      "  v_mfma_f32_32x32x16_bf16 %[dv1], v[248:251], %[pp1], %[dv1]\n"
      "  .if 10 < 4 * %[nb]\n"
      "    ds_read_b64_tr_b16 v[248:249], %[a2] offset:24576\n"
      "    v_add_u32 v238, %[a2], %[d2]\n"
      "    ds_read_b64_tr_b16 v[250:251], v238 offset:24576\n"
      "  .endif\n"
      ".endif\n"
      ".if 7 < 4 * %[nb]\n"
      "  .if 7 + 3 < 4 * %[nb]\n    s_waitcnt lgkmcnt(6)\n"
      "  .elseif 7 + 2 < 4 * %[nb]\n    s_waitcnt lgkmcnt(4)\n"
      "  .elseif 7 + 1 < 4 * %[nb]\n    s_waitcnt lgkmcnt(2)\n"
      "  .else\n    s_waitcnt lgkmcnt(0)\n  .endif\n"
      "  v_mfma_f32_32x32x16_bf16 %[dk1], v[252:255], %[ds1], %[dk1]\n"
      "  .if 11 < 4 * %[nb]\n"
      "    ds_read_b64_tr_b16 v[252:253], %[a2] offset:8192\n"
      "    v_add_u32 v239, %[a2], %[d2]\n"
      "    ds_read_b64_tr_b16 v[254:255], v239 offset:8192\n"
      "  .endif\n"
      ".endif\n"
      ".if 8 < 4 * %[nb]\n"
      "  .if 8 + 3 < 4 * %[nb]\n    s_waitcnt lgkmcnt(6)\n"
      "  .elseif 8 + 2 < 4 * %[nb]\n    s_waitcnt lgkmcnt(4)\n"
      "  .elseif 8 + 1 < 4 * %[nb]\n    s_waitcnt lgkmcnt(2)\n"
      "  .else\n    s_waitcnt lgkmcnt(0)\n  .endif\n"
      "  v_mfma_f32_32x32x16_bf16 %[dv2], v[240:243], %[pp0], %[dv2]\n"
      "  .if 12 < 4 * %[nb]\n"
      "    ds_read_b64_tr_b16 v[240:241], %[a3] offset:16384\n"
      "    v_add_u32 v236, %[a3], %[d2]\n"
      "    ds_read_b64_tr_b16 v[242:243], v236 offset:16384\n"
      "  .endif\n"
      ".endif\n"
      ".if 9 < 4 * %[nb]\n"
      "  .if 9 + 3 < 4 * %[nb]\n    s_waitcnt lgkmcnt(6)\n"
      "  .elseif 9 + 2 < 4 * %[nb]\n    s_waitcnt lgkmcnt(4)\n"
      "  .elseif 9 + 1 < 4 * %[nb]\n    s_waitcnt lgkmcnt(2)\n"
      "  .else\n    s_waitcnt lgkmcnt(0)\n  .endif\n"
      "  v_mfma_f32_32x32x16_bf16 %[dk2], v[244:247], %[ds0], %[dk2]\n"
      "  .if 13 < 4 * %[nb]\n"
      "    ds_read_b64_tr_b16 v[244:245], %[a3] offset:0\n"
      "    v_add_u32 v237, %[a3], %[d2]\n"
      "    ds_read_b64_tr_b16 v[246:247], v237 offset:0\n"
      "  .endif\n"
      ".endif\n"
      ".if 10 < 4 * %[nb]\n"
      "  .if 10 + 3 < 4 * %[nb]\n    s_waitcnt lgkmcnt(6)\n"
      "  .elseif 10 + 2 < 4 * %[nb]\n    s_waitcnt lgkmcnt(4)\n"
      "  .elseif 10 + 1 < 4 * %[nb]\n    s_waitcnt lgkmcnt(2)\n"
      "  .else\n    s_waitcnt lgkmcnt(0)\n  .endif\n"
      "  v_mfma_f32_32x32x16_bf16 %[dv2], v[248:251], %[pp1], %[dv2]\n"
      "  .if 14 < 4 * %[nb]\n"
      "    ds_read_b64_tr_b16 v[248:249], %[a3] offset:24576\n"
      "    v_add_u32 v238, %[a3], %[d2]\n"
      "    ds_read_b64_tr_b16 v[250:251], v238 offset:24576\n"
      "  .endif\n"
      ".endif\n"
      ".if 11 < 4 * %[nb]\n"
      "  .if 11 + 3 < 4 * %[nb]\n    s_waitcnt lgkmcnt(6)\n"
      "  .elseif 11 + 2 < 4 * %[nb]\n    s_waitcnt lgkmcnt(4)\n"
      "  .elseif 11 + 1 < 4 * %[nb]\n    s_waitcnt lgkmcnt(2)\n"
      "  .else\n    s_waitcnt lgkmcnt(0)\n  .endif\n"
      "  v_mfma_f32_32x32x16_bf16 %[dk2], v[252:255], %[ds1], %[dk2]\n"
      "  .if 15 < 4 * %[nb]\n"
      "    ds_read_b64_tr_b16 v[252:253], %[a3] offset:8192\n"
      "    v_add_u32 v239, %[a3], %[d2]\n"
      "    ds_read_b64_tr_b16 v[254:255], v239 offset:8192\n"
      "  .endif\n"
      ".endif\n"
      ".if 12 < 4 * %[nb]\n"
      "  .if 12 + 3 < 4 * %[nb]\n    s_waitcnt lgkmcnt(6)\n"
      "  .elseif 12 + 2 < 4 * %[nb]\n    s_waitcnt lgkmcnt(4)\n"
      "  .elseif 12 + 1 < 4 * %[nb]\n    s_waitcnt lgkmcnt(2)\n"
      "  .else\n    s_waitcnt lgkmcnt(0)\n  .endif\n"
      "  v_mfma_f32_32x32x16_bf16 %[dv3], v[240:243], %[pp0], %[dv3]\n"
      ".endif\n"
      ".if 13 < 4 * %[nb]\n"
      "  .if 13 + 3 < 4 * %[nb]\n    s_waitcnt lgkmcnt(6)\n"
      "  .elseif 13 + 2 < 4 * %[nb]\n    s_waitcnt lgkmcnt(4)\n"
      "  .elseif 13 + 1 < 4 * %[nb]\n    s_waitcnt lgkmcnt(2)\n"
      "  .else\n    s_waitcnt lgkmcnt(0)\n  .endif\n"
      "  v_mfma_f32_32x32x16_bf16 %[dk3], v[244:247], %[ds0], %[dk3]\n"
      ".endif\n"
      ".if 14 < 4 * %[nb]\n"
      "  .if 14 + 3 < 4 * %[nb]\n    s_waitcnt lgkmcnt(6)\n"
      "  .elseif 14 + 2 < 4 * %[nb]\n    s_waitcnt lgkmcnt(4)\n"
      "  .elseif 14 + 1 < 4 * %[nb]\n    s_waitcnt lgkmcnt(2)\n"
      "  .else\n    s_waitcnt lgkmcnt(0)\n  .endif\n"
      "  v_mfma_f32_32x32x16_bf16 %[dv3], v[248:251], %[pp1], %[dv3]\n"
      ".endif\n"
      ".if 15 < 4 * %[nb]\n"
      "  .if 15 + 3 < 4 * %[nb]\n    s_waitcnt lgkmcnt(6)\n"
      "  .elseif 15 + 2 < 4 * %[nb]\n    s_waitcnt lgkmcnt(4)\n"
      "  .elseif 15 + 1 < 4 * %[nb]\n    s_waitcnt lgkmcnt(2)\n"
      "  .else\n    s_waitcnt lgkmcnt(0)\n  .endif\n"
      "  v_mfma_f32_32x32x16_bf16 %[dk3], v[252:255], %[ds1], %[dk3]\n"
      ".endif\n"
      "s_nop 7\n"
      "s_nop 7\n"
      "s_nop 7\n"  // the MFMA results may be read by vector instructions right after
      : [dv0] "+v"(dv0), [dv1] "+v"(dv1), [dv2] "+v"(dv2), [dv3] "+v"(dv3), [dk0] "+v"(dk0), [dk1] "+v"(dk1),
        [dk2] "+v"(dk2), [dk3] "+v"(dk3), "=&{v[240:255]}"(junk), "=&{v[236:239]}"(junk2)
      : [a0] "v"(addr[0]), [a1] "v"(addr[1]), [a2] "v"(addr[2]), [a3] "v"(addr[3]), [d2] "v"(d2), [pp0] "v"(pp0),
        [pp1] "v"(pp1), [ds0] "v"(ds0), [ds1] "v"(ds1), [nb] "i"(NB)
      : "memory");
}

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

  // this wave's half of dK^T and dV^T: d blocks dh*kHalfBlocks .. (those below kDBlocks)
  f32x16 dk[kHalfBlocks], dv[kHalfBlocks];
#pragma unroll
  for (int i = 0; i < kHalfBlocks; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[i][r] = dv[i][r] = 0.f;
  const float c = a.scale_log2;
  // K (S-forming wave) or V (dP-forming wave) of this wave's keys as B
  // operands: key column l32, d = ds*16 + half*8 + 0..7
  // (held as four 16-register groups, fragment ds at registers 4*(ds mod 4) of group ds/4)
  f32x16 kvg[4];
  {
    const __bf16* __restrict__ src = dh == 0 ? K : V;
    const int crow = key < N ? key : N - 1;
#pragma unroll
    for (int ds = 0; ds < 16; ++ds) {
      const bf16x8 f = ds < kDSteps ? *(const bf16x8*)(src + (size_t)crow * D + ds * 16 + half * 8) : bf16x8{};
      const f32x4 f4 = __builtin_bit_cast(f32x4, f);
#pragma unroll
      for (int i = 0; i < 4; ++i) kvg[ds >> 2][(ds & 3) * 4 + i] = f4[i];
    }
  }
  // the lane's byte offsets of fragments 0..7 of a row-major tile row l32
  int roff[8];
#pragma unroll
  for (int ds = 0; ds < 8; ++ds) roff[ds] = lds_off_bytes<DP>(l32, ds * 2 + half);
  // the lane's byte offsets of the first transposed read of d block
  // dh*kHalfBlocks + i (queries 0..15 of a tile), and of its second read
  // relative to the first (the same for every block)
  int troff[4];
  int trd2;
  {
    const int g = lane >> 4, j16 = lane & 15;
    const int r1 = half * 4 + (j16 >> 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int dcol = (dh * kHalfBlocks + i) * 32 + (g & 1) * 16 + (j16 & 3) * 4;
      troff[i] = lds_off_bytes<DP>(r1, dcol >> 3) + (dcol & 7) * 2;
    }
    const int dcol0 = (dh * kHalfBlocks) * 32 + (g & 1) * 16 + (j16 & 3) * 4;
    trd2 = lds_off_bytes<DP>(r1 + 8, dcol0 >> 3) - lds_off_bytes<DP>(r1, dcol0 >> 3);
  }

  // does key group kgrp see any query of tile t?
  auto tile_work = [&](int t) { return group_active && !(CAUSAL && t * C::kQTile + C::kQTile - 1 < wk0); };

  for (int t = t_begin; t <= n_qtiles; ++t) {
    // publishes tile t (loaded last step) and the exchange of tile t-1
    wait_vmcnt<0>();
    __syncthreads();
    // tile t+1 into the slot of tile t-2, finished last step: its Q and dO
    // rows from inside this wave's part-1 chain (a whole tile and a chain to
    // run), else here
    const bool part1 = t < n_qtiles && tile_work(t);
    KvCopy kc = {0, 0, 0, 0, 0, {cp.off[0], cp.off[1], cp.off[2], cp.off[3]}};
    if (t + 1 < n_qtiles) {
      const int sl1 = (t + 1) % 3, row1 = (t + 1) * C::kQTile;
      if (part1 && row1 + C::kQTile <= N) {
        kc.qg = (uint64_t)(uintptr_t)(Q + (size_t)row1 * D);
        kc.og = (uint64_t)(uintptr_t)(dO + (size_t)row1 * D);
        kc.lq = (uint32_t)(uintptr_t)qbuf(sl1) + cp.lds_wave;
        kc.lo = (uint32_t)(uintptr_t)obuf(sl1) + cp.lds_wave;
        kc.exec = ~0ull;
      } else {
        load_rows(t + 1);
      }
      load_stats(t + 1);
    }

    // 1. tile t: S = Q_t K^T (dh = 0) or dP = dO_t V^T (dh = 1), to the exchange
    if (t < n_qtiles && tile_work(t)) {
      const int sl = t % 3, xb = t & 1, tq0 = t * C::kQTile;
      const lds_char* at = dh == 0 ? qbuf(sl) : obuf(sl);
      int addr[8];
      const int tb = (int)(uint32_t)(uintptr_t)at;
#pragma unroll
      for (int ds = 0; ds < 8; ++ds) addr[ds] = tb + roff[ds];
      // L of the lane's 16 queries (four runs of four consecutive rows), read
      // before the chain so that its latency overlaps the MFMAs
      float lq[16];
      if (dh == 0) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 l4 = *(const f32x4 __attribute__((address_space(3)))*)(lbuf(sl) + 4 * (g * 8 + half * 4));
#pragma unroll
          for (int i = 0; i < 4; ++i) lq[g * 4 + i] = l4[i];
        }
      }
      f32x16 mine = kv_chain<kDSteps>(addr, kvg[0], kvg[1], kvg[2], kvg[3], kc);
      if (dh == 0) {  // P = exp(S - L), masked; queries of register r: (r/4)*8 + half*4 + r%4
        const bool masked = (CAUSAL && tq0 < wk0 + 31) || (tq0 + C::kQTile > N);
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
      int taddr[4];
      const int qb0 = (int)(uint32_t)(uintptr_t)qbuf(sl);
#pragma unroll
      for (int i = 0; i < 4; ++i) taddr[i] = qb0 + troff[i];
      if constexpr (kHalfBlocks == 4) {
        kv_tr_chain<4>(taddr, trd2, ppk[0], ppk[1], dspk[0], dspk[1], dv[0], dv[1], dv[2], dv[3], dk[0], dk[1], dk[2],
                       dk[3]);
      } else {
        // D = 160: blocks 0..2 (half 0) or 3..4 (half 1); the unused operand
        // slots take scratch accumulators (no two operands may name one variable)
        f32x16 sv0 = {}, sk0 = {}, sv1 = {}, sk1 = {};
        if (dh == 0)
          kv_tr_chain<3>(taddr, trd2, ppk[0], ppk[1], dspk[0], dspk[1], dv[0], dv[1], dv[2], sv0, dk[0], dk[1], dk[2],
                         sk0);
        else
          kv_tr_chain<2>(taddr, trd2, ppk[0], ppk[1], dspk[0], dspk[1], dv[0], dv[1], sv0, sv1, dk[0], dk[1], sk0,
                         sk1);
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
