// fa_device.h -- device primitives shared by the gfx950 attention kernels.
//
// Everything here is written for CDNA4 (gfx950) and wave64 only: bf16 MFMA
// 32x32x16 with float32 accumulators, the LDS transpose read
// ds_read_b64_tr_b16, direct global->LDS loads of 16 bytes per lane and the
// cross-half lane swap v_permlane32_swap.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(8))) short s16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef s16x4 __attribute__((address_space(3))) * lds_s16x4_ptr;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// ---------------------------------------------------------------- MFMA
//
// v_mfma_f32_32x32x16_bf16, C[32x32] += A[32x16] * B[16x32].  Lane l holds
//   A: row m = l % 32, k = (l / 32) * 8 + i    (i = 0..7)
//   B: col n = l % 32, k = (l / 32) * 8 + i
//   C: acc[r] = C[(r / 4) * 8 + (l / 32) * 4 + r % 4][l % 32]
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ bf16x2 pack_bf16(float lo, float hi) {
  f32x2 f = {lo, hi};
  return __builtin_convertvector(f, bf16x2);  // v_cvt_pk_bf16_f32, round to nearest even
}

__device__ __forceinline__ uint32_t pack_bf16_u32(float lo, float hi) {
  bf16x2 p = pack_bf16(lo, hi);
  return __builtin_bit_cast(uint32_t, p);
}

// Four packed pairs -> one bf16x8 MFMA operand.
__device__ __forceinline__ bf16x8 join8(bf16x2 a, bf16x2 b, bf16x2 c, bf16x2 d) {
  return __builtin_shufflevector(__builtin_shufflevector(a, b, 0, 1, 2, 3), __builtin_shufflevector(c, d, 0, 1, 2, 3),
                                 0, 1, 2, 3, 4, 5, 6, 7);
}

// Eight float32 accumulator values -> one bf16x8 MFMA operand.
__device__ __forceinline__ bf16x8 pack8(float a0, float a1, float a2, float a3, float a4, float a5, float a6,
                                        float a7) {
  u32x4 u = {pack_bf16_u32(a0, a1), pack_bf16_u32(a2, a3), pack_bf16_u32(a4, a5), pack_bf16_u32(a6, a7)};
  return __builtin_bit_cast(bf16x8, u);
}

// ---------------------------------------------------------------- math
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }  // v_exp_f32
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }   // v_log_f32
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }    // v_rcp_f32
__device__ __forceinline__ float max3f(float a, float b, float c) { return __builtin_fmaxf(a, __builtin_fmaxf(b, c)); }

// Value of x from lanes l % 32 and 32 + l % 32, in every lane: (lower, upper).
__device__ __forceinline__ void halves(float x, float& lo, float& hi) {
  uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_halves(float x) {
  float lo, hi;
  halves(x, lo, hi);
  return __builtin_fmaxf(lo, hi);
}
__device__ __forceinline__ float sum_halves(float x) {
  float lo, hi;
  halves(x, lo, hi);
  return lo + hi;
}

// ---------------------------------------------------------------- LDS
//
// K and V tiles live in LDS as rows of D bf16 split into 16-byte chunks.
// The chunk c of row r is stored at physical chunk c ^ swz(r).  The LDS
// serves 256 bytes (16 chunk slots) per cycle; swz is chosen so that both
// access patterns of the kernels hit 16 distinct slots:
//   * ds_read_b128: 16 lanes read one logical chunk from 16 consecutive rows
//     (swz must be a bijection on those rows);
//   * ds_read_b64_tr_b16: 32 lanes read 4 consecutive chunks (4-aligned)
//     from 4 consecutive rows (4-aligned), so each of the 4 rows must land
//     its 4 chunks in a different 4-slot group.
// For rows of 256 bytes (D = 128; D = 256 rows span two windows) this is
// the swap of the two 2-bit halves of r % 16.  For D = 64 two rows share a
// window: x = (r / 2) % 8 must be a bijection, with bit 2 of the result
// separating rows r and r + 2.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D >= 128) {
    const int x = r & 15;
    return ((x & 3) << 2) | (x >> 2);
  } else {
    const int x = (r >> 1) & 7;
    return ((x & 1) << 2) | (x >> 1);
  }
}

template <int D>
__device__ __forceinline__ int lds_off_bytes(int row, int chunk) {
  return row * (D * 2) + ((chunk ^ swz<D>(row)) << 4);
}

__device__ __forceinline__ s16x4 ds_read_tr(const char __attribute__((address_space(3))) * p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)p);
}

// Direct global -> LDS copy of 16 bytes per lane: lane l's 16 bytes land at
// LDS byte address lds_base + 16 * l.  lds_base must be the same in every
// lane of the wave (it is passed in M0).  Issued from inline assembly so
// that the compiler does not guard every later LDS read with a wait on it.
// The caller orders these copies itself: wait_vmcnt + a workgroup barrier
// before the copied data is read, and a barrier between the last read of a
// buffer and the next copy into it (the barrier also keeps the compiler
// from moving LDS reads across the copy).  The s_nop is the wait state a
// write of M0 needs before an LDS DMA reads it.
__device__ __forceinline__ void load_lds16(const void* gptr, const void __attribute__((address_space(3))) * lds_base) {
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile(
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(gptr), "{m0}"(base));
}

// Same copy with a wave-uniform 64-bit base in SGPRs and a per-lane 32-bit
// byte offset: the address arithmetic per copy is scalar only.  The compiler
// may rebuild the SGPR base with v_readfirstlane right before this
// instruction, and a VMEM instruction may read an SGPR written by a VALU
// instruction only after 5 wait states; the compiler cannot see the read
// inside the assembly, so the s_nop 4 here provides them (and covers the
// M0 write too).
__device__ __forceinline__ void load_lds16_sbase(const void* sbase, uint32_t voff,
                                                 const void __attribute__((address_space(3))) * lds_base) {
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  // readfirstlane returns a signed int: widen each half through uint32_t so
  // the low half is zero-extended (a sign-extended low half with bit 31 set
  // would corrupt the upper address bits).
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)sbase);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uintptr_t)sbase >> 32));
  const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile(
      "s_nop 4\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sb), "{m0}"(base));
}

// Same copy for a base and an LDS address that are already wave-uniform
// scalars (computed by scalar instructions, never rebuilt from a VGPR): only
// the M0 write needs its wait state.  The hazard scan of the built assembly
// checks that no VALU instruction writes the base SGPRs shortly before.
__device__ __forceinline__ void load_lds16_s(const void* sbase, uint32_t voff, uint32_t lds) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)sbase);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uintptr_t)sbase >> 32));
  const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile(
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sb), "{m0}"(lds));
}

// Same, 4 bytes per lane: lane l's dword lands at lds_base + 4 * l.
__device__ __forceinline__ void load_lds4(const void* gptr, const void __attribute__((address_space(3))) * lds_base) {
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile(
      "s_nop 0\n\t"
      "global_load_lds_dword %0, off"
      :
      : "v"(gptr), "{m0}"(base));
}

typedef char __attribute__((address_space(3))) lds_char;

// Copy rows row0 .. row0+ROWS-1 (clamped to N-1) of a [N][D] bf16 matrix into
// an LDS buffer of ROWS x DP (DP >= D, in {64, 128, 256}), in the swizzled
// layout above.  All WAVES waves of the workgroup take part; each issues
// ROWS*DP/8/WAVES/64 direct loads.  A slot whose chunk lies past D copies the
// row's first chunk again (into the unused part of the LDS row).
template <int D, int DP, int ROWS, int WAVES>
__device__ __forceinline__ void copy_rows_lds(const __bf16* __restrict__ src, int N, int row0, lds_char* buf, int wave,
                                              int lane) {
  static_assert(D <= DP && D % 8 == 0, "row widths");
  constexpr int kRowChunks = DP / 8;
  constexpr int kChunksPerWave = ROWS * kRowChunks / WAVES;
  static_assert(kChunksPerWave % 64 == 0, "tile must split into whole wave loads");
#pragma unroll
  for (int i = 0; i < kChunksPerWave / 64; ++i) {
    const int slot0 = wave * kChunksPerWave + i * 64;  // wave-uniform
    const int slot = slot0 + lane;
    const int r = slot / kRowChunks;
    int c = (slot % kRowChunks) ^ swz<DP>(r);
    c = c < D / 8 ? c : 0;
    int grow = row0 + r;
    grow = grow < N ? grow : N - 1;
    load_lds16(src + (size_t)grow * D + c * 8, buf + slot0 * 16);
  }
}

// Row-tile copier with loop-invariant per-lane offsets: ROWS x D bf16 rows
// starting at a uniform row go to a swizzled LDS tile with a scalar base per
// copy.  Callers keep every tile inside the tensor (a ragged last tile is
// taken shifted back so that it ends at row N-1); only tensors shorter than
// a tile need per-lane clamping.  The LDS rows are DP >= D wide (DP in
// {64, 128, 256}); a slot whose chunk lies past D (D = 96, 160) copies the
// row's first chunk again into the unused part of the LDS row, so every
// lane of a copy stays inside the global row.
template <int D, int DP, int ROWS, int WAVES>
struct RowTileCopier {
  static_assert(D <= DP && D % 8 == 0, "row widths");
  static constexpr int kRowChunks = DP / 8;
  static constexpr int kChunksPerWave = ROWS * kRowChunks / WAVES;
  static constexpr int kLoads = kChunksPerWave / 64;
  static_assert(kChunksPerWave % 64 == 0, "tile must split into whole wave loads");
  uint32_t off[kLoads];  // byte offset of this lane's chunk relative to the tile's first row
  int rowi[kLoads];      // its row within the tile
  int wave_slot0;
  uint32_t lds_wave;     // byte offset of this wave's first chunk in a tile (wave-uniform)

  __device__ __forceinline__ void init(int wave, int lane) {
    wave_slot0 = wave * kChunksPerWave;
    lds_wave = (uint32_t)__builtin_amdgcn_readfirstlane(wave_slot0 * 16);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int slot = wave_slot0 + i * 64 + lane;
      const int r = slot / kRowChunks;
      int c = (slot % kRowChunks) ^ swz<DP>(r);
      c = c < D / 8 ? c : 0;
      rowi[i] = r;
      off[i] = (uint32_t)((r * D + c * 8) * 2);
    }
  }

  // Rows of the tile starting byte_off bytes into src (a whole tile inside
  // the tensor).  All address arithmetic is scalar: src + byte_off as the
  // SGPR base, the LDS address in M0.
  __device__ __forceinline__ void copy_at(const __bf16* __restrict__ src, uint32_t byte_off, lds_char* buf) const {
    // readfirstlane pins the offset to an SGPR before the 64-bit add (the
    // compiler may otherwise strength-reduce it into a VGPR and rebuild the
    // base with a VALU instruction right before the copy)
    const char* base = (const char*)src + (uint32_t)__builtin_amdgcn_readfirstlane((int)byte_off);
    const uint32_t lds = (uint32_t)(uintptr_t)buf + lds_wave;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) load_lds16_s(base, off[i], lds + i * 64 * 16);
  }

  // Load i (of kLoads) of copy_at alone, for copies spread between other work.
  __device__ __forceinline__ void copy_one_at(const __bf16* __restrict__ src, uint32_t byte_off, lds_char* buf,
                                              int i) const {
    const char* base = (const char*)src + (uint32_t)__builtin_amdgcn_readfirstlane((int)byte_off);
    const uint32_t lds = (uint32_t)(uintptr_t)buf + lds_wave;
    load_lds16_s(base, off[i], lds + i * 64 * 16);
  }

  // A tile reaching past row N-1 (row0 <= N-1): rows past it are clamped
  // onto it per lane.
  __device__ __forceinline__ void copy_clamped(const __bf16* __restrict__ src, int N, int row0, lds_char* buf) const {
    const __bf16* base = src + (size_t)row0 * D;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int over = row0 + rowi[i] - (N - 1);
      const uint32_t o = over > 0 ? off[i] - (uint32_t)(over * D * 2) : off[i];
      load_lds16_sbase(base, o, buf + (wave_slot0 + i * 64) * 16);
    }
  }
};

// MFMA operand of 8 bf16 along k, read transposed out of a swizzled [rows][D]
// LDS tile (rows are the k index, D the m/n index).  The 32 m/n values are
// d0 .. d0+31; the k slots are rows r0 + {half*4 + 0..3, 8 + half*4 + 0..3},
// which is the order in which a 32x32 accumulator holds its rows, so an
// accumulator packed to bf16 is the matching other operand.
template <int D>
__device__ __forceinline__ bf16x8 read_tr_operand(const lds_char* tile, int r0, int d0, int lane) {
  const int g = lane >> 4, j16 = lane & 15, half = lane >> 5;
  const int dcol = d0 + (g & 1) * 16 + (j16 & 3) * 4;
  const int chunk = dcol >> 3;
  const int boff = (dcol & 7) * 2;
  const int r1 = r0 + half * 4 + (j16 >> 2);
  const s16x4 va = ds_read_tr(tile + lds_off_bytes<D>(r1, chunk) + boff);
  const s16x4 vb = ds_read_tr(tile + lds_off_bytes<D>(r1 + 8, chunk) + boff);
  const s16x8 v8 = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
  return __builtin_bit_cast(bf16x8, v8);
}

// MFMA operand of 8 bf16 along k = d, read row-wise: row `row`, d = ds*16 + half*8 + 0..7.
template <int D>
__device__ __forceinline__ bf16x8 read_row_operand(const lds_char* tile, int row, int ds, int half) {
  return *(const bf16x8 __attribute__((address_space(3)))*)(tile + lds_off_bytes<D>(row, ds * 2 + half));
}

// s_waitcnt with only vmcnt constrained (expcnt and lgkmcnt left at max).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

}  // namespace fa
