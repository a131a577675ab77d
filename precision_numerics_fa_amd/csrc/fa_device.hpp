// Device-side building blocks shared by the forward and backward kernels:
// vector types, the gfx950 bf16 and f16 MFMAs, LDS loads (plain and
// transposing), 16-bit packing, and the repeated-maximum shift rule.
//
// MFMA v_mfma_f32_32x32x16_{bf16,f16} operand layout (wave64, lane l,
// element j):
//   A[m][k]: m = l % 32, k = 8 * (l / 32) + j      (8 16-bit values per lane)
//   B[k][n]: n = l % 32, k = 8 * (l / 32) + j
//   C[r][n]: n = l % 32, r = 8 * (i / 4) + 4 * (l / 32) + (i % 4), i = 0..15
// Both operands want the contraction index contiguous in a lane's registers.
//
// ds_read_b64_tr_b16 (gfx950 LDS transpose read), per group of 16 lanes:
// lane j supplies the address of four consecutive 16-bit elements E[j][0..3];
// lane i receives, in slot s, E[4 s + i / 4][i % 4].  Pointing lane j at
// row (base_row + j / 4), column (base_col + 4 * (j % 4)) of a row-major tile
// therefore hands lane i the column (base_col + i) of rows base_row + 0..3:
// a transposed 4x16 read, which is how the kernels feed V^T, Q^T, dO^T and
// K^T operands from row-major LDS tiles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t bf16_t;  // storage type of a bf16 value in global memory

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_huge_valf();

// Shift-rule constants (base-2 exponent units) for bf16.
constexpr float kDeltaMin = 0.0625f;
constexpr float kDeltaMax = 64.0f;
constexpr float kFold = 32.0f;
// For binary16 the largest probability 2^-delta must stay far inside its
// exponent range (normal numbers end at 2^-14), so |R| is folded by whole
// units into (0, 1].
constexpr float kF16DeltaMax = 1.0f;
constexpr float kF16Fold = 1.0f;

template <typename E>
struct ShiftRule {
  static constexpr float dmin = kDeltaMin, dmax = kDeltaMax, fold = kFold;
};
template <>
struct ShiftRule<_Float16> {
  static constexpr float dmin = kDeltaMin, dmax = kF16DeltaMax, fold = kF16Fold;
};

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Element types.  Tiles and MFMA operands hold 16-bit values as raw bits (a
// bf16x8 register vector is eight 16-bit lanes, whatever their format); the
// element type E, __bf16 or _Float16 (IEEE binary16), selects only the MFMA
// instruction, the float -> 16-bit rounding (to nearest even) and the
// 16-bit -> float widening.
template <typename E>
__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c);
template <>
__device__ __forceinline__ f32x16 mfma<__bf16>(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x16 mfma<_Float16>(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

// 16-byte LDS load of 8 bf16 (address must be 16-byte aligned).
__device__ __forceinline__ bf16x8 lds_load8(const bf16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// Transposing LDS read of four 16-bit values (see the header comment).
__device__ __forceinline__ s16x4 lds_load_tr4(const bf16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)((__attribute__((address_space(3))) char*)(p)));
}

__device__ __forceinline__ bf16x8 join8(s16x4 lo, s16x4 hi) {
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Round-to-nearest-even float -> 16-bit pattern of E (bf16: v_cvt_pk_bf16_f32
// per pair on gfx950; binary16: v_cvt_f16_f32 per value).
template <typename E>
__device__ __forceinline__ uint16_t round16(float x) {
  return __builtin_bit_cast(uint16_t, (E)x);
}

// Exact 16-bit pattern of E -> float.
template <typename E>
__device__ __forceinline__ float widen16(uint32_t h);
template <>
__device__ __forceinline__ float widen16<__bf16>(uint32_t h) { return __uint_as_float(h << 16); }
template <>
__device__ __forceinline__ float widen16<_Float16>(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

template <typename E>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return (uint32_t)round16<E>(a) | ((uint32_t)round16<E>(b) << 16);
}

// Eight consecutive accumulator entries c[base .. base+7] as an MFMA operand.
template <typename E>
__device__ __forceinline__ bf16x8 pack8(const f32x16& c, int base) {
  typedef E e8 __attribute__((ext_vector_type(8)));
  e8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (E)c[base + j];
  return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// The values of x in lanes (l mod 32) and 32 + (l mod 32), in every lane l:
// one v_permlane32_swap (gfx950) instead of an LDS permute.  Any symmetric
// combination of the two (max, min, sum) is then the lane pair's.
__device__ __forceinline__ void lane_pair(float x, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// The same wait issued through the builtin, which the compiler's wait-count
// tracking sees (the inline-asm form above is opaque to it).  Issued once
// after the prologue's register loads have landed, it clears the compiler's
// record of them; otherwise a path on which they might still be in flight
// makes it place a vmcnt(0) wait inside the main loop, where it would also
// wait for the tile prefetches issued there.  (gfx9 encoding: vmcnt 0,
// expcnt 7, lgkmcnt 15.)
__device__ __forceinline__ void wait_vmem_tracked() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ---------------------------------------------------------------------------
// Swizzled LDS tiles.  A tile holds ROWS rows of D bf16 with no padding; the
// 16-byte chunk k of row r is stored at chunk position k ^ swz<D>(r).  LDS has
// 64 four-byte banks, so a chunk position is a group of 4 banks and a D = 128
// row spans all of them (a D = 64 row spans half; rows alternate halves).
// The map is chosen so that both access patterns of the kernels are free of
// bank conflicts:
//   * 16 lanes reading the same logical chunk of 16 consecutive rows
//     (ds_read_b128 of an MFMA operand with the row as m/n index);
//   * 32 lanes of a transposing read: 4 consecutive rows (a multiple-of-4
//     start) x 4 consecutive logical chunks starting at a multiple of 4.
// D = 128: swz = 4 (r % 4) + (r / 4) % 4 -- the 16 rows get 16 distinct
//   values, and 4 consecutive rows differ in bits 2-3, so an aligned block of
//   4 chunks lands on 4 disjoint blocks.
// D = 64: with u = (r / 2) % 8, swz = 4 (u % 2) + u / 2 -- a bijection of u
//   for each row parity, and rows 4a, 4a+2 (same parity) differ in bit 2.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  const int u = (row >> 1) & 7;
  return ((u & 1) << 2) | (u >> 1);
}

// Element offset of (row, col) in a swizzled tile.
template <int D>
__device__ __forceinline__ int tile_off(int row, int col) {
  return row * D + ((((col >> 3) ^ swz<D>(row))) << 3) + (col & 7);
}

// Per-lane element offsets (within a ROWS x D block of the source matrix) of
// the chunks a tile copy moves: copy r of lane `lane` in wave `wave` writes
// physical chunk c = r*NT + wave*64 + lane of the tile, which holds logical
// chunk (c % CPR) ^ swz(row) of row c / CPR.  For a block that lies fully
// inside N the copy is then a wave-uniform base pointer plus a fixed
// per-lane offset.
template <int D, int ROWS, int NT>
__device__ __forceinline__ void tile_offsets(int* off, int wave, int lane) {
  constexpr int CPR = D / 8;
  constexpr int PER_LANE = ROWS * CPR / NT;
#pragma unroll
  for (int r = 0; r < PER_LANE; ++r) {
    const int c = r * NT + wave * 64 + lane;
    const int row = c / CPR;
    off[r] = row * D + (((c % CPR) ^ swz<D>(row)) << 3);
  }
}

// A copy of x the compiler cannot see through, so that values computed from
// it in a rarely taken branch are not hoisted out of an enclosing loop.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// One direct global -> LDS copy of 16 bytes per lane: lane i's bytes land at
// LDS byte address lds_base + 16 i and come from gbase + voff (gbase and
// lds_base wave-uniform; lds_base travels in M0).  Written as inline assembly
// so that the compiler does not treat the LDS writes as pending stores that
// every later LDS read has to wait for: the caller waits (s_waitcnt vmcnt)
// and synchronises the workgroup before anyone reads the tile.  The global
// base stays in scalar registers, so a lane holds a single 32-bit offset.
__device__ __forceinline__ void dma16(const bf16_t* gbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(gbase), "s"(lds_base)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

// Rows [r0, r0 + ROWS) of X (N rows) into a swizzled tile with dma16 (r0 and
// tile wave-uniform, r0 < N).  Rows past N read row N-1 (in bounds);
// zero_tail() clears them afterwards.  off[] from tile_offsets().
// FULL: the caller guarantees r0 + ROWS <= N (no branch is emitted).
template <int D, int ROWS, int NT, bool FULL = false>
__device__ __forceinline__ void load_tile_async(const int* off, const bf16_t* __restrict__ X, int r0, int N,
                                                bf16_t* tile, int wave, int lane) {
  constexpr int CPR = D / 8;
  constexpr int PER_LANE = ROWS * CPR / NT;
  const bf16_t* base = X + (size_t)r0 * D;
  if (FULL || r0 + ROWS <= N) {
    // copy r covers rows r * (NT / CPR) + (the rows of copy 0), and the
    // swizzle repeats every 16 rows: its offsets are copy 0's plus a
    // uniform step, which goes into the scalar base
    static_assert((NT / CPR) % 16 == 0, "swizzle period");
    const uint32_t v0 = (uint32_t)off[0] * 2u;
#pragma unroll
    for (int r = 0; r < PER_LANE; ++r)
      dma16(base + r * (NT / CPR) * D, v0, lds_addr(tile + (r * NT + wave * 64) * 8));
  } else {
    // (the lane index passes through an opaque copy: the tail path's lane
    // constants are then formed here, when the path runs, instead of being
    // hoisted out of the caller's loop into registers held throughout)
    const int ln = opaque(lane);
#pragma unroll
    for (int r = 0; r < PER_LANE; ++r) {
      const int c = r * NT + wave * 64 + ln;
      const int row = c / CPR;
      const int k = (c % CPR) ^ swz<D>(row);
      const int src = min(r0 + row, N - 1) - r0;
      dma16(base, (uint32_t)(src * D + k * 8) * 2u, lds_addr(tile + (r * NT + wave * 64) * 8));
    }
  }
}

// Zero the rows of a swizzled tile that lie past N (after its loads landed).
template <int D, int ROWS, int NT>
__device__ __forceinline__ void zero_tail(int r0, int N, bf16_t* tile, int wave, int lane) {
  constexpr int CPR = D / 8;
  constexpr int PER_LANE = ROWS * CPR / NT;
  if (r0 + ROWS <= N) return;
  // (lane and the zero pass through opaque copies, so that neither the
  // offsets nor a register quad of zeros is hoisted out of the caller's loop)
  const int ln = opaque(lane);
  const uint32_t z = (uint32_t)opaque(0);
#pragma unroll
  for (int r = 0; r < PER_LANE; ++r) {
    const int c = r * NT + wave * 64 + ln;
    if (r0 + c / CPR >= N) *reinterpret_cast<uint4*>(tile + c * 8) = make_uint4(z, z, z, z);
  }
}

// The repeated-maximum shift (base-2 units).  R = running max * scale*log2e.
// The shifted offset is R + delta with delta = max(|R|, dmin), |R| folded by
// whole multiples of `fold` into (dmax - fold, dmax] when larger than dmax
// (the constants of ShiftRule<E>).  Every step of delta is exact in fp32;
// delta is finite for any R (a NaN from R = -inf is replaced by dmin).
template <typename E>
__device__ __forceinline__ float shift_delta(float R) {
  using C = ShiftRule<E>;
  const float a = __builtin_fabsf(R);
  const float folded = a - C::fold * __builtin_ceilf((a - C::dmax) * (1.0f / C::fold));
  const float d = a > C::dmax ? folded : a;
  return __builtin_fmaxf(d, C::dmin);
}

// Offset for a row: R + delta when the running maximum is tied, else R.
// Written as R + delta * {0, 1} (exactly R or R + delta) so that it stays
// branch-free inside the softmax basic block.
template <typename E>
__device__ __forceinline__ float row_offset(float R, bool tied) {
  return R + shift_delta<E>(R) * (tied ? 1.0f : 0.0f);
}

// Schedule of one stage: LEAD groups of RD LDS operand reads first, then,
// per MFMA, the MFMA, the reads of a later one, and VALU instructions --
// so the operand reads run a few products ahead and the vector work fills
// the matrix pipe's shadow without holding many operands in flight.
template <int NMFMA, int RD, int LEAD, int VALU>
__device__ __forceinline__ void interleave() {
  __builtin_amdgcn_sched_group_barrier(0x100, RD * LEAD, 0);
#pragma unroll
  for (int i = 0; i < NMFMA; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i + LEAD < NMFMA) __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
    if (VALU > 0) __builtin_amdgcn_sched_group_barrier(0x002, VALU, 0);
  }
}

}  // namespace fa
