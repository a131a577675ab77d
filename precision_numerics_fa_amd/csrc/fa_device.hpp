// Device-side building blocks shared by the forward and backward kernels:
// vector types, the gfx950 bf16 MFMA, LDS loads (plain and transposing),
// bf16 packing, and the repeated-maximum shift rule.
//
// MFMA v_mfma_f32_32x32x16_bf16 operand layout (wave64, lane l, element j):
//   A[m][k]: m = l % 32, k = 8 * (l / 32) + j      (8 bf16 per lane)
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

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t bf16_t;  // storage type of a bf16 value in global memory

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_huge_valf();

// Shift-rule constants (base-2 exponent units).
constexpr float kDeltaMin = 0.0625f;
constexpr float kDeltaMax = 64.0f;
constexpr float kFold = 32.0f;

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
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

// Round-to-nearest-even float -> bf16 (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ __bf16 to_bf16(float x) { return (__bf16)x; }

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  __bf16 x = to_bf16(a), y = to_bf16(b);
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// Eight consecutive accumulator entries c[base .. base+7] as a bf16 MFMA operand.
__device__ __forceinline__ bf16x8 pack8(const f32x16& c, int base) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = to_bf16(c[base + j]);
  return r;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// The repeated-maximum shift (base-2 units).  R = running max * scale*log2e.
// Returns R + delta with delta = max(|R|, kDeltaMin), |R| folded by whole
// multiples of kFold into (kDeltaMax - kFold, kDeltaMax] when larger than
// kDeltaMax.  Every step is exact in fp32 except the final addition.
__device__ __forceinline__ float shifted_offset(float R) {
  float a = __builtin_fabsf(R);
  if (a > kDeltaMax) a -= kFold * __builtin_ceilf((a - kDeltaMax) * (1.0f / kFold));
  a = __builtin_fmaxf(a, kDeltaMin);
  return R + a;
}

}  // namespace fa
