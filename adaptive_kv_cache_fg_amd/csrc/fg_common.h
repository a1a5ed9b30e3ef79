// Internal helpers shared by the libfastgen kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -3.0e38f;   // finite "minus infinity" for running maxima

constexpr uint8_t kNormal = 0, kSpecial = 1, kPunct = 2;

// 32x32 MFMA tile traits.  One MFMA multiplies a 32 x KS block of A (rows
// m = lane % 32, k = (lane / 32) * EPL + e) by a KS x 32 block of B (columns
// n = lane % 32, same k mapping) into a 32 x 32 fp32 tile whose element
// (row 8*(r/4) + 4*(lane/32) + r%4, column lane%32) sits in accumulator r.
template <typename T> struct Mfma;

template <> struct Mfma<__bf16> {
  using op_t = bf16x8;
  static constexpr int KS = 16;   // reduction depth per instruction
  static constexpr int EPL = 8;   // elements per lane per instruction
  static __device__ __forceinline__ f32x16 mac(op_t a, op_t b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma<float> {
  using op_t = float;
  static constexpr int KS = 2;
  static constexpr int EPL = 1;
  static __device__ __forceinline__ f32x16 mac(op_t a, op_t b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// Row (within the 32x32 tile) held by accumulator r of this lane, and its lane-independent part
// (acc_row(r, lane) = acc_row0(r) + 4 * (lane >> 5)).
__device__ __forceinline__ constexpr int acc_row0(int r) { return 8 * (r >> 2) + (r & 3); }
__device__ __forceinline__ int acc_row(int r, int lane) { return acc_row0(r) + 4 * (lane >> 5); }

// Index of this thread's wave in the workgroup, as a scalar (wave-uniform) value so
// that branches on it stay scalar branches instead of exec-masked regions.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// Sum over aligned groups of N lanes (N = 1..64, power of two); every lane of a
// group receives the group's sum.  Groups up to 16 lanes use DPP lane permutes
// on the VALU (quad_perm, row_half_mirror, row_mirror), wider ones fall back to
// cross-lane shuffles.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if (N >= 2) v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
  if (N >= 4) v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
  if (N >= 8) v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true));
  if (N >= 16) v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, true));
  if (N >= 32) v += __shfl_xor(v, 16);
  if (N >= 64) v += __shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// m + log2(l) for a running (reference, sum) pair whose sum may be far from 1 (l > 0): the
// logarithm is taken of l's mantissa only (in [0.5, 1), where log2 is accurate to a few units
// of 2^-24 absolute) and the exponent and reference are added in double, so the result is
// rounded to fp32 once.
__device__ __forceinline__ float log2_of_scaled(float m, float l) {
  int e;
  const float mant = frexpf(l, &e);
  return (float)((double)m + (double)e + (double)fast_log2(mant));
}

template <typename T>
__device__ __forceinline__ T zero_val() { return T(0.0f); }

}  // namespace fg
