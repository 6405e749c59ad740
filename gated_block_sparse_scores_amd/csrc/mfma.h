// gfx950 bf16 MFMA helpers (wave64).
//
// v_mfma_f32_32x32x16_bf16, as used here (checked by tests/test_gpu_mfma_layout
// through the attention parity tests):
//   A (32 x 16): lane l supplies row l % 32, eight k-values of k-group l / 32;
//   B (16 x 32): lane l supplies column l % 32, the same eight k-values;
//   D (32 x 32): lane l holds column l % 32, rows
//                (r / 4) * 8 + (l / 32) * 4 + (r % 4) for r = 0..15.
// The contraction only needs A's and B's k-values paired by (k-group, element),
// so any consistent assignment of actual k indices to (group, element) works.
#pragma once

#include <hip/hip_runtime.h>

namespace sas {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row (within a 32-row tile) of accumulator register r for lane group g.
__device__ __forceinline__ constexpr int acc_row(int r, int g) {
  return (r >> 2) * 8 + g * 4 + (r & 3);
}

__device__ __forceinline__ bf16x8 cat4(const bf16x4& lo, const bf16x4& hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Packs eight accumulator values (registers r0 .. r0+7) to bf16 (RNE).
__device__ __forceinline__ bf16x8 pack8(const f32x16& x, int r0) {
  bf16x8 o;
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = (__bf16)x[r0 + j];
  return o;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace sas
