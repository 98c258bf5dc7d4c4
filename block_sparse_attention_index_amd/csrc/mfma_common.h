// mfma_common.h -- gfx950 matrix-core helpers shared by the sparse prefill
// and decode kernels: bf16 MFMA operand types, the 32x32x16 bf16 MFMA, the
// transposing LDS read and the lane-half exchanges.
//
// Lane layouts of v_mfma_f32_32x32x16_bf16 (lane l, h = l / 32, j = l % 32):
//   A[i][k]: lane holds i = j, k = 8h .. 8h+7
//   B[k][n]: lane holds n = j, k = 8h .. 8h+7
//   D[i][n]: lane register r holds n = j, i = 8*(r/4) + 4h + r%4
#pragma once
#include "msa_internal.h"

namespace msa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));


typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 *lds_s16x4_ptr;

// ds_read_b64_tr_b16: lane i of each 16-lane group gets element i%16 of the
// group's 16 eight-byte rows read as a 4 x 16 matrix (row r = lanes 4r..4r+3).
__device__ __forceinline__ u32x2 lds_read_tr(const uint16_t *p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4_ptr)(const_cast<uint16_t *>(p)));
  return __builtin_bit_cast(u32x2, r);
}

// Value of the lane l^32 combined with the own value: v_permlane32_swap(x, x)
// returns x from lanes l%32 and l%32+32 in its two results.
__device__ __forceinline__ float max_with_partner(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                                  __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_with_partner(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                                  __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}


}  // namespace msa
