// mfma.h -- CDNA4 (gfx950) bf16 matrix-core fragments used by libdynconv.
//
// Lane layouts (wave64), checked on the hardware against a CPU matmul:
//   v_mfma_f32_16x16x32_bf16  D[16x16] += A[16x32] B[32x16]
//     A: lane l holds A[l%16][8*(l/16) + i], i = 0..7
//     B: lane l holds B[8*(l/16) + i][l%16]
//     D: lane l holds D[4*(l/16) + r][l%16], r = 0..3
//   v_mfma_f32_32x32x16_bf16  D[32x32] += A[32x16] B[16x32]
//     A: lane l holds A[l%32][8*(l/32) + i]
//     B: lane l holds B[8*(l/32) + i][l%32]
//     D: lane l holds D[8*b + 4*(l/32) + r][l%32] in element 4*b + r, b, r = 0..3
#pragma once

#include "common.h"

namespace dynconv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x4 mfma16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ds_read_b64_tr_b16 (gfx950): in each group of 16 lanes, lane L receives
// element L%4 of the 8-byte reads of lanes L/4, 4 + L/4, 8 + L/4 and
// 12 + L/4, in that order.  When lane 4e + c reads row r0 + e at column
// 4c, lane L gets rows r0 .. r0+3 of column L: four bf16 of one column of a
// row-major LDS tile.  p is the lane's LDS address.
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
__device__ __forceinline__ uint2 read_tr16(const unsigned char *p) {
  const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p));
  return __builtin_bit_cast(uint2, v);
}

// 16 bytes of bf16 as an MFMA operand.
__device__ __forceinline__ bf16x8 as_bf16x8(const uint4 &r) { return __builtin_bit_cast(bf16x8, r); }

__device__ __forceinline__ bf16x8 zero_bf16x8() { return as_bf16x8(make_uint4(0, 0, 0, 0)); }

// Round 8 fp32 values to bf16 (nearest even) as an MFMA operand.
// the fp32 value of a bf16 bit pattern
__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits) { return __uint_as_float(bits << 16); }

__device__ __forceinline__ bf16x8 pack_bf16x8(const float (&v)[8]) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (bf16)v[i];
  return r;
}

}  // namespace dynconv
