// MFMA and LDS-transpose helpers for gfx950 (wave64).
//
// Operand layouts (verified on the device):
//   v_mfma_f32_16x16x32_{bf16,f16}: A[m][k]: lane l holds m = l%16,
//     k = 8*(l/16) .. +8;  B[k][n]: n = l%16, same k;  C[m][n] (4 fp32):
//     n = l%16, m = 4*(l/16) + i.
//   v_mfma_f32_32x32x16_{bf16,f16}: A: m = l%32, k = 8*(l/32) .. +8; B alike;
//     C (16 fp32): n = l%32, m = 8*(i/4) + 4*(l/32) + i%4.
//   ds_read_b64_tr_b16: within each 16-lane group, lane r*4+cb supplies the
//     address of row r, columns 4cb..4cb+3 of a 4x16 block of 16-bit elements;
//     lane c receives column c of the block (rows 0..3).
#pragma once

#include "device_common.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));

#define PA_LDS __attribute__((address_space(3)))

// 16x16x32 MFMA on eight 16-bit elements per lane held as raw bits.
template <int DT>
__device__ __forceinline__ f32x4_t mfma16(const i16x8_t& a, const i16x8_t& b, f32x4_t c) {
  if constexpr (DT == BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
}

template <int DT>
__device__ __forceinline__ f32x16_t mfma32(const i16x8_t& a, const i16x8_t& b, f32x16_t c) {
  if constexpr (DT == BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
}

// Transposed 4x16 read (see above); `p` points at this lane's row/column quad.
__device__ __forceinline__ i16x4_t lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((PA_LDS i16x4_t*)(p));
}

// fp32 -> 16-bit storage bits of DT (RNE)
template <int DT>
__device__ __forceinline__ uint32_t to_bits16(float x) {
  if constexpr (DT == BF16) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
  } else {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
  }
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// two fp32 -> packed 16-bit bits of DT (RNE), a in the low half: one
// v_cvt_pk_{bf16,f16}_f32
template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const f32x2_t v = {a, b};
  if constexpr (DT == BF16) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
  }
}

// acc + the two 16-bit values of DT packed in `bits` (v_dot2 against ones, fp32 sum)
template <int DT>
__device__ __forceinline__ float sum2(uint32_t bits, float acc) {
  if constexpr (DT == BF16) {
    const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, bits), one, acc, false);
  } else {
    const f16x2_t one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, bits), one, acc, false);
  }
}

__device__ __forceinline__ i16x8_t as_i16x8(const uint4& u) { return __builtin_bit_cast(i16x8_t, u); }

// Reductions of a lane's value with that of lane l ^ 16 or l ^ 32 through the
// gfx950 permlane swaps (VALU, no LDS): v_permlane16_swap exchanges the odd
// 16-lane rows of its first operand with the even rows of its second, so with
// both operands equal to v one result holds rows (0,0,2,2) and the other
// (1,1,3,3); v_permlane32_swap does the same with the two 32-lane halves.
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ void lds_wait() { __builtin_amdgcn_s_waitcnt(0xC07F); }

}  // namespace pa
