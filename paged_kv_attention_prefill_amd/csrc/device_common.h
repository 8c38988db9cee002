// Device helpers shared by the library's kernels: storage-dtype decoding,
// output encoding, wavefront reductions.  gfx950, wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "params.h"

namespace pa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t u16) { return __uint_as_float(u16 << 16); }

__device__ __forceinline__ float f16_bits_to_f32(uint32_t u16) {
  _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)u16);
  return (float)h;
}

// OCP e4m3fn -> fp32, exact.  Normal codes rebias the exponent (7 -> 127);
// subnormals are m * 2^-9; S.1111.111 is NaN.
__device__ __forceinline__ float fp8e4m3_bits_to_f32(uint32_t c) {
  const uint32_t sign = (c & 0x80u) << 24;
  const uint32_t em = c & 0x7fu;
  const float normal = __uint_as_float(sign | ((em + (120u << 3)) << 20));
  const float sub = __uint_as_float(sign | __float_as_uint((float)em * 0x1p-9f));
  float r = em < 8u ? sub : normal;
  return em == 0x7fu ? __uint_as_float(0x7fc00000u) : r;
}

template <int DT>
__device__ __forceinline__ float load_elem(const void* base, int64_t idx) {
  if constexpr (DT == F32) {
    return static_cast<const float*>(base)[idx];
  } else if constexpr (DT == F16) {
    return f16_bits_to_f32(static_cast<const uint16_t*>(base)[idx]);
  } else if constexpr (DT == BF16) {
    return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[idx]);
  } else {
    return fp8e4m3_bits_to_f32(static_cast<const uint8_t*>(base)[idx]);
  }
}

// fp32 -> bf16 bits with round-to-nearest-even (NaN kept quiet)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;
  return __builtin_bit_cast(uint16_t, h);
}

template <int DT>
__device__ __forceinline__ void store_elem(void* base, int64_t idx, float v) {
  if constexpr (DT == F32) {
    static_cast<float*>(base)[idx] = v;
  } else if constexpr (DT == F16) {
    static_cast<uint16_t*>(base)[idx] = (uint16_t)f32_to_f16_bits(v);
  } else {
    static_cast<uint16_t*>(base)[idx] = (uint16_t)f32_to_bf16_bits(v);
  }
}

// Sum over the 64 lanes, every lane receiving the total, in VALU cross-lane
// steps: DPP quad permutations (lanes l ^ 1, l ^ 2), row half-mirror and row
// mirror (pairing the quads of each 8 and the halves of each 16 lanes), then the
// gfx950 permlane swaps of 16-lane rows and 32-lane halves.  Each step adds a
// lane's value to its partner's, so partners hold identical sums at every step.
template <int CTRL>
__device__ __forceinline__ float dpp_partner(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_allreduce_sum(float v) {
  v += dpp_partner<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_partner<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_partner<0x141>(v);  // row_half_mirror
  v += dpp_partner<0x140>(v);  // row_mirror
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_allreduce_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// n / d given magic = ceil(2^32 / d) for d >= 2 (exact while n * d < 2^32), or
// magic = 0 for d == 1; branch-free
__device__ __forceinline__ uint32_t div_by_magic(uint32_t n, uint32_t magic) {
  const uint32_t one = magic == 0 ? 0xFFFFFFFFu : 0u;
  return __umulhi(n, magic) + (n & one);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Batch of query token t: uniform decode layout, or a search of qo_indptr.
__device__ __forceinline__ int batch_of_token(const AttnParams& p, int t) {
  if (p.qo_indptr == nullptr) return t / p.q_len;
  int lo = 0, hi = p.batch - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (p.qo_indptr[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace pa
