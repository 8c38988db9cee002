// merge_states: combine S partial attention states of each row through their
// log-sum-exp ("Move the Query, Not the Cache" summary, method section: the
// Route primitive merges partial attention results by online softmax; the
// SM110 XQA split kernel, kernel-design section, merges partials and row
// statistics the same way).
//   m = max_c s_c; w_c = exp(s_c - m); out = sum_c w_c v_c / sum_c w_c;
//   s_out = m + ln(sum_c w_c); -inf states carry no weight; all -inf -> 0, -inf.
//
// HBM-bound: each row's S x D partials are read once (16-byte loads of four
// fp32 elements per lane), the S LSEs once per lane from cache.
#include "device_common.h"

namespace pa {
namespace {

template <int VT>
__device__ __forceinline__ void load4(const void* base, int64_t idx, float (&x)[4]) {
  if constexpr (VT == F32) {
    const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
  } else {
    const uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + idx);
    const uint32_t w[4] = {v.x & 0xffffu, v.x >> 16, v.y & 0xffffu, v.y >> 16};
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = VT == F16 ? f16_bits_to_f32(w[i]) : bf16_bits_to_f32(w[i]);
  }
}

template <int OT>
__device__ __forceinline__ void store4(void* base, int64_t idx, const float (&x)[4]) {
  if constexpr (OT == F32) {
    *reinterpret_cast<float4*>(static_cast<float*>(base) + idx) = make_float4(x[0], x[1], x[2], x[3]);
  } else {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = OT == F16 ? f32_to_f16_bits(x[i]) : f32_to_bf16_bits(x[i]);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + idx) =
        make_uint2(w[0] | (w[1] << 16), w[2] | (w[3] << 16));
  }
}

template <int VT, int OT>
__global__ __launch_bounds__(256) void merge_kernel(const void* v, const float* s, int S,
                                                    int64_t rows, int D, int tpr,
                                                    int64_t v_ss, int64_t s_ss, void* out,
                                                    float* s_out) {
  const int rpb = blockDim.x / tpr;
  const int64_t row = (int64_t)blockIdx.x * rpb + threadIdx.x / tpr;
  const int li = threadIdx.x % tpr;
  if (threadIdx.x >= rpb * tpr || row >= rows) return;
  const int d0 = li * 4;
  float m = -INFINITY;
  for (int c = 0; c < S; ++c) m = fmaxf(m, s[c * s_ss + row]);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  if (m == -INFINITY) {
    store4<OT>(out, row * D + d0, acc);
    if (s_out && li == 0) s_out[row] = -INFINITY;
    return;
  }
  float wsum = 0.f;
  for (int c = 0; c < S; ++c) {
    const float lc = s[c * s_ss + row];
    if (lc == -INFINITY) continue;
    const float w = fast_exp2((lc - m) * kLog2e);
    wsum += w;
    float x[4];
    load4<VT>(v, c * v_ss + row * D + d0, x);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = fmaf(w, x[i], acc[i]);
  }
  const float inv = 1.f / wsum;
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] *= inv;
  store4<OT>(out, row * D + d0, acc);
  if (s_out && li == 0) s_out[row] = m + fast_log2(wsum) * kLn2;
}

template <int VT>
hipError_t launch_vt(const void* v, const float* s, int S, int64_t rows, int D, int64_t v_ss,
                     int64_t s_ss, void* out, int out_dtype, float* s_out, hipStream_t stream) {
  const int tpr = D / 4;
  const int rpb = tpr >= 256 ? 1 : 256 / tpr;
  const dim3 block(rpb * tpr);
  const dim3 grid((unsigned)((rows + rpb - 1) / rpb));
  if (rows == 0) return hipSuccess;
  if (out_dtype == F32)
    merge_kernel<VT, F32><<<grid, block, 0, stream>>>(v, s, S, rows, D, tpr, v_ss, s_ss, out, s_out);
  else if (out_dtype == F16)
    merge_kernel<VT, F16><<<grid, block, 0, stream>>>(v, s, S, rows, D, tpr, v_ss, s_ss, out, s_out);
  else
    merge_kernel<VT, BF16><<<grid, block, 0, stream>>>(v, s, S, rows, D, tpr, v_ss, s_ss, out, s_out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const void* v, int v_dtype, const float* s, int num_states, int64_t rows,
                        int head_dim, int64_t v_state_stride, int64_t s_state_stride, void* out,
                        int out_dtype, float* s_out, hipStream_t stream) {
  if (v_dtype == F32)
    return launch_vt<F32>(v, s, num_states, rows, head_dim, v_state_stride, s_state_stride, out,
                          out_dtype, s_out, stream);
  if (v_dtype == F16)
    return launch_vt<F16>(v, s, num_states, rows, head_dim, v_state_stride, s_state_stride, out,
                          out_dtype, s_out, stream);
  return launch_vt<BF16>(v, s, num_states, rows, head_dim, v_state_stride, s_state_stride, out,
                         out_dtype, s_out, stream);
}

}  // namespace pa
