// merge_states: combine S partial attention states of each row through their
// log-sum-exp ("Move the Query, Not the Cache" summary, method section: the
// Route primitive merges partial attention results by online softmax; the
// SM110 XQA split kernel, kernel-design section, merges partials and row
// statistics the same way).
//   m = max_c s_c; w_c = exp(s_c - m); out = sum_c w_c v_c / sum_c w_c;
//   s_out = m + ln(sum_c w_c); -inf states carry no weight; all -inf -> 0, -inf.
//
// HBM-bound: each row's S x D partials are read once (16-byte loads of four
// fp32 elements per lane, issued eight states at a time together with their
// LSEs, folded by a running maximum so a block of states needs one round trip).
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
  // one pass over blocks of BLK states: their LSEs and partials are loaded
  // together (one round trip per block) and folded into a running maximum m,
  // weight sum and accumulator, rescaled when m grows
  constexpr int BLK = 8;
  float m = -INFINITY, wsum = 0.f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < S; c0 += BLK) {
    float ls[BLK];
    float x[BLK][4];
#pragma unroll
    for (int k = 0; k < BLK; ++k) {
      const bool ok = c0 + k < S;
      ls[k] = ok ? s[(c0 + k) * s_ss + row] : -INFINITY;
      if (ok) {
        load4<VT>(v, (c0 + k) * v_ss + row * D + d0, x[k]);
      } else {
        x[k][0] = x[k][1] = x[k][2] = x[k][3] = 0.f;
      }
    }
    float bm = -INFINITY;
#pragma unroll
    for (int k = 0; k < BLK; ++k) bm = fmaxf(bm, ls[k]);
    const float mn = fmaxf(m, bm);
    if (mn == -INFINITY) continue;  // every state so far is empty
    const float a = m == -INFINITY ? 0.f : fast_exp2((m - mn) * kLog2e);
    wsum *= a;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] *= a;
#pragma unroll
    for (int k = 0; k < BLK; ++k) {
      const float w = ls[k] == -INFINITY ? 0.f : fast_exp2((ls[k] - mn) * kLog2e);
      wsum += w;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = fmaf(w, x[k][i], acc[i]);
    }
    m = mn;
  }
  if (m == -INFINITY) {
    store4<OT>(out, row * D + d0, acc);
    if (s_out && li == 0) s_out[row] = -INFINITY;
    return;
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

// Merge of internal KV chunks or balanced-split segments (the same LSE formula):
// one group of D/4 lanes per folded row (b, KV head g, row r < q_len*G); rows
// whose item was done in one piece were written directly by the attention kernel
// and are skipped here.
__global__ __launch_bounds__(256) void chunk_merge_kernel(AttnParams p, int tpr) {
  const int rpb = blockDim.x / tpr;
  const int64_t rho = (int64_t)blockIdx.x * rpb + threadIdx.x / tpr;
  const int li = threadIdx.x % tpr;
  const int R = p.q_len * p.group;
  const int WR = p.ws_rows;
  const int64_t total = (int64_t)p.batch * p.num_kv_heads * WR;
  if (threadIdx.x >= rpb * tpr || rho >= total) return;
  const int r = (int)(rho % WR);
  const int g = (int)((rho / WR) % p.num_kv_heads);
  const int b = (int)(rho / ((int64_t)WR * p.num_kv_heads));
  if (r >= R) return;
  const int item = b * p.num_kv_heads + g;
  int nch;
  int64_t wrow0;
  if (p.bal_blocks > 0) {
    // balanced split: the item's partial states sit in slots item + i for its
    // workgroups i = first..last
    const int i0 = p.ws_seg[2 * item], i1 = p.ws_seg[2 * item + 1];
    nch = i1 - i0 + 1;
    wrow0 = ((int64_t)item + i0) * WR + r;
  } else {
    const int kb = p.broadcast ? 0 : b;
    const int n = p.kv_indptr[kb + 1] - p.kv_indptr[kb];
    const int L = n ? (n - 1) * p.page_size + p.kv_last[kb] : 0;
    nch = num_chunks(L, p.chunk_tokens, p.max_chunks);
    wrow0 = (int64_t)item * p.max_chunks * WR + r;
  }
  if (nch <= 1) return;
  const int D = p.dvo;
  const int d0 = li * 4;
  // one pass: the LSE, max and O of a block of 8 partial states are loaded
  // together and folded into a running (M, weight sum, acc) that is rescaled
  // when M grows, so the loads of a row need a single round trip
  constexpr int BLK = 8;
  float M = -INFINITY, MX = -INFINITY;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  for (int c0 = 0; c0 < nch; c0 += BLK) {
    float ls[BLK], ms[BLK];
    float4 x[BLK];
#pragma unroll
    for (int k = 0; k < BLK; ++k) {
      const bool ok = c0 + k < nch;
      const int64_t wr = wrow0 + (int64_t)(c0 + k) * WR;
      ls[k] = ok ? p.ws_lse[wr] : -INFINITY;
      ms[k] = ok ? p.ws_mx[wr] : -INFINITY;
      x[k] = ok ? *reinterpret_cast<const float4*>(p.ws_o + wr * D + d0) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float bm = -INFINITY;
#pragma unroll
    for (int k = 0; k < BLK; ++k) {
      bm = fmaxf(bm, ls[k]);
      MX = fmaxf(MX, ms[k]);
    }
    const float Mn = fmaxf(M, bm);
    if (Mn == -INFINITY) continue;  // every state so far is empty
    const float a = M == -INFINITY ? 0.f : fast_exp2((M - Mn) * kLog2e);
    wsum *= a;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] *= a;
#pragma unroll
    for (int k = 0; k < BLK; ++k) {
      const float w = ls[k] == -INFINITY ? 0.f : fast_exp2((ls[k] - Mn) * kLog2e);
      wsum += w;
      acc[0] = fmaf(w, x[k].x, acc[0]);
      acc[1] = fmaf(w, x[k].y, acc[1]);
      acc[2] = fmaf(w, x[k].z, acc[2]);
      acc[3] = fmaf(w, x[k].w, acc[3]);
    }
    M = Mn;
  }
  if (M != -INFINITY) {
    const float inv = 1.f / wsum;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] *= inv;
  }
  const int qi = r / p.group, qh = r % p.group;
  const int64_t rid = (int64_t)(b * p.q_len + qi) * p.num_qo_heads + (int64_t)g * p.group + qh;
  if (p.o_dtype == F32) store4<F32>(p.o, rid * D + d0, acc);
  else if (p.o_dtype == F16) store4<F16>(p.o, rid * D + d0, acc);
  else store4<BF16>(p.o, rid * D + d0, acc);
  if (li == 0) {
    if (p.lse) p.lse[rid] = M == -INFINITY ? -INFINITY : M + fast_log2(wsum) * kLn2;
    if (p.mx) p.mx[rid] = MX;
  }
}

}  // namespace

hipError_t launch_chunk_merge(const AttnParams& p, hipStream_t stream) {
  const int tpr = p.dvo / 4;
  const int rpb = 256 / tpr;
  const int64_t total = (int64_t)p.batch * p.num_kv_heads * p.ws_rows;
  const dim3 grid((unsigned)((total + rpb - 1) / rpb));
  chunk_merge_kernel<<<grid, dim3(rpb * tpr), 0, stream>>>(p, tpr);
  return hipGetLastError();
}

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
