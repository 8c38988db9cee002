// Generic paged attention kernel: vector ALU, fp32 arithmetic, any supported
// dtype combination and head dims, decode or prefill, causal, broadcast, split
// states.  It is the exact-fp32 path (fp32 caches) and the fallback for shapes
// the MFMA kernels do not cover.
//
// One workgroup owns one (query token t, KV head g, block of up to 8 query
// heads of g's group) and one KV split; its four waves take the item's KV tokens
// in groups of U, group q going to wave q mod 4, and merge their four states in
// LDS at the end (the in-workgroup split and merge of the SM110 XQA split
// kernel, kernel-design section).  Lanes own head-dim elements d = lane + 64*c.
// Per KV token: page-table walk, K row load, dot products reduced across the
// wavefront, online softmax (running max m, running sum l, rescale by
// exp(m_old - m_new)), O accumulation with the V row.
// Online softmax as merged partial states: "Move the Query, Not the Cache"
// summary, method section.
#include "device_common.h"

namespace pa {
namespace {

constexpr int kHB = 8;      // query heads per item
constexpr int kWaves = 4;   // wavefronts per workgroup, all on one item

template <int QT, int KT, int DQC, int DVC>
__global__ __launch_bounds__(256) void generic_attn_kernel(AttnParams p, int n_hb, int64_t n_items) {
  // the waves' states, merged at the end
  __shared__ float s_o[kWaves][kHB][DVC * 64];
  __shared__ float s_m[kWaves][kHB], s_l[kWaves][kHB];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int64_t item = blockIdx.x;
  if (item >= n_items) return;  // uniform over the workgroup
  const int hb = (int)(item % n_hb);
  const int64_t rest = item / n_hb;
  const int g = (int)(rest % p.num_kv_heads);
  const int t = (int)(rest / p.num_kv_heads);

  const int b = batch_of_token(p, t);
  const int q0 = p.qo_indptr ? p.qo_indptr[b] : b * p.q_len;
  const int qb = p.qo_indptr ? p.qo_indptr[b + 1] - q0 : p.q_len;
  const int kb = p.broadcast ? 0 : b;
  const int pbeg = p.kv_indptr[kb];
  const int n = p.kv_indptr[kb + 1] - pbeg;
  const int64_t L = n ? (int64_t)(n - 1) * p.page_size + p.kv_last[kb] : 0;
  const int64_t pos = L - qb + (t - q0);
  const int c = blockIdx.y;
  const int S = p.num_splits;
  const int64_t j0 = ((int64_t)c * n / S) * p.page_size;
  int64_t j1 = ((int64_t)(c + 1) * n / S) * p.page_size;
  if (j1 > L) j1 = L;
  if (p.causal && j1 > pos + 1) j1 = pos + 1;

  const int h0 = g * p.group + hb * kHB;
  const int nh = min(kHB, p.group - hb * kHB);

  float qf[kHB][DQC];
#pragma unroll
  for (int r = 0; r < kHB; ++r) {
#pragma unroll
    for (int cc = 0; cc < DQC; ++cc) {
      const int d = lane + 64 * cc;
      qf[r][cc] = (r < nh && d < p.dqk)
                      ? load_elem<QT>(p.q, ((int64_t)t * p.num_qo_heads + h0 + r) * p.dqk + d)
                      : 0.f;
    }
  }
  float of[kHB][DVC];
  float m[kHB], l[kHB];
#pragma unroll
  for (int r = 0; r < kHB; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.f;
#pragma unroll
    for (int cc = 0; cc < DVC; ++cc) of[r][cc] = 0.f;
  }
  const float qk_scale = p.sm_scale * p.k_scale * kLog2e;

  // U tokens per step: their page ids, K and V rows are loaded together (no
  // load waits on another), then folded in token order
  constexpr int U = DQC + DVC <= 4 ? 8 : DQC + DVC <= 8 ? 4 : 1;
  for (int64_t j = j0 + (int64_t)w * U; j < j1; j += (int64_t)kWaves * U) {
    float kf[U][DQC], vf[U][DVC];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t jj = j + u < j1 ? j + u : j1 - 1;  // a valid token
      const int64_t page = p.kv_indices[pbeg + (int)(jj / p.page_size)];
      const int64_t slot = jj % p.page_size;
      const int64_t kbase = page * p.ks0 + slot * p.ks1 + (int64_t)g * p.ks2;
      const int64_t vbase = page * p.vs0 + slot * p.vs1 + (int64_t)g * p.vs2;
#pragma unroll
      for (int cc = 0; cc < DQC; ++cc) {
        const int d = lane + 64 * cc;
        kf[u][cc] = d < p.dqk ? load_elem<KT>(p.k, kbase + d) : 0.f;
      }
#pragma unroll
      for (int cc = 0; cc < DVC; ++cc) {
        const int d = lane + 64 * cc;
        vf[u][cc] = d < p.dvo ? load_elem<KT>(p.v, vbase + d) : 0.f;
      }
    }
#pragma unroll
    for (int r = 0; r < kHB; ++r) {
      if (r >= nh) break;
      float s[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float part = 0.f;
#pragma unroll
        for (int cc = 0; cc < DQC; ++cc) part = fmaf(qf[r][cc], kf[u][cc], part);
        s[u] = wave_allreduce_sum(part) * qk_scale;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (j + u >= j1) break;
        const float mn = fmaxf(m[r], s[u]);
        const float a = fast_exp2(m[r] - mn);
        const float pr = fast_exp2(s[u] - mn);
        l[r] = fmaf(l[r], a, pr);
#pragma unroll
        for (int cc = 0; cc < DVC; ++cc) of[r][cc] = fmaf(of[r][cc], a, pr * vf[u][cc]);
        m[r] = mn;
      }
    }
  }

  // merge: wave w finishes heads w, w + 4, ... of the block
#pragma unroll
  for (int r = 0; r < kHB; ++r) {
#pragma unroll
    for (int cc = 0; cc < DVC; ++cc) s_o[w][r][64 * cc + lane] = of[r][cc];
    if (lane == 0) {
      s_m[w][r] = m[r];
      s_l[w][r] = l[r];
    }
  }
  __syncthreads();
  for (int r = w; r < nh; r += kWaves) {
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, s_m[ww][r]);
    const float Mref = M == -INFINITY ? 0.f : M;
    float L = 0.f;
    float acc[DVC];
#pragma unroll
    for (int cc = 0; cc < DVC; ++cc) acc[cc] = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float cw = fast_exp2(s_m[ww][r] - Mref);  // 0 for a wave that saw no token
      L = fmaf(cw, s_l[ww][r], L);
#pragma unroll
      for (int cc = 0; cc < DVC; ++cc) acc[cc] = fmaf(cw, s_o[ww][r][64 * cc + lane], acc[cc]);
    }
    const int64_t row = (int64_t)t * p.num_qo_heads + h0 + r;
    const bool empty = !(L > 0.f);
    const float inv = empty ? 0.f : p.v_scale / L;
#pragma unroll
    for (int cc = 0; cc < DVC; ++cc) {
      const int d = lane + 64 * cc;
      if (d < p.dvo) {
        const int64_t idx = c * p.o_split_stride + row * p.dvo + d;
        const float val = acc[cc] * inv;
        if (p.o_dtype == F32) store_elem<F32>(p.o, idx, val);
        else if (p.o_dtype == F16) store_elem<F16>(p.o, idx, val);
        else store_elem<BF16>(p.o, idx, val);
      }
    }
    if (lane == 0) {
      const int64_t sidx = c * p.s_split_stride + row;
      if (p.lse) p.lse[sidx] = empty ? -INFINITY : (M + fast_log2(L)) * kLn2;
      if (p.mx) p.mx[sidx] = empty ? -INFINITY : M * kLn2;
    }
  }
}

template <int QT, int KT>
hipError_t launch_dims(const AttnParams& p, hipStream_t stream) {
  const int n_hb = (p.group + kHB - 1) / kHB;
  const int64_t n_items = (int64_t)p.total_q * p.num_kv_heads * n_hb;
  if (n_items == 0) return hipSuccess;
  dim3 grid((unsigned)n_items, (unsigned)p.num_splits);
  dim3 block(64 * kWaves);
  if (p.dqk == 64 && p.dvo == 64)
    generic_attn_kernel<QT, KT, 1, 1><<<grid, block, 0, stream>>>(p, n_hb, n_items);
  else if (p.dqk == 128 && p.dvo == 128)
    generic_attn_kernel<QT, KT, 2, 2><<<grid, block, 0, stream>>>(p, n_hb, n_items);
  else if (p.dqk == 256 && p.dvo == 256)
    generic_attn_kernel<QT, KT, 4, 4><<<grid, block, 0, stream>>>(p, n_hb, n_items);
  else if (p.dqk == 576 && p.dvo == 512)
    generic_attn_kernel<QT, KT, 9, 8><<<grid, block, 0, stream>>>(p, n_hb, n_items);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_generic(const AttnParams& p, hipStream_t stream) {
  if (p.q_dtype == F32 && p.kv_dtype == F32) return launch_dims<F32, F32>(p, stream);
  if (p.q_dtype == F16 && p.kv_dtype == F16) return launch_dims<F16, F16>(p, stream);
  if (p.q_dtype == BF16 && p.kv_dtype == BF16) return launch_dims<BF16, BF16>(p, stream);
  if (p.q_dtype == BF16 && p.kv_dtype == FP8) return launch_dims<BF16, FP8>(p, stream);
  if (p.q_dtype == F16 && p.kv_dtype == FP8) return launch_dims<F16, FP8>(p, stream);
  if (p.q_dtype == FP8 && p.kv_dtype == FP8) return launch_dims<FP8, FP8>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
