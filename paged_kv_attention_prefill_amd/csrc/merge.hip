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

// Where the partial states of folded row (b, KV head g, r) of a balanced split
// sit: the number of states and the workspace row of the first (the next ones
// are WR rows apart).  The states of item (b, g) sit in slots item + i for its
// shares i = first..last.
__device__ __forceinline__ int row_states(const AttnParams& p, int b, int g, int r,
                                          int64_t& wrow0) {
  const int WR = p.ws_rows;
  const int item = b * p.num_kv_heads + g;
  const int i0 = p.ws_seg[2 * item], i1 = p.ws_seg[2 * item + 1];
  wrow0 = ((int64_t)item + i0) * WR + r;
  return i1 - i0 + 1;
}

// Partial O elements per lane in the balanced split's merges: one 16-byte load
// per state, four fp32 or eight bf16 elements.
template <int VT>
constexpr int epl() { return VT == F32 ? 4 : 8; }

// EPL consecutive partial-O elements of type VT (fp32 or bf16) as fp32.
template <int VT>
__device__ __forceinline__ void load_part(const void* base, int64_t idx, float (&x)[epl<VT>()]) {
  if constexpr (VT == F32) {
    const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
  } else {
    const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
      x[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
    }
  }
}

// Running merge state of one lane: LSE maximum M, weight sum, the lane's EPL
// output dims, and the row maximum MX.
template <int EPL>
struct Fold {
  float M = -INFINITY, MX = -INFINITY, wsum = 0.f;
  float acc[EPL] = {};
};

// Folds states [c0, c1) of a row: the LSE, max and O of a block of 8 partial
// states are loaded together and folded into the running state, which is
// rescaled when M grows, so a block costs a single memory round trip.  The
// partial O are of element type VT (fp32 or bf16).
template <int VT>
__device__ __forceinline__ void fold_states(const AttnParams& p, int64_t wrow0, int c0, int c1,
                                            int d0, Fold<epl<VT>()>& f) {
  constexpr int kEPL = epl<VT>();
  const int WR = p.ws_rows;
  const int D = p.dvo;
  constexpr int BLK = 8;
  for (int cb = c0; cb < c1; cb += BLK) {
    float ls[BLK], ms[BLK];
    float x[BLK][kEPL];
#pragma unroll
    for (int k = 0; k < BLK; ++k) {
      const bool ok = cb + k < c1;
      const int64_t wr = wrow0 + (int64_t)(cb + k) * WR;
      ls[k] = ok ? p.ws_lse[wr] : -INFINITY;
      ms[k] = ok ? p.ws_mx[wr] : -INFINITY;
      if (ok) {
        load_part<VT>(p.ws_o, wr * D + d0, x[k]);
      } else {
#pragma unroll
        for (int i = 0; i < kEPL; ++i) x[k][i] = 0.f;
      }
    }
    float bm = -INFINITY;
#pragma unroll
    for (int k = 0; k < BLK; ++k) {
      bm = fmaxf(bm, ls[k]);
      f.MX = fmaxf(f.MX, ms[k]);
    }
    const float Mn = fmaxf(f.M, bm);
    if (Mn == -INFINITY) continue;  // every state so far is empty
    const float a = f.M == -INFINITY ? 0.f : fast_exp2((f.M - Mn) * kLog2e);
    f.wsum *= a;
#pragma unroll
    for (int i = 0; i < kEPL; ++i) f.acc[i] *= a;
#pragma unroll
    for (int k = 0; k < BLK; ++k) {
      const float w = ls[k] == -INFINITY ? 0.f : fast_exp2((ls[k] - Mn) * kLog2e);
      f.wsum += w;
#pragma unroll
      for (int i = 0; i < kEPL; ++i) f.acc[i] = fmaf(w, x[k][i], f.acc[i]);
    }
    f.M = Mn;
  }
}

// Normalises a row's merged state and writes O (EPL dims per lane), LSE and max.
template <int kEPL>
__device__ __forceinline__ void store_row(const AttnParams& p, int b, int g, int r, int d0, int li,
                                          Fold<kEPL>& f) {
  if (f.M != -INFINITY) {
    const float inv = 1.f / f.wsum;
#pragma unroll
    for (int i = 0; i < kEPL; ++i) f.acc[i] *= inv;
  }
  const int D = p.dvo;
  const int qi = r / p.group, qh = r % p.group;
  const int64_t rid = (int64_t)(b * p.q_len + qi) * p.num_qo_heads + (int64_t)g * p.group + qh;
#pragma unroll
  for (int h = 0; h < kEPL; h += 4) {
    const float(&a)[4] = *reinterpret_cast<const float(*)[4]>(&f.acc[h]);
    if (p.o_dtype == F32) store4<F32>(p.o, rid * D + d0 + h, a);
    else if (p.o_dtype == F16) store4<F16>(p.o, rid * D + d0 + h, a);
    else store4<BF16>(p.o, rid * D + d0 + h, a);
  }
  if (li == 0) {
    if (p.lse) p.lse[rid] = f.M == -INFINITY ? -INFINITY : f.M + fast_log2(f.wsum) * kLn2;
    if (p.mx) p.mx[rid] = f.MX;
  }
}

// Merge of the balanced split's partial states (the same LSE formula):
// one group of D/EPL lanes per folded row (b, KV head g, row r < q_len*G; the
// workspace's padding row slots get no lanes); rows whose item was done in one
// piece were written directly by the attention kernel and are skipped here.
template <int VT>
__global__ __launch_bounds__(256) void chunk_merge_kernel(AttnParams p, int tpr) {
  const int rpb = blockDim.x / tpr;
  const int64_t rho = (int64_t)blockIdx.x * rpb + threadIdx.x / tpr;
  const int li = threadIdx.x % tpr;
  const int R = p.q_len * p.group;
  const int64_t total = (int64_t)p.batch * p.num_kv_heads * R;
  if (threadIdx.x >= rpb * tpr || rho >= total) return;
  const int r = (int)(rho % R);
  const int g = (int)((rho / R) % p.num_kv_heads);
  const int b = (int)(rho / ((int64_t)R * p.num_kv_heads));
  int64_t wrow0;
  const int nch = row_states(p, b, g, r, wrow0);
  if (nch <= 1) return;
  const int d0 = li * epl<VT>();
  Fold<epl<VT>()> f;
  fold_states<VT>(p, wrow0, 0, nch, d0, f);
  store_row(p, b, g, r, d0, li, f);
}

// The same merge for rows with many states (few long items split over many
// workgroups): one workgroup per folded row, its NG = 256 / (D/EPL) lane groups
// each folding an equal contiguous share of the states, then lane group 0
// combining the NG shares in group order through LDS (a fixed order, so the
// result does not depend on timing).
template <int VT>
__global__ __launch_bounds__(256) void chunk_merge_wide_kernel(AttnParams p, int tpr) {
  __shared__ float4 s_acc[2][256];
  __shared__ float s_m[256], s_w[256], s_x[256];
  const int NG = blockDim.x / tpr;
  const int R = p.q_len * p.group;
  const int64_t rho = blockIdx.x;  // (b, g, r < R)
  const int r = (int)(rho % R);
  const int g = (int)((rho / R) % p.num_kv_heads);
  const int b = (int)(rho / ((int64_t)R * p.num_kv_heads));
  const int k = threadIdx.x / tpr, li = threadIdx.x % tpr;
  int64_t wrow0;
  const int nch = row_states(p, b, g, r, wrow0);
  if (nch <= 1) return;  // uniform over the workgroup
  constexpr int kEPL = epl<VT>();
  const int d0 = li * kEPL;
  const int per = (nch + NG - 1) / NG;
  Fold<kEPL> f;
  if (k < NG) fold_states<VT>(p, wrow0, min(nch, k * per), min(nch, (k + 1) * per), d0, f);
#pragma unroll
  for (int h = 0; h < kEPL; h += 4)
    s_acc[h / 4][threadIdx.x] = make_float4(f.acc[h], f.acc[h + 1], f.acc[h + 2], f.acc[h + 3]);
  if (li == 0 && k < NG) {
    s_m[k] = f.M;
    s_w[k] = f.wsum;
    s_x[k] = f.MX;
  }
  __syncthreads();
  if (k != 0) return;
  Fold<kEPL> t;
  for (int j = 0; j < NG; ++j) t.M = fmaxf(t.M, s_m[j]);
  if (t.M != -INFINITY) {
    for (int j = 0; j < NG; ++j) {
      const float mj = s_m[j];
      const float a = mj == -INFINITY ? 0.f : fast_exp2((mj - t.M) * kLog2e);
      t.wsum = fmaf(a, s_w[j], t.wsum);
#pragma unroll
      for (int h = 0; h < kEPL; h += 4) {
        const float4 v = s_acc[h / 4][j * tpr + li];
        t.acc[h] = fmaf(a, v.x, t.acc[h]);
        t.acc[h + 1] = fmaf(a, v.y, t.acc[h + 1]);
        t.acc[h + 2] = fmaf(a, v.z, t.acc[h + 2]);
        t.acc[h + 3] = fmaf(a, v.w, t.acc[h + 3]);
      }
    }
  }
  for (int j = 0; j < NG; ++j) t.MX = fmaxf(t.MX, s_x[j]);
  store_row(p, b, g, r, d0, li, t);
}

template <int VT>
hipError_t launch_chunk_merge_vt(const AttnParams& p, bool wide, hipStream_t stream) {
  const int tpr = p.dvo / epl<VT>();
  if (wide) {
    const int64_t rows = (int64_t)p.batch * p.num_kv_heads * p.q_len * p.group;
    if (rows == 0) return hipSuccess;
    chunk_merge_wide_kernel<VT><<<(unsigned)rows, 256 / tpr * tpr, 0, stream>>>(p, tpr);
    return hipGetLastError();
  }
  const int rpb = 256 / tpr;
  const int64_t total = (int64_t)p.batch * p.num_kv_heads * p.q_len * p.group;
  if (total == 0) return hipSuccess;
  const dim3 grid((unsigned)((total + rpb - 1) / rpb));
  chunk_merge_kernel<VT><<<grid, dim3(rpb * tpr), 0, stream>>>(p, tpr);
  return hipGetLastError();
}

}  // namespace

// The workspace's partial O are of type ws_dtype: fp32 or bf16.
hipError_t launch_chunk_merge(const AttnParams& p, bool wide, hipStream_t stream) {
  if (p.ws_dtype == F32) return launch_chunk_merge_vt<F32>(p, wide, stream);
  return launch_chunk_merge_vt<BF16>(p, wide, stream);
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
