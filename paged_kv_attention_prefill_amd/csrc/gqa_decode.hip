// GQA paged decode on MFMA: the q_len x G query rows that share one KV head are
// folded into the N side of 16x16x32 MFMA tiles (the fold of query tokens into
// heads of the FlashInfer PR #3309 analysis, code section 1, used here to feed
// one KV load to every row of the group).
//
// Per wave and 32-token tile (the streaming core, stream_range):
//   page ids of a 64-page window sit in registers (lane i: page wbase+i) and
//   are fetched per token with a lane shuffle, so no dependent table load sits
//   between tiles;
//   K: each lane loads 16 B (8 elements) of two token rows straight into the
//   MFMA A-operand layout (token = lane%16 [+16], dims 32kk + 8*(lane/16));
//   with equal K/V strides the V offset is the K offset (the SAME_KV_STRIDES
//   specialisation of the FlashInfer PR #4736 analysis, code section 2);
//   S^T[token][row] = K Q^T (Q^T is the B operand, loaded once); mask (KV end,
//   causal position, rows beyond the group), scale, online softmax (running
//   max m, running sum l, rescale by exp2(m_old - m_new)) with wavefront
//   reductions across the four 16-lane groups;
//   V rows go to the wave's LDS tile (invalid tokens as zeros) and come back
//   transposed (ds_read_b64_tr_b16) as the A operand of O^T += V^T P^T; P^T is
//   exactly the score registers converted to 16-bit (no shuffles).
//
// A workgroup = (KV head, query batch, KV chunk or explicit split) with four
// waves that take the range's tiles round-robin and merge their states in LDS
// at the end — the in-workgroup split-and-merge of the SM110 XQA split kernel
// (kernel-design section).  (Measured on MI355X: one wave per KV head with the
// waves of a workgroup reading the same pages, and two tiles in flight per
// wave, were both slower for the Llama-70B-like decode.)
// Internal chunking cuts long KV batches into fixed-size chunks whose partial
// states (O normalised by the chunk's own sum, LSE, max) go to the workspace for
// the chunk-merge launch; explicit splits write the caller's partial states.
#include "mfma_common.h"

namespace pa {
namespace {

constexpr int kTile = 32;

template <int D>
struct Geo {
  static constexpr int KK = D / 32;          // 32-dim k-steps of Q.K
  static constexpr int NDT = D / 16;         // 16-dim tiles of O
  static constexpr int ROWB = D * 2 + 32;    // LDS pitch of a V row (pad: conflict-free tr reads)
  static constexpr int VBUF = kTile * ROWB;  // bytes of one wave's V tile
};

// Token range of work item c of a KV batch with n pages / L tokens.
// Returns false if the item does not exist (beyond the batch's chunks).
__device__ __forceinline__ bool item_range(const AttnParams& p, int c, int n, int L, int& j0,
                                           int& j1, bool& to_ws) {
  to_ws = false;
  if (p.chunk_tokens > 0) {
    const int nch = num_chunks(L, p.chunk_tokens, p.max_chunks);
    if (c >= nch) return false;
    j0 = c * p.chunk_tokens;
    j1 = (c == nch - 1) ? L : j0 + p.chunk_tokens;
    to_ws = nch > 1;
  } else {
    const int S = p.num_splits;
    j0 = (int)(((int64_t)c * n / S) * p.page_size);
    j1 = min((int)(((int64_t)(c + 1) * n / S) * p.page_size), L);
  }
  return true;
}

// Q^T B operand of this lane's row (lane%16), zero for rows beyond q_len*G.
template <int D>
__device__ __forceinline__ void load_q(const AttnParams& p, int b, int g, int row, int lg,
                                       i16x8_t (&qreg)[Geo<D>::KK]) {
  const int R = p.q_len * p.group;
  const bool ok = row < R;
  const int qi = ok ? row / p.group : 0;
  const int qh = ok ? row % p.group : 0;
  const uint16_t* qp = static_cast<const uint16_t*>(p.q) +
                       ((int64_t)(b * p.q_len + qi) * p.num_qo_heads + (int64_t)g * p.group + qh) * D +
                       8 * lg;
#pragma unroll
  for (int kk = 0; kk < Geo<D>::KK; ++kk) {
    const uint4 v = ok ? *reinterpret_cast<const uint4*>(qp + 32 * kk) : make_uint4(0, 0, 0, 0);
    qreg[kk] = as_i16x8(v);
  }
}

// Stream tiles k = tfirst, tfirst + tstep, ... of [j0, j1) for KV head g.  Each
// wave has one 16 KB tile in flight; latency is hidden across the resident waves.
template <int DT, int D, bool SAME>
__device__ __forceinline__ void stream_range(const AttnParams& p, int g, int pbeg, int j0, int j1,
                                             int row_lim, const i16x8_t (&qreg)[Geo<D>::KK],
                                             int tfirst, int tstep, uint8_t* vbuf, float& m,
                                             float& lsum, f32x4_t (&oacc)[Geo<D>::NDT]) {
  constexpr int KK = Geo<D>::KK, NDT = Geo<D>::NDT, ROWB = Geo<D>::ROWB;
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15, lg = lane >> 4;
  const int P = p.page_size;
  const float qk_scale = p.sm_scale * p.k_scale * kLog2e;
  const uint16_t* kbase = static_cast<const uint16_t*>(p.k);
  const uint16_t* vbase = static_cast<const uint16_t*>(p.v);
  if (j1 <= j0) return;
  const int pfirst = j0 / P, plast = (j1 - 1) / P;
  for (int wbase = pfirst; wbase <= plast; wbase += 64) {
    const int pid = wbase + lane <= plast ? p.kv_indices[pbeg + wbase + lane] : 0;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the window is in registers
    const int ws_tok = max(j0, wbase * P);
    const int we_tok = min(j1, (wbase + 64) * P);
    const int kbeg = (ws_tok - j0 + kTile - 1) / kTile;
    const int kend = (we_tok - j0 + kTile - 1) / kTile;
    int tile = tfirst;
    if (tile < kbeg) tile += (kbeg - tile + tstep - 1) / tstep * tstep;
    for (; tile < kend; tile += tstep) {
      const int jb = j0 + tile * kTile;
      uint4 kr[2][KK], vr[2][KK];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int j = jb + 16 * st + l16;
        const int jj = j < j1 ? j : j1 - 1;  // a valid token of this batch: no stray reads
        const int64_t page = __shfl(pid, jj / P - wbase, 64);
        const int slot = jj % P;
        const int64_t koff = page * p.ks0 + slot * p.ks1 + (int64_t)g * p.ks2 + 8 * lg;
        const int64_t voff = SAME ? koff : page * p.vs0 + slot * p.vs1 + (int64_t)g * p.vs2 + 8 * lg;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          kr[st][kk] = *reinterpret_cast<const uint4*>(kbase + koff + 32 * kk);
          vr[st][kk] = *reinterpret_cast<const uint4*>(vbase + voff + 32 * kk);
        }
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const bool ok = jb + 16 * st + l16 < j1;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          *reinterpret_cast<uint4*>(vbuf + (16 * st + l16) * ROWB + (32 * kk + 8 * lg) * 2) =
              ok ? vr[st][kk] : make_uint4(0, 0, 0, 0);
      }
      f32x4_t sacc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int st = 0; st < 2; ++st) sacc[st] = mfma16<DT>(as_i16x8(kr[st][kk]), qreg[kk], sacc[st]);

      float s[2][4];
      float tmax = -INFINITY;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = jb + 16 * st + 4 * lg + i;
          s[st][i] = j < row_lim ? sacc[st][i] * qk_scale : -INFINITY;
          tmax = fmaxf(tmax, s[st][i]);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float mnew = fmaxf(m, tmax);
      const float mref = mnew == -INFINITY ? 0.f : mnew;
      const float alpha = fast_exp2(m - mref);
      float pr[2][4];
      float psum = 0.f;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pr[st][i] = fast_exp2(s[st][i] - mref);
          psum += pr[st][i];
        }
      lsum = fmaf(lsum, alpha, psum);
      m = mnew;
#pragma unroll
      for (int t = 0; t < NDT; ++t) oacc[t] *= alpha;

      const uint4 pbits = make_uint4(pack2<DT>(pr[0][0], pr[0][1]), pack2<DT>(pr[0][2], pr[0][3]),
                                     pack2<DT>(pr[1][0], pr[1][1]), pack2<DT>(pr[1][2], pr[1][3]));
      const i16x8_t pb = as_i16x8(pbits);
      lds_wait();
      const uint16_t* r0 = reinterpret_cast<const uint16_t*>(vbuf + (4 * lg + (l16 >> 2)) * ROWB) +
                           4 * (l16 & 3);
      const uint16_t* r1 = r0 + 16 * (ROWB / 2);
#pragma unroll
      for (int t = 0; t < NDT; ++t) {
        const i16x4_t lo = lds_read_tr(r0 + 16 * t);
        const i16x4_t hi = lds_read_tr(r1 + 16 * t);
        const i16x8_t va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        oacc[t] = mfma16<DT>(va, pb, oacc[t]);
      }
    }
  }
}

// Store EPT consecutive output elements of one row (final O or workspace partial).
template <int EPT>
__device__ __forceinline__ void store_row(const AttnParams& p, bool to_ws, int64_t idx,
                                         const float* x, float scale) {
  if (to_ws || p.o_dtype == F32) {
    float* op = (to_ws ? p.ws_o : static_cast<float*>(p.o)) + idx;
#pragma unroll
    for (int e = 0; e < EPT; e += 4)
      *reinterpret_cast<float4*>(op + e) =
          make_float4(x[e] * scale, x[e + 1] * scale, x[e + 2] * scale, x[e + 3] * scale);
  } else {
    uint32_t* op = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(p.o) + idx);
#pragma unroll
    for (int e = 0; e < EPT; e += 2)
      op[e / 2] = p.o_dtype == F16 ? pack2<F16>(x[e] * scale, x[e + 1] * scale)
                                   : pack2<BF16>(x[e] * scale, x[e + 1] * scale);
  }
}

__device__ __forceinline__ void store_stats(const AttnParams& p, bool to_ws, int64_t ws_row,
                                            int64_t sidx, float M, float Lt) {
  const bool empty = !(Lt > 0.f);
  const float lse = empty ? -INFINITY : (M + fast_log2(Lt)) * kLn2;
  const float mx = empty ? -INFINITY : M * kLn2;
  if (to_ws) {
    p.ws_lse[ws_row] = lse;
    p.ws_mx[ws_row] = mx;
  } else {
    if (p.lse) p.lse[sidx] = lse;
    if (p.mx) p.mx[sidx] = mx;
  }
}

// ---------------------------------------------------------------- split kernel
template <int DT, int D, bool SAME, int NW>
__global__ __launch_bounds__(64 * NW) void gqa_decode_split_kernel(AttnParams p) {
  constexpr int NDT = Geo<D>::NDT;
  constexpr int MERGE_BYTES = NW * 16 * D * 4 + NW * 16 * 2 * 4;
  constexpr int SMEM = (NW * Geo<D>::VBUF > MERGE_BYTES) ? NW * Geo<D>::VBUF : MERGE_BYTES;
  __shared__ __align__(16) uint8_t smem[SMEM];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int g = blockIdx.x;
  const int b = blockIdx.y;
  const int c = blockIdx.z;
  const int kb = p.broadcast ? 0 : b;
  const int pbeg = p.kv_indptr[kb];
  const int n = p.kv_indptr[kb + 1] - pbeg;
  const int L = n ? (n - 1) * p.page_size + p.kv_last[kb] : 0;
  int j0, j1;
  bool to_ws;
  if (!item_range(p, c, n, L, j0, j1, to_ws)) return;

  const int R = p.q_len * p.group;
  i16x8_t qreg[Geo<D>::KK];
  load_q<D>(p, b, g, l16, lg, qreg);
  int row_lim = j1;
  if (p.causal) row_lim = min(row_lim, L - p.q_len + (l16 < R ? l16 / p.group : 0) + 1);
  if (l16 >= R) row_lim = INT_MIN;

  float m = -INFINITY, lsum = 0.f;
  f32x4_t oacc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) oacc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  stream_range<DT, D, SAME>(p, g, pbeg, j0, j1, row_lim, qreg, w, NW, smem + w * Geo<D>::VBUF, m,
                            lsum, oacc);

  // merge the waves' states in LDS
  float ltot = lsum + __shfl_xor(lsum, 16, 64);
  ltot += __shfl_xor(ltot, 32, 64);
  __syncthreads();
  float* obuf = reinterpret_cast<float*>(smem);  // [NW][16][D]
  float* stat = obuf + NW * 16 * D;              // [NW][16][2]
#pragma unroll
  for (int t = 0; t < NDT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) obuf[(w * 16 + l16) * D + 16 * t + 4 * lg + i] = oacc[t][i];
  if (lg == 0) {
    stat[(w * 16 + l16) * 2] = m;
    stat[(w * 16 + l16) * 2 + 1] = ltot;
  }
  __syncthreads();

  constexpr int EPT = (16 * D) / (64 * NW);  // output elements per thread
  constexpr int TPR = D / EPT;               // threads per row
  static_assert(EPT >= 4 && (EPT % 4) == 0, "merge mapping");
  const int orow = threadIdx.x / TPR;
  const int d0 = (threadIdx.x % TPR) * EPT;
  if (orow >= R) return;
  float M = -INFINITY;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, stat[(ww * 16 + orow) * 2]);
  const float Mref = M == -INFINITY ? 0.f : M;
  float Lt = 0.f;
  float acc[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) acc[e] = 0.f;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) {
    const float cw = fast_exp2(stat[(ww * 16 + orow) * 2] - Mref);
    Lt = fmaf(cw, stat[(ww * 16 + orow) * 2 + 1], Lt);
#pragma unroll
    for (int e = 0; e < EPT; ++e) acc[e] = fmaf(cw, obuf[(ww * 16 + orow) * D + d0 + e], acc[e]);
  }
  const float scale = Lt > 0.f ? p.v_scale / Lt : 0.f;
  const int oi = orow / p.group, oh = orow % p.group;
  const int64_t rid = (int64_t)(b * p.q_len + oi) * p.num_qo_heads + (int64_t)g * p.group + oh;
  const int64_t ws_row = ((int64_t)(b * p.num_kv_heads + g) * p.max_chunks + c) * 16 + orow;
  store_row<EPT>(p, to_ws, (to_ws ? ws_row * D : c * p.o_split_stride + rid * D) + d0, acc, scale);
  if (d0 == 0) store_stats(p, to_ws, ws_row, c * p.s_split_stride + rid, M, Lt);
}

template <int DT, int D>
hipError_t launch_d(const AttnParams& p, bool same, hipStream_t stream) {
  constexpr int NW = 4;
  const dim3 grid(p.num_kv_heads, p.batch, p.chunk_tokens > 0 ? p.max_chunks : p.num_splits);
  if (same)
    gqa_decode_split_kernel<DT, D, true, NW><<<grid, 64 * NW, 0, stream>>>(p);
  else
    gqa_decode_split_kernel<DT, D, false, NW><<<grid, 64 * NW, 0, stream>>>(p);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const AttnParams& p, bool same, hipStream_t stream) {
  if (p.dqk == 64) return launch_d<DT, 64>(p, same, stream);
  if (p.dqk == 128) return launch_d<DT, 128>(p, same, stream);
  if (p.dqk == 256) return launch_d<DT, 256>(p, same, stream);
  return hipErrorInvalidValue;
}

}  // namespace

bool gqa_decode_supported(const AttnParams& p) {
  return p.qo_indptr == nullptr && p.q_dtype == p.kv_dtype && (p.q_dtype == BF16 || p.q_dtype == F16) &&
         p.dqk == p.dvo && (p.dqk == 64 || p.dqk == 128 || p.dqk == 256) &&
         p.q_len * p.group <= 16;
}

hipError_t launch_gqa_decode(const AttnParams& p, bool same_strides, hipStream_t stream) {
  if (p.q_dtype == BF16) return launch_dt<BF16>(p, same_strides, stream);
  return launch_dt<F16>(p, same_strides, stream);
}

}  // namespace pa
