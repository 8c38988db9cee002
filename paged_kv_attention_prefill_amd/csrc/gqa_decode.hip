// GQA paged decode on MFMA: the q_len x G query rows that share one KV head are
// folded into the N side of 16x16x32 MFMA tiles (the fold of query tokens into
// heads of the FlashInfer PR #3309 analysis, code section 1, used here to feed
// one KV load to every row of the group).
//
// Per wave and 32-token tile (the streaming core, stream_range):
//   K and V rows are fetched whole: 16-byte lanes cover consecutive 16-byte
//   pieces of a token's head row, so one load instruction reads 64/(D/8) full
//   rows (four 256-byte rows at D = 128).  On MI355X this shape streams HBM
//   about 30% faster than loads laid out straight in the MFMA operand order
//   (16 rows x 64 bytes per instruction).  The page of each lane's token comes
//   from the range's page ids staged in LDS, and with equal K/V strides the V offset is the K offset (the SAME_KV_STRIDES
//   specialisation of the FlashInfer PR #4736 analysis, code section 2);
//   the rows pass through the wave's LDS tile: K comes back in the MFMA A
//   layout for S^T[token][row] = K Q^T (Q^T is the B operand, loaded once), V
//   comes back transposed (ds_read_b64_tr_b16) as the A operand of
//   O^T += V^T P^T, P^T being the score registers converted to 16-bit;
//   the wave's next tile's loads are issued as soon as this tile is in LDS, so
//   they are in flight during this tile's math;
//   mask (KV end, causal position, rows beyond the group), online softmax
//   (running max m, running sum l, rescale by exp2(m_old - m_new)) with
//   cross-lane reductions over the four 16-lane groups.
//
// A workgroup = (KV head, query batch, explicit split), or a share of the
// balanced split, with four waves that take the range's tiles round-robin and
// merge their states in LDS at the end — the in-workgroup split-and-merge of the
// SM110 XQA split kernel (kernel-design section).  Pieces of a balanced split
// leave partial states (O normalised by the piece's own sum, LSE, max) in the
// workspace for the merge launch; explicit splits write the caller's partial
// states.
#include "balance.h"
#include "mfma_common.h"

namespace pa {
namespace {

constexpr int kTile = 32;

template <int D>
struct Geo {
  static constexpr int KK = D / 32;          // 32-dim k-steps of Q.K
  static constexpr int NDT = D / 16;         // 16-dim tiles of O
  static constexpr int CPR = D / 8;          // 16-byte pieces per head row
  static constexpr int RPI = 64 / CPR;       // rows per load instruction
  static constexpr int NI = kTile / RPI;     // load instructions per tile (each of K, V)
  // LDS pitch of a K and of a V row: 2D + 32 bytes puts the K operand reads
  // (ds_read_b128: four cycles of 16 lanes, by lane / 32 and the parity of the
  // quad index) and the transposed V reads (two cycles of 32 lanes) on distinct
  // banks of the 64 (as measured with the LDS bank-conflict counter); 2D + 16
  // leaves the K reads 2-way conflicted
  static constexpr int KP = D * 2 + 32;
  static constexpr int VP = D * 2 + 32;
  static constexpr int VBUF = kTile * VP;    // bytes of one wave's tile buffer (K, then V)
};

// Token range of explicit split c of a KV batch with n pages / L tokens: pages
// [c n / S, (c + 1) n / S).
__device__ __forceinline__ void item_range(const AttnParams& p, int c, int n, int L, int& j0, int& j1) {
  const int S = p.num_splits;
  j0 = (int)(((int64_t)c * n / S) * p.page_size);
  j1 = min((int)(((int64_t)(c + 1) * n / S) * p.page_size), L);
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

constexpr int kPageWin = 1024;  // page ids staged in LDS at a time

// Streams [j0, j1) of KV head g: the range's page ids go to LDS (s_pages) a
// window at a time, and the window's 32-token tiles are dealt round-robin to the
// nw waves, so the waves of a workgroup (and the workgroups of the other heads,
// launched next to it) read neighbouring pages together.  Each wave's next tile
// is in flight while its current one is computed; the tile buffer `buf` (LDS,
// per wave) holds K, then V.  Called by every thread of the workgroup (barriers).
template <int DT, int D, bool SAME>
__device__ __forceinline__ void stream_range(const AttnParams& p, int g, int pbeg, int j0, int j1,
                                             int row_lim, const i16x8_t (&qreg)[Geo<D>::KK],
                                             int w, int nw, uint8_t* buf, int* s_pages, float& m,
                                             float& lsum, f32x4_t (&oacc)[Geo<D>::NDT]) {
  using Gm = Geo<D>;
  constexpr int KK = Gm::KK, NDT = Gm::NDT, NI = Gm::NI, RPI = Gm::RPI;
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15, lg = lane >> 4;
  const int rsub = lane / Gm::CPR;  // row of this lane within a load instruction
  const int cch = lane % Gm::CPR;   // its 16-byte piece of the row
  if (j1 <= j0) return;
  const int P = p.page_size;
  const uint32_t pmagic = p.page_magic;
  const float qk_scale = p.sm_scale * p.k_scale * kLog2e;
  const uint16_t* kbase = static_cast<const uint16_t*>(p.k);
  const uint16_t* vbase = static_cast<const uint16_t*>(p.v);
  const uint32_t ks0 = (uint32_t)p.ks0, ks1 = (uint32_t)p.ks1;
  const uint32_t vs0 = (uint32_t)p.vs0, vs1 = (uint32_t)p.vs1;
  const uint32_t kc = (uint32_t)(g * p.ks2) + 8 * cch;
  const uint32_t vc = (uint32_t)(g * p.vs2) + 8 * cch;
  const int pfirst = j0 / P, plast = (j1 - 1) / P;

  for (int wb = pfirst; wb <= plast; wb += kPageWin) {
    const int npw = min(kPageWin, plast - wb + 1);
    __syncthreads();  // the previous window's readers are done
    for (int i = threadIdx.x; i < npw; i += 64 * nw) s_pages[i] = p.kv_indices[pbeg + wb + i];
    __syncthreads();
    const int ws = max(j0, wb * P), we = min(j1, (wb + npw) * P);
    const int nk = (we - ws + kTile - 1) / kTile;
    const int lim = min(row_lim, we);
    i16x8_t kr[NI], vr[NI];
    // loads of window tile k (clamped to the last tile: every path issues them)
    auto issue = [&](int k) __attribute__((always_inline)) {
      const int jb = ws + min(k, nk - 1) * kTile;
      uint64_t koff[NI], voff[NI];
#pragma unroll
      for (int s = 0; s < NI; ++s) {
        const int j = jb + s * RPI + rsub;
        const uint32_t jj = (j < we ? j : we - 1) - wb * P;  // a valid token, window-relative
        // page and slot, division-free (jj * P < 1024 P^2 <= 2^32)
        const uint32_t pi = div_by_magic(jj, pmagic);
        const uint32_t slot = jj - pi * P;
        const uint32_t page = s_pages[pi];
        koff[s] = (uint64_t)page * ks0 + (slot * ks1 + kc);
        voff[s] = SAME ? koff[s] : (uint64_t)page * vs0 + (slot * vs1 + vc);
      }
      // all K rows of the tile, then all V rows; non-temporal (the nt bit): every
      // K/V row is read once per launch, and streaming the cache past L2 and the
      // memory-side cache measured 11% faster (Llama-70B-like decode 197 -> 176 us)
#pragma unroll
      for (int s = 0; s < NI; ++s)
        kr[s] = __builtin_nontemporal_load(reinterpret_cast<const i16x8_t*>(kbase + koff[s]));
#pragma unroll
      for (int s = 0; s < NI; ++s)
        vr[s] = __builtin_nontemporal_load(reinterpret_cast<const i16x8_t*>(vbase + voff[s]));
    };
    if (w < nk) issue(w);
    for (int k = w; k < nk; k += nw) {
      const int jb = ws + k * kTile;
      // K rows -> LDS, back in the MFMA A layout (token l16 [+16], dims 32kk + 8lg)
#pragma unroll
      for (int s = 0; s < NI; ++s)
        *reinterpret_cast<i16x8_t*>(buf + (s * RPI + rsub) * Gm::KP + cch * 16) = kr[s];
      f32x4_t sacc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const i16x8_t a = *reinterpret_cast<const i16x8_t*>(buf + (16 * st + l16) * Gm::KP +
                                                              (32 * kk + 8 * lg) * 2);
          sacc[st] = mfma16<DT>(a, qreg[kk], sacc[st]);
        }
      // V rows -> the same buffer (the K reads above come first: one wave's LDS
      // operations complete in order)
#pragma unroll
      for (int s = 0; s < NI; ++s)
        *reinterpret_cast<i16x8_t*>(buf + (s * RPI + rsub) * Gm::VP + cch * 16) = vr[s];
      issue(k + nw);  // registers are free: the next tile is in flight during the math

      float sv[2][4];
      float tmax = -INFINITY;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = jb + 16 * st + 4 * lg + i;
          sv[st][i] = j < lim ? sacc[st][i] * qk_scale : -INFINITY;
          tmax = fmaxf(tmax, sv[st][i]);
        }
      tmax = xor32_max(xor16_max(tmax));
      const float mnew = fmaxf(m, tmax);
      const float mref = mnew == -INFINITY ? 0.f : mnew;
      const float alpha = fast_exp2(m - mref);
      float pr[2][4];
      float psum = 0.f;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pr[st][i] = fast_exp2(sv[st][i] - mref);
          psum += pr[st][i];
        }
      lsum = fmaf(lsum, alpha, psum);
      m = mnew;
#pragma unroll
      for (int d = 0; d < NDT; ++d) oacc[d] *= alpha;

      const uint4 pbits = make_uint4(pack2<DT>(pr[0][0], pr[0][1]), pack2<DT>(pr[0][2], pr[0][3]),
                                     pack2<DT>(pr[1][0], pr[1][1]), pack2<DT>(pr[1][2], pr[1][3]));
      const i16x8_t pb = as_i16x8(pbits);
      const uint16_t* r0 =
          reinterpret_cast<const uint16_t*>(buf + (4 * lg + (l16 >> 2)) * Gm::VP) + 4 * (l16 & 3);
      const uint16_t* r1 = r0 + 16 * (Gm::VP / 2);
#pragma unroll
      for (int d = 0; d < NDT; ++d) {
        const i16x4_t lo = lds_read_tr(r0 + 16 * d);
        const i16x4_t hi = lds_read_tr(r1 + 16 * d);
        const i16x8_t va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        oacc[d] = mfma16<DT>(va, pb, oacc[d]);
      }
    }
  }
}

// Store EPT consecutive output elements of one row (final O or workspace partial).
template <int EPT>
__device__ __forceinline__ void store_row(const AttnParams& p, bool to_ws, int64_t idx,
                                         const float* x, float scale) {
  if (to_ws || p.o_dtype == F32) {
    float* op = static_cast<float*>(to_ws ? p.ws_o : p.o) + idx;
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
// One (query batch b, KV head g) token range [j0, j1): the waves stream it and
// merge their states in LDS; the result goes to the final O / LSE (split index
// c_out) or, for a partial range, to workspace slot wslot.  Called by every
// thread of the workgroup.
template <int DT, int D, bool SAME, int NW>
__device__ __forceinline__ void decode_range(const AttnParams& p, int b, int g, int L, int j0, int j1,
                                             bool to_ws, int64_t wslot, int c_out, uint8_t* smem,
                                             int* s_pages) {
  constexpr int NDT = Geo<D>::NDT;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int kb = p.broadcast ? 0 : b;
  const int pbeg = p.kv_indptr[kb];

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
  stream_range<DT, D, SAME>(p, g, pbeg, j0, j1, row_lim, qreg, w, NW, smem + w * Geo<D>::VBUF,
                            s_pages, m, lsum, oacc);

  // merge the waves' states in LDS
  const float ltot = xor32_sum(xor16_sum(lsum));
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
  if (orow < R) {
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
    const int64_t ws_row = wslot * 16 + orow;
    store_row<EPT>(p, to_ws, (to_ws ? ws_row * D : c_out * p.o_split_stride + rid * D) + d0, acc, scale);
    if (d0 == 0) store_stats(p, to_ws, ws_row, c_out * p.s_split_stride + rid, M, Lt);
  }
}

// Workgroups: (KV head, query batch, explicit split) on a 3-D grid, or,
// under the balanced split, a 1-D grid whose workgroups walk their share of the
// (batch, KV head, 32-token unit) sequence.
template <int DT, int D, bool SAME, int NW>
__global__ __launch_bounds__(64 * NW, (D > 128 ? 1 : 3)) void gqa_decode_split_kernel(AttnParams p) {
  constexpr int MERGE_BYTES = NW * 16 * D * 4 + NW * 16 * 2 * 4;
  constexpr int SMEM = (NW * Geo<D>::VBUF > MERGE_BYTES) ? NW * Geo<D>::VBUF : MERGE_BYTES;
  __shared__ __align__(16) uint8_t smem[SMEM];
  __shared__ int s_pages[kPageWin];
  if (p.bal_blocks > 0) {
    BalCursor cur;
    if (!cur.start(p, blockIdx.x)) return;
    do {
      decode_range<DT, D, SAME, NW>(p, cur.b, cur.g, cur.L, cur.j0(p), cur.j1(p), !cur.whole(),
                                    cur.slot(p), 0, smem, s_pages);
    } while (cur.next(p));
    return;
  }
  const int g = blockIdx.x;
  const int b = blockIdx.y;
  const int c = blockIdx.z;
  const int kb = p.broadcast ? 0 : b;
  const int n = p.kv_indptr[kb + 1] - p.kv_indptr[kb];
  const int L = n ? (n - 1) * p.page_size + p.kv_last[kb] : 0;
  int j0, j1;
  item_range(p, c, n, L, j0, j1);
  decode_range<DT, D, SAME, NW>(p, b, g, L, j0, j1, false, 0, c, smem, s_pages);
}

template <int DT, int D>
hipError_t launch_d(const AttnParams& p, bool same, hipStream_t stream) {
  constexpr int NW = 4;
  const dim3 grid = p.bal_blocks > 0
                        ? dim3(p.bal_blocks)
                        : dim3(p.num_kv_heads, p.batch, p.num_splits);
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
  // element offsets: page strides fit 32 bits and so does every offset within a
  // page; window-relative token indices (< 1024 pages) times the page size stay
  // below 2^32 (division by the page size as a multiply with its rounded-up
  // reciprocal)
  const int64_t lim = int64_t(1) << 31;
  const bool offsets32 =
      p.ks0 < lim && p.vs0 < lim &&
      (p.page_size - 1) * p.ks1 + (p.num_kv_heads - 1) * p.ks2 + p.dqk < lim &&
      (p.page_size - 1) * p.vs1 + (p.num_kv_heads - 1) * p.vs2 + p.dvo < lim;
  return p.qo_indptr == nullptr && p.q_dtype == p.kv_dtype && (p.q_dtype == BF16 || p.q_dtype == F16) &&
         p.dqk == p.dvo && (p.dqk == 64 || p.dqk == 128 || p.dqk == 256) &&
         p.q_len * p.group <= 16 && offsets32 && p.page_size <= 2048;
}

namespace {
template <int DT, int D>
const void* decode_kernel_ptr(bool same) {
  if (same) return reinterpret_cast<const void*>(&gqa_decode_split_kernel<DT, D, true, 4>);
  return reinterpret_cast<const void*>(&gqa_decode_split_kernel<DT, D, false, 4>);
}
}  // namespace

int gqa_decode_blocks_per_cu(const AttnParams& p, bool same_strides) {
  const void* f = nullptr;
  if (p.q_dtype == BF16)
    f = p.dqk == 64 ? decode_kernel_ptr<BF16, 64>(same_strides)
        : p.dqk == 128 ? decode_kernel_ptr<BF16, 128>(same_strides)
                       : decode_kernel_ptr<BF16, 256>(same_strides);
  else
    f = p.dqk == 64 ? decode_kernel_ptr<F16, 64>(same_strides)
        : p.dqk == 128 ? decode_kernel_ptr<F16, 128>(same_strides)
                       : decode_kernel_ptr<F16, 256>(same_strides);
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, 256, 0) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    n = p.dqk > 128 ? 1 : 3;  // the kernel's launch bounds
  }
  return n;
}

hipError_t launch_gqa_decode(const AttnParams& p, bool same_strides, hipStream_t stream) {
  if (p.q_dtype == BF16) return launch_dt<BF16>(p, same_strides, stream);
  return launch_dt<F16>(p, same_strides, stream);
}

}  // namespace pa
