// Paged flash attention on MFMA for many query rows per KV head: ragged causal
// prefill (the batched paged prefill of the FlashInfer PR #4736 analysis, code
// section 2) and broadcast decode/prefill where every query batch reads one KV
// batch (PyTorch 2.14 MPS FlexAttention post, introduction) — the query rows of
// all batches are folded into the same row tiles so the shared KV is read once
// per tile instead of once per query batch.
//
// Rows: a row is (query token t, query head h) with h in KV group g; a row tile
// holds TQ = 128/G tokens x G heads (r = token_offset*G + head_in_group).
// Without broadcast a tile's tokens come from one query batch; with broadcast
// they run over all query tokens of all batches.
//
// A workgroup = (row tile, KV head g, explicit KV split) with 4 waves of 32
// rows.  Per 64-token KV tile (double-buffered in LDS, loaded cooperatively
// with the page ids of the range staged in LDS):
//   S^T = K Q^T on v_mfma_f32_32x32x16 (K from LDS as the A operand, Q^T from
//   registers as the B operand); causal/length mask; online softmax (running
//   max and sum per row, one lane-pair shuffle per reduction);
//   O^T += V^T P^T with V^T read from LDS by ds_read_b64_tr_b16 and P^T taken
//   straight from the score registers.
// Tiles past a tile's last visible position (causal) are skipped, and tiles of
// late query positions — the heaviest under a causal mask — are dispatched first.
#include "mfma_common.h"

namespace pa {
namespace {

constexpr int kRows = 128;      // rows per workgroup
constexpr int kKT = 64;         // KV tokens per tile
constexpr int kPageWin = 1024;  // page ids staged in LDS at a time

template <int D>
struct FGeo {
  static constexpr int KK = D / 16;            // 16-dim k-steps of Q.K
  static constexpr int NDT = D / 32;           // 32-dim tiles of O
  static constexpr int KP = D * 2 + 16;        // K row pitch (bytes): conflict-free b128 reads
  static constexpr int VP = D * 2 + 32;        // V row pitch (bytes): spread transposed reads
  static constexpr int KBYTES = kKT * KP;
  static constexpr int VBYTES = kKT * VP;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int CPR = D / 8;            // 16-byte chunks per row
  static constexpr int LPT = kKT * CPR / 256;  // chunks per thread per tile (each of K, V)
};

struct RowInfo {
  int64_t t;  // query token (global), -1 if the row is padding
  int h;      // query head
  int lim;    // visible KV tokens are j < lim (causal position + 1, or L)
};

__device__ __forceinline__ int batch_of(const AttnParams& p, int t) { return batch_of_token(p, t); }

template <int DT, int D, bool SAME>
__global__ __launch_bounds__(256, 2) void flash_attn_kernel(AttnParams p, int tiles_per_batch,
                                                           int num_row_tiles) {
  using Gm = FGeo<D>;
  constexpr int KK = Gm::KK, NDT = Gm::NDT;
  __shared__ __align__(16) uint8_t smem[2 * Gm::STAGE];
  __shared__ int s_pages[kPageWin];
  __shared__ int s_red[8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31, h2 = lane >> 5;
  const int G = p.group;
  const int TQ = kRows / G;

  // ---- which (row tile, KV head, split).  Workgroups are dealt round-robin to
  // the 8 XCDs; when the (head, split) groups divide evenly, every group lives on
  // one XCD (its KV stays in that XCD's L2) and each XCD walks its row tiles
  // from the latest (heaviest under a causal mask) to the earliest.
  const int HS = p.num_kv_heads * p.num_splits;
  const int lam = blockIdx.x;
  int rank, gc;
  if (HS % 8 == 0) {
    const int per = HS / 8;
    const int xcd = lam % 8, k = lam / 8;
    rank = k / per;
    gc = xcd + 8 * (k % per);
  } else {
    rank = lam / HS;
    gc = lam % HS;
  }
  const int g = gc % p.num_kv_heads;
  const int c = gc / p.num_kv_heads;
  const int tile_lin = num_row_tiles - 1 - rank;
  int b = 0, t_begin, t_end;  // query tokens [t_begin, t_end) of this tile
  if (p.broadcast) {
    t_begin = tile_lin * TQ;
    t_end = min(t_begin + TQ, p.total_q);
  } else {
    b = tile_lin / tiles_per_batch;
    const int tb = tile_lin % tiles_per_batch;
    const int q0 = p.qo_indptr ? p.qo_indptr[b] : b * p.q_len;
    const int q1 = p.qo_indptr ? p.qo_indptr[b + 1] : q0 + p.q_len;
    t_begin = q0 + tb * TQ;
    t_end = min(t_begin + TQ, q1);
  }
  if (t_begin >= t_end) return;
  const int kb = p.broadcast ? 0 : b;
  const int pbeg = p.kv_indptr[kb];
  const int n = p.kv_indptr[kb + 1] - pbeg;
  const int L = n ? (n - 1) * p.page_size + p.kv_last[kb] : 0;
  const int S = p.num_splits;
  const int j0 = (int)(((int64_t)c * n / S) * p.page_size);
  const int j1 = min((int)(((int64_t)(c + 1) * n / S) * p.page_size), L);

  // ---- this lane's row (B-operand column / C column): wave w rows 32w..32w+31
  RowInfo ri;
  {
    const int r = 32 * w + l32;
    const int64_t t = t_begin + r / G;
    const bool ok = (r / G) < TQ && t < t_end;
    ri.t = ok ? t : -1;
    ri.h = g * G + r % G;
    int lim = j1;
    if (ok && p.causal) {
      const int bb = p.broadcast ? batch_of(p, (int)t) : b;
      const int q0 = p.qo_indptr ? p.qo_indptr[bb] : bb * p.q_len;
      const int qb = p.qo_indptr ? p.qo_indptr[bb + 1] - q0 : p.q_len;
      lim = min(lim, L - qb + ((int)t - q0) + 1);
    }
    ri.lim = ok ? lim : INT_MIN;
  }
  // workgroup-wide last visible token (tiles past it are skipped)
  int hi = ri.lim;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) hi = max(hi, __shfl_xor(hi, off, 64));
  if (lane == 0) s_red[w] = hi;
  __syncthreads();
  const int jhi = min(j1, max(max(s_red[0], s_red[1]), max(s_red[2], s_red[3])));
  // tiles ending at or before this wave's smallest row limit need no mask
  int lo = ri.t >= 0 ? ri.lim : INT_MAX;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) lo = min(lo, __shfl_xor(lo, off, 64));
  const int wave_lim_min = lo;

  // ---- Q^T B operand: 8 x 16 B per lane, kept in registers
  i16x8_t qreg[KK];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(p.q) +
                         ((ri.t < 0 ? 0 : ri.t) * p.num_qo_heads + ri.h) * (int64_t)D + 8 * h2;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const uint4 v = ri.t >= 0 ? *reinterpret_cast<const uint4*>(qp + 16 * kk) : make_uint4(0, 0, 0, 0);
      qreg[kk] = as_i16x8(v);
    }
  }

  float m = -INFINITY, lsum = 0.f;
  f32x16_t oacc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[t][i] = 0.f;
  const float qk_scale = p.sm_scale * p.k_scale * kLog2e;
  const uint16_t* kbase = static_cast<const uint16_t*>(p.k);
  const uint16_t* vbase = static_cast<const uint16_t*>(p.v);
  const int P = p.page_size;
  const int pshift = p.page_shift;
  float true_max = -INFINITY;  // running row max (the lazily updated m may lag it)

  // cooperative tile load: thread -> (chunk cc, tokens tk0 + 16u)
  const int cc = tid % Gm::CPR;
  const int tk0 = tid / Gm::CPR;
  constexpr int TSTEP = 256 / Gm::CPR;

  if (jhi > j0) {
    const int pfirst = j0 / P, plast = (jhi - 1) / P;
    for (int wb = pfirst; wb <= plast; wb += kPageWin) {
      const int npw = min(kPageWin, plast - wb + 1);
      __syncthreads();  // previous window's readers are done
      for (int i = tid; i < npw; i += 256) s_pages[i] = p.kv_indices[pbeg + wb + i];
      __syncthreads();
      const int ws = max(j0, wb * P), we = min(jhi, (wb + npw) * P);
      const int nk = (we - ws + kKT - 1) / kKT;

      uint4 kreg[Gm::LPT], vreg[Gm::LPT];
      auto gload = [&](int jb) {
#pragma unroll
        for (int u = 0; u < Gm::LPT; ++u) {
          const int j = jb + tk0 + TSTEP * u;
          const int jj = j < we ? j : we - 1;  // clamp: a valid token, never a poisoned slot
          const int rel = jj - wb * P;
          const int64_t page = s_pages[pshift >= 0 ? rel >> pshift : rel / P];
          const int slot = pshift >= 0 ? (jj & (P - 1)) : jj % P;
          const int64_t koff = page * p.ks0 + slot * p.ks1 + (int64_t)g * p.ks2 + 8 * cc;
          const int64_t voff = SAME ? koff : page * p.vs0 + slot * p.vs1 + (int64_t)g * p.vs2 + 8 * cc;
          kreg[u] = *reinterpret_cast<const uint4*>(kbase + koff);
          vreg[u] = *reinterpret_cast<const uint4*>(vbase + voff);
        }
      };
      auto lstore = [&](int jb, int stage) {
        uint8_t* kl = smem + stage * Gm::STAGE;
        uint8_t* vl = kl + Gm::KBYTES;
#pragma unroll
        for (int u = 0; u < Gm::LPT; ++u) {
          const int row = tk0 + TSTEP * u;
          *reinterpret_cast<uint4*>(kl + row * Gm::KP + cc * 16) = kreg[u];
          *reinterpret_cast<uint4*>(vl + row * Gm::VP + cc * 16) =
              jb + row < we ? vreg[u] : make_uint4(0, 0, 0, 0);  // V rows past the end read as 0
        }
      };

      gload(ws);
      lstore(ws, 0);
      __syncthreads();
      for (int k = 0; k < nk; ++k) {
        const int jb = ws + k * kKT;
        const int stage = k & 1;
        if (k + 1 < nk) gload(jb + kKT);
        const uint8_t* kl = smem + stage * Gm::STAGE;
        const uint8_t* vl = kl + Gm::KBYTES;

        // S^T[token][row] = K Q^T: two 32-token blocks
        f32x16_t sacc[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) sacc[mb][i] = 0.f;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) {
            const uint4 a = *reinterpret_cast<const uint4*>(kl + (32 * mb + l32) * Gm::KP +
                                                            (16 * kk + 8 * h2) * 2);
            sacc[mb] = mfma32<DT>(as_i16x8(a), qreg[kk], sacc[mb]);
          }

        // mask (boundary tiles only), online softmax (lane: row l32, tokens
        // 32mb + 8(i/4) + 4h2 + i%4).  Scores stay unscaled; the scale is fused
        // into the exponent's FMA.  The reference max m is re-based only when
        // the tile max exceeds it by more than 8 (log2 units), so most tiles skip
        // the O rescale; P <= 2^8 keeps 16-bit P and fp32 sums exact enough, and
        // LSE = m + log2(l) holds for any reference m.
        if (jb + kKT > wave_lim_min) {
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int j = jb + 32 * mb + 8 * (i >> 2) + 4 * h2 + (i & 3);
              sacc[mb][i] = j < ri.lim ? sacc[mb][i] : -INFINITY;
            }
        }
        float tmax = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sacc[mb][i]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64)) * qk_scale;
        true_max = fmaxf(true_max, tmax);
        const bool grow = tmax > m + 8.f;
        if (__ballot(grow)) {
          const float mnew = grow ? tmax : m;
          const float alpha = fast_exp2((m == -INFINITY ? -INFINITY : m) -
                                        (mnew == -INFINITY ? 0.f : mnew));
          const float a = grow ? alpha : 1.f;
          lsum *= a;
#pragma unroll
          for (int t = 0; t < NDT; ++t) oacc[t] *= a;
          m = mnew;
        }
        const float nmref = -(m == -INFINITY ? 0.f : m);
        float psum = 0.f;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float e = fast_exp2(fmaf(sacc[mb][i], qk_scale, nmref));
            sacc[mb][i] = e;
            psum += e;
          }
        lsum += psum;

        // P^T operands of the four 16-token PV steps
        i16x8_t pb[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int mb = t >> 1, i0 = 8 * (t & 1);
          const uint4 bits = make_uint4(pack2<DT>(sacc[mb][i0 + 0], sacc[mb][i0 + 1]),
                                        pack2<DT>(sacc[mb][i0 + 2], sacc[mb][i0 + 3]),
                                        pack2<DT>(sacc[mb][i0 + 4], sacc[mb][i0 + 5]),
                                        pack2<DT>(sacc[mb][i0 + 6], sacc[mb][i0 + 7]));
          pb[t] = as_i16x8(bits);
        }
        // O^T += V^T P^T; V^T via transposed LDS reads
        const int l16 = lane & 15;
        const uint16_t* vrow = reinterpret_cast<const uint16_t*>(vl + (4 * h2 + (l16 >> 2)) * Gm::VP) +
                               16 * ((lane >> 4) & 1) + 4 * (l16 & 3);
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            const uint16_t* ra = vrow + (16 * t) * (Gm::VP / 2) + 32 * dt;
            const i16x4_t lo = lds_read_tr(ra);
            const i16x4_t hi4 = lds_read_tr(ra + 8 * (Gm::VP / 2));
            const i16x8_t va = {lo[0], lo[1], lo[2], lo[3], hi4[0], hi4[1], hi4[2], hi4[3]};
            oacc[dt] = mfma32<DT>(va, pb[t], oacc[dt]);
          }

        if (k + 1 < nk) lstore(jb + kKT, stage ^ 1);
        __syncthreads();
      }
    }
  }

  // ---- epilogue: lane (row l32, half h2) holds dims 32dt + 8q + 4h2 + (0..3)
  const float ltot = lsum + __shfl_xor(lsum, 32, 64);
  if (ri.t < 0) return;
  const bool empty = !(ltot > 0.f);
  const float scale = empty ? 0.f : p.v_scale / ltot;
  const int64_t rid = ri.t * p.num_qo_heads + ri.h;
  const int64_t obase = c * p.o_split_stride + rid * D;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int d = 32 * dt + 8 * q + 4 * h2;
      const float x0 = oacc[dt][4 * q] * scale, x1 = oacc[dt][4 * q + 1] * scale;
      const float x2 = oacc[dt][4 * q + 2] * scale, x3 = oacc[dt][4 * q + 3] * scale;
      if (p.o_dtype == F32) {
        *reinterpret_cast<float4*>(static_cast<float*>(p.o) + obase + d) = make_float4(x0, x1, x2, x3);
      } else if (p.o_dtype == F16) {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.o) + obase + d) =
            make_uint2(pack2<F16>(x0, x1), pack2<F16>(x2, x3));
      } else {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.o) + obase + d) =
            make_uint2(pack2<BF16>(x0, x1), pack2<BF16>(x2, x3));
      }
    }
  if (h2 == 0) {
    const int64_t sidx = c * p.s_split_stride + rid;
    if (p.lse) p.lse[sidx] = empty ? -INFINITY : (m + fast_log2(ltot)) * kLn2;
    if (p.mx) p.mx[sidx] = empty ? -INFINITY : true_max * kLn2;
  }
}

template <int DT, int D>
hipError_t launch_fd(const AttnParams& p, bool same, hipStream_t stream) {
  const int TQ = kRows / p.group;
  int tiles_per_batch = 0, num_row_tiles;
  if (p.broadcast) {
    num_row_tiles = (p.total_q + TQ - 1) / TQ;
  } else {
    tiles_per_batch = (p.max_q_len + TQ - 1) / TQ;
    num_row_tiles = p.batch * tiles_per_batch;
  }
  if (num_row_tiles == 0) return hipSuccess;
  const dim3 grid(num_row_tiles * p.num_kv_heads * p.num_splits);
  if (same)
    flash_attn_kernel<DT, D, true><<<grid, 256, 0, stream>>>(p, tiles_per_batch, num_row_tiles);
  else
    flash_attn_kernel<DT, D, false><<<grid, 256, 0, stream>>>(p, tiles_per_batch, num_row_tiles);
  return hipGetLastError();
}

}  // namespace

bool flash_attn_supported(const AttnParams& p) {
  return p.q_dtype == p.kv_dtype && (p.q_dtype == BF16 || p.q_dtype == F16) && p.dqk == p.dvo &&
         (p.dqk == 64 || p.dqk == 128) && p.group <= kRows;
}

hipError_t launch_flash_attn(const AttnParams& p, bool same_strides, hipStream_t stream) {
  if (p.q_dtype == BF16)
    return p.dqk == 128 ? launch_fd<BF16, 128>(p, same_strides, stream)
                        : launch_fd<BF16, 64>(p, same_strides, stream);
  return p.dqk == 128 ? launch_fd<F16, 128>(p, same_strides, stream)
                      : launch_fd<F16, 64>(p, same_strides, stream);
}

}  // namespace pa
