// Paged flash attention on MFMA for many query rows per KV head: ragged causal
// prefill (the batched paged prefill of the FlashInfer PR #4736 analysis, code
// section 2) and broadcast decode/prefill where every query batch reads one KV
// batch (PyTorch 2.14 MPS FlexAttention post, introduction) — the query rows of
// all batches are folded into the same row tiles so the shared KV is read once
// per tile instead of once per query batch.
//
// Rows: a row is (query token t, query head h) with h in KV group g; a row tile
// holds TQ = 256/G tokens x G heads (r = token_offset*G + head_in_group).
// Without broadcast a tile's tokens come from one query batch; with broadcast
// they run over all query tokens of all batches.
//
// A workgroup = (row tile, KV head g, explicit KV split) with 8 waves of 32
// rows (256 rows share each KV tile).  Per 64-token KV tile (double-buffered in
// LDS and fetched two tiles ahead into registers, cooperatively, with the page
// ids of the range staged in LDS):
//   S^T = K Q^T on v_mfma_f32_32x32x16 (K from LDS as the A operand, Q^T from
//   registers as the B operand); causal/length mask on boundary tiles only;
//   online softmax (running max and sum per row, one lane-pair shuffle per
//   reduction; the reference max is re-based lazily);
//   O^T += V^T P^T with V^T read from LDS by ds_read_b64_tr_b16 and P^T taken
//   straight from the score registers.
// Tiles past a tile's last visible position (causal) are skipped; workgroups
// are ordered so that every (KV head, split) group lives on one XCD (its KV
// stays in that XCD's L2) and each XCD starts with its heaviest row tiles.
#include "mfma_common.h"

namespace pa {
namespace {

constexpr int kNW = 8;           // waves per workgroup
constexpr int kRows = 32 * kNW;  // rows per workgroup (32 per wave)
constexpr int kThreads = 64 * kNW;
constexpr int kKT = 64;          // KV tokens per tile
constexpr int kPageWin = 1024;   // page ids staged in LDS at a time

template <int D>
struct FGeo {
  static constexpr int KK = D / 16;            // 16-dim k-steps of Q.K
  static constexpr int NDT = D / 32;           // 32-dim tiles of O
  static constexpr int KP = D * 2 + 16;        // K row pitch (bytes): conflict-free b128 reads
  static constexpr int VP = D * 2 + 64;        // V row pitch (bytes): a 32-lane transposed read
                                               // pass (4 rows x 64 B) covers 64 distinct banks
  static constexpr int KBYTES = kKT * KP;
  static constexpr int VBYTES = kKT * VP;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static constexpr int LPT = kKT * CPR / kThreads;  // chunks per thread per tile (each of K, V)
  static constexpr int TSTEP = kThreads / CPR;      // token stride between a thread's chunks
};

// Per-thread view of the cooperative tile fetch over one page-id window.
struct Fetch {
  const uint16_t* kbase;
  const uint16_t* vbase;
  const int* s_pages;
  const uint64_t* s_poff;  // PO2: element offset of each window page (page id x page stride)
  uint32_t pshift, pmask;  // PO2: log2(P), P - 1
  uint32_t ks0, ks1, kc, vs0, vs1, vc;  // kc / vc: KV-head plus 16-byte-chunk offsets
  int tk0, P;
  uint32_t pmagic;         // ceil(2^32 / P), or 0 for P == 1
  int wbP, ws, we, nk;  // window's first token (page-aligned); its range [ws, we); tiles in it
};

// One tile's worth of this thread's K and V chunks (at most two of each: a
// tile is 64 rows x D/8 chunks over 512 threads, D <= 128).  Named members, not
// arrays, so the sets stay in VGPRs across the pipelined loop.
struct TileRegs {
  i16x8_t k0, k1, v0, v1;
};

template <int D, bool SAME, bool PO2>
__device__ __forceinline__ void fetch_chunk(const Fetch& f, int jb, int u, i16x8_t& kr,
                                            i16x8_t& vr) {
  using Gm = FGeo<D>;
  if constexpr (PO2) {
    // power-of-two page size, equal K/V strides: the page's offset comes from the
    // window table (its 64-bit multiply done once per page when staged), the page
    // and slot by shift and mask, the in-page offset by a 24-bit multiply
    const int rel = min(jb - f.wbP + f.tk0 + Gm::TSTEP * u, f.we - 1 - f.wbP);
    const uint32_t pw = (uint32_t)rel >> f.pshift;
    const uint32_t slot = (uint32_t)rel & f.pmask;
    const uint64_t e = f.s_poff[pw] + (__umul24(slot, f.ks1) + f.kc);  // in-page part < 2^31
    kr = *reinterpret_cast<const i16x8_t*>(f.kbase + e);
    vr = *reinterpret_cast<const i16x8_t*>(f.vbase + e);
  } else {
    const int j = jb + f.tk0 + Gm::TSTEP * u;
    const int jj = j < f.we ? j : f.we - 1;  // a valid token, never a poisoned slot
    // page within the window and slot within the page, division-free: rel < 1024 P
    // and P <= 2048 keep rel * P < 2^32, where the rounded-up reciprocal is exact
    const uint32_t rel = jj - f.wbP;
    const uint32_t pw = div_by_magic(rel, f.pmagic);
    const int slot = rel - pw * f.P;
    const uint32_t page = f.s_pages[pw];
    // 32x32->64-bit page offset plus a 32-bit offset within the page
    const uint64_t koff = (uint64_t)page * f.ks0 + (slot * f.ks1 + f.kc);
    const uint64_t voff = SAME ? koff : (uint64_t)page * f.vs0 + (slot * f.vs1 + f.vc);
    kr = *reinterpret_cast<const i16x8_t*>(f.kbase + koff);
    vr = *reinterpret_cast<const i16x8_t*>(f.vbase + voff);
  }
}

template <int D, bool SAME, bool PO2>
__device__ __forceinline__ void fetch_tile(const Fetch& f, int t, TileRegs& r) {
  static_assert(FGeo<D>::LPT == 1 || FGeo<D>::LPT == 2, "tile fetch covers one or two chunks");
  const int jb = f.ws + min(t, f.nk - 1) * kKT;  // clamped: fetches are unconditional
  fetch_chunk<D, SAME, PO2>(f, jb, 0, r.k0, r.v0);
  if constexpr (FGeo<D>::LPT == 2) fetch_chunk<D, SAME, PO2>(f, jb, 1, r.k1, r.v1);
}

// Rows past the range end hold a clamped valid token: finite, and their P is 0.
template <int D>
__device__ __forceinline__ void store_tile(uint8_t* stage, int tk0, int cc, const TileRegs& r) {
  using Gm = FGeo<D>;
  uint8_t* kl = stage + tk0 * Gm::KP + cc * 16;
  uint8_t* vl = stage + Gm::KBYTES + tk0 * Gm::VP + cc * 16;
  *reinterpret_cast<i16x8_t*>(kl) = r.k0;
  *reinterpret_cast<i16x8_t*>(vl) = r.v0;
  if constexpr (Gm::LPT == 2) {
    *reinterpret_cast<i16x8_t*>(kl + Gm::TSTEP * Gm::KP) = r.k1;
    *reinterpret_cast<i16x8_t*>(vl + Gm::TSTEP * Gm::VP) = r.v1;
  }
}

struct RowState {
  float m;         // reference max (log2 units, scaled); re-based lazily
  float lsum;      // this lane's partial sum of exp2(s - m)
  float true_max;  // running row max (m may lag it)
};

// S^T[token][row] = K Q^T for one 64-token tile, as two 32-token blocks.  Lane
// (row l32, half h2) holds tokens 32mb + 8(i/4) + 4h2 + i%4 of its row.
template <int DT, int D>
__device__ __forceinline__ void tile_qk(const uint8_t* stage, const i16x8_t (&qreg)[FGeo<D>::KK],
                                        f32x16_t (&s)[2], int lane) {
  using Gm = FGeo<D>;
  const int l32 = lane & 31, h2 = lane >> 5;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) s[mb][i] = 0.f;
#pragma unroll
  for (int kk = 0; kk < Gm::KK; ++kk)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const i16x8_t a = *reinterpret_cast<const i16x8_t*>(stage + (32 * mb + l32) * Gm::KP +
                                                          (16 * kk + 8 * h2) * 2);
      s[mb] = mfma32<DT>(a, qreg[kk], s[mb]);
    }
}

// Tokens j >= lim of this lane's row get -inf (boundary tiles only).
__device__ __forceinline__ void tile_mask(f32x16_t (&s)[2], int jb, int lim, int lane) {
  const int h2 = lane >> 5;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = jb + 32 * mb + 8 * (i >> 2) + 4 * h2 + (i & 3);
      s[mb][i] = j < lim ? s[mb][i] : -INFINITY;
    }
}

// Running max over the tile.  Scores stay unscaled; the scale is fused into the
// exponent's FMA.  The reference max is re-based only when the tile max exceeds
// it by more than 8 (log2 units): most tiles skip the O rescale, P <= 2^8 keeps
// 16-bit P and fp32 sums well in range, and LSE = m + log2(l) holds for any
// reference m.
// A tile that is not `valid` (past the range) leaves the state as it is.
template <int NDT>
__device__ __forceinline__ void tile_max(const f32x16_t (&s)[2], float qk_scale, RowState& st,
                                         f32x16_t (&oacc)[NDT], bool valid) {
  float tmax = -INFINITY;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[mb][i]);
  tmax = valid ? xor32_max(tmax) * qk_scale : -INFINITY;
  st.true_max = fmaxf(st.true_max, tmax);
  const bool grow = tmax > st.m + 8.f;
  if (__ballot(grow)) {
    const float mnew = grow ? tmax : st.m;
    const float alpha =
        fast_exp2((st.m == -INFINITY ? -INFINITY : st.m) - (mnew == -INFINITY ? 0.f : mnew));
    const float a = grow ? alpha : 1.f;
    st.lsum *= a;
#pragma unroll
    for (int t = 0; t < NDT; ++t) oacc[t] *= a;
    st.m = mnew;
  }
}

// S^T of the next tile (sn = K Q^T, as tile_qk) and, interleaved with its MFMAs,
// P of the current tile: exp2(sc * scale - m) packed to 16-bit as the B operands
// of the four 16-token PV steps (pb), the row sum accumulating in fp32.  Each
// k-step issues the K reads of the next k-step, its two MFMAs and a share of the
// exponentials, so the VALU work runs while the MFMAs execute.
template <int DT, int D>
__device__ __forceinline__ void tile_qk_exp(const uint8_t* stage,
                                            const i16x8_t (&qreg)[FGeo<D>::KK],
                                            f32x16_t (&sn)[2], const f32x16_t (&sc)[2],
                                            float qk_scale, RowState& st, i16x8_t (&pb)[4],
                                            int lane) {
  using Gm = FGeo<D>;
  constexpr int KK = Gm::KK;
  constexpr int EPK = 32 / KK;  // exponentials per k-step
  static_assert(EPK * KK == 32 && (EPK % 4) == 0, "k-steps split the 32 scores evenly");
  const int l32 = lane & 31, h2 = lane >> 5;
  const uint8_t* krow = stage + l32 * Gm::KP + 16 * h2;
  const float nmref = -(st.m == -INFINITY ? 0.f : st.m);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) sn[mb][i] = 0.f;
  float e[32];
  float psum = 0.f;
  i16x8_t a0 = *reinterpret_cast<const i16x8_t*>(krow);
  i16x8_t a1 = *reinterpret_cast<const i16x8_t*>(krow + 32 * Gm::KP);
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    i16x8_t n0 = a0, n1 = a1;
    if (kk + 1 < KK) {
      n0 = *reinterpret_cast<const i16x8_t*>(krow + 32 * (kk + 1));
      n1 = *reinterpret_cast<const i16x8_t*>(krow + 32 * Gm::KP + 32 * (kk + 1));
    }
    sn[0] = mfma32<DT>(a0, qreg[kk], sn[0]);
    sn[1] = mfma32<DT>(a1, qreg[kk], sn[1]);
#pragma unroll
    for (int i = 0; i < EPK; ++i) {
      const int idx = kk * EPK + i;
      e[idx] = fast_exp2(fmaf(sc[idx >> 4][idx & 15], qk_scale, nmref));
    }
    if (((kk + 1) * EPK) % 8 == 0) {
      const int t = (kk + 1) * EPK / 8 - 1;
      const uint4 bits = make_uint4(pack2<DT>(e[8 * t + 0], e[8 * t + 1]),
                                    pack2<DT>(e[8 * t + 2], e[8 * t + 3]),
                                    pack2<DT>(e[8 * t + 4], e[8 * t + 5]),
                                    pack2<DT>(e[8 * t + 6], e[8 * t + 7]));
      pb[t] = as_i16x8(bits);
      // the row sum is taken over the rounded P that the PV step multiplies
      psum = sum2<DT>(bits.x, sum2<DT>(bits.y, sum2<DT>(bits.z, sum2<DT>(bits.w, psum))));
    }
    __builtin_amdgcn_sched_barrier(0);
    a0 = n0;
    a1 = n1;
  }
  asm volatile("" : "+v"(psum));
  st.lsum += psum;
}

// O^T += V^T P^T, V^T by transposed LDS reads.
template <int DT, int D>
__device__ __forceinline__ void tile_pv(const uint8_t* stage, const i16x8_t (&pb)[4],
                                        f32x16_t (&oacc)[FGeo<D>::NDT], int lane) {
  using Gm = FGeo<D>;
  const int l16 = lane & 15, h2 = lane >> 5;
  const uint16_t* vrow =
      reinterpret_cast<const uint16_t*>(stage + Gm::KBYTES + (4 * h2 + (l16 >> 2)) * Gm::VP) +
      16 * ((lane >> 4) & 1) + 4 * (l16 & 3);
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int dt = 0; dt < Gm::NDT; ++dt) {
      const uint16_t* ra = vrow + (16 * t) * (Gm::VP / 2) + 32 * dt;
      const i16x4_t lo = lds_read_tr(ra);
      const i16x4_t hi4 = lds_read_tr(ra + 8 * (Gm::VP / 2));
      const i16x8_t va = {lo[0], lo[1], lo[2], lo[3], hi4[0], hi4[1], hi4[2], hi4[3]};
      oacc[dt] = mfma32<DT>(va, pb[t], oacc[dt]);
    }
}

template <int DT, int D, bool SAME, bool PO2>
__global__ __launch_bounds__(kThreads, 1) void flash_attn_kernel(AttnParams p, int tiles_per_batch,
                                                                int num_row_tiles) {
  using Gm = FGeo<D>;
  constexpr int KK = Gm::KK, NDT = Gm::NDT;
  __shared__ __align__(16) uint8_t smem[3 * Gm::STAGE];
  // page-id window: int ids, or (PO2) the 64-bit element offset of each page
  __shared__ uint64_t s_pagebuf[kPageWin];
  __shared__ int s_red[kNW];
  int* const s_pages = reinterpret_cast<int*>(s_pagebuf);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31, h2 = lane >> 5;
  const int G = p.group;
  const int TQ = kRows / G;

  // ---- which (row tile, KV head, split).  Workgroups are dealt round-robin to
  // the 8 XCDs; when the (head, split) groups divide evenly, every group lives on
  // one XCD and each XCD walks its row tiles from the latest (heaviest under a
  // causal mask) to the earliest.
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
  int64_t row_t;  // query token (global), -1 for a padding row
  int row_h;      // query head
  int lim;        // visible KV tokens are j < lim
  {
    const int r = 32 * w + l32;
    const int64_t t = t_begin + r / G;
    const bool ok = (r / G) < TQ && t < t_end;
    row_t = ok ? t : -1;
    row_h = g * G + r % G;
    int l = j1;
    if (ok && p.causal) {
      const int bb = p.broadcast ? batch_of_token(p, (int)t) : b;
      const int q0 = p.qo_indptr ? p.qo_indptr[bb] : bb * p.q_len;
      const int qb = p.qo_indptr ? p.qo_indptr[bb + 1] - q0 : p.q_len;
      l = min(l, L - qb + ((int)t - q0) + 1);
    }
    lim = ok ? l : INT_MIN;
  }
  // workgroup-wide last visible token (tiles past it are skipped)
  int hi = lim;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) hi = max(hi, __shfl_xor(hi, off, 64));
  if (lane == 0) s_red[w] = hi;
  __syncthreads();
  int jmax = s_red[0];
#pragma unroll
  for (int i = 1; i < kNW; ++i) jmax = max(jmax, s_red[i]);
  const int jhi = min(j1, jmax);
  // tiles ending at or before this wave's smallest row limit need no mask
  int lo = row_t >= 0 ? lim : INT_MAX;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) lo = min(lo, __shfl_xor(lo, off, 64));
  const int wave_lim_min = __builtin_amdgcn_readfirstlane(lo);

  // ---- Q^T B operand: KK x 16 B per lane, kept in registers
  i16x8_t qreg[KK];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(p.q) +
                         ((row_t < 0 ? 0 : row_t) * p.num_qo_heads + row_h) * (int64_t)D + 8 * h2;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const uint4 v =
          row_t >= 0 ? *reinterpret_cast<const uint4*>(qp + 16 * kk) : make_uint4(0, 0, 0, 0);
      qreg[kk] = as_i16x8(v);
    }
  }

  RowState st{-INFINITY, 0.f, -INFINITY};
  f32x16_t oacc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[t][i] = 0.f;
  const float qk_scale = p.sm_scale * p.k_scale * kLog2e;

  // cooperative fetch: thread -> (16-byte chunk cc, tokens tk0 + TSTEP*u)
  const int cc = tid % Gm::CPR;
  Fetch f;
  f.kbase = static_cast<const uint16_t*>(p.k);
  f.vbase = static_cast<const uint16_t*>(p.v);
  f.s_pages = s_pages;
  f.s_poff = s_pagebuf;
  f.pshift = __builtin_ctz((unsigned)p.page_size);
  f.pmask = (uint32_t)p.page_size - 1;
  f.ks0 = (uint32_t)p.ks0;
  f.ks1 = (uint32_t)p.ks1;
  f.kc = (uint32_t)(g * p.ks2 + 8 * cc);
  f.vs0 = (uint32_t)p.vs0;
  f.vs1 = (uint32_t)p.vs1;
  f.vc = (uint32_t)(g * p.vs2 + 8 * cc);
  f.tk0 = tid / Gm::CPR;
  f.P = p.page_size;
  f.pmagic = p.page_magic;

  TileRegs rg;  // the tile in flight from HBM to LDS
  if (jhi > j0) {
    const int P = p.page_size;
    const int pfirst = j0 / P, plast = (jhi - 1) / P;
    for (int wb = pfirst; wb <= plast; wb += kPageWin) {
      const int npw = min(kPageWin, plast - wb + 1);
      __syncthreads();  // previous window's readers are done
      if constexpr (PO2) {
        for (int i = tid; i < npw; i += kThreads)
          s_pagebuf[i] = (uint64_t)(uint32_t)p.kv_indices[pbeg + wb + i] * (uint32_t)p.ks0;
      } else {
        for (int i = tid; i < npw; i += kThreads) s_pages[i] = p.kv_indices[pbeg + wb + i];
      }
      __syncthreads();
      f.wbP = wb * P;
      f.ws = max(j0, wb * P);
      f.we = min(jhi, (wb + npw) * P);
      f.nk = (f.we - f.ws + kKT - 1) / kKT;
      const int nk = f.nk;

      // Software pipeline over three LDS stages (tile t in stage t % 3), one
      // barrier per tile.  Iteration k issues the QK MFMAs of tile k+1 next to the
      // exponentials of tile k, then the PV MFMAs of tile k next to the store of
      // tile k+2 (fetched into registers one iteration earlier), the fetch of tile
      // k+3 and the mask/max of tile k+1.  Fetches are unconditional (tile index
      // clamped) so every path has the same loads in flight.
      {
        TileRegs r1;
        fetch_tile<D, SAME, PO2>(f, 0, rg);
        fetch_tile<D, SAME, PO2>(f, 1, r1);
        store_tile<D>(smem, f.tk0, cc, rg);
        store_tile<D>(smem + Gm::STAGE, f.tk0, cc, r1);
      }
      fetch_tile<D, SAME, PO2>(f, 2, rg);
      __syncthreads();
      f32x16_t sa[2], sb[2];
      tile_qk<DT, D>(smem, qreg, sa, lane);
      if (f.ws + kKT > wave_lim_min) tile_mask(sa, f.ws, lim, lane);
      tile_max(sa, qk_scale, st, oacc, true);
      int cur = 0, nxt = Gm::STAGE, nn = 2 * Gm::STAGE;  // stage offsets of tiles k, k+1, k+2
      auto step = [&](int k, f32x16_t (&sc)[2], f32x16_t (&sn)[2]) __attribute__((always_inline)) {
        const bool more = k + 1 < nk;  // sn past the last tile is computed but unused
        i16x8_t pb[4];
        tile_qk_exp<DT, D>(smem + nxt, qreg, sn, sc, qk_scale, st, pb, lane);
        const int jn = f.ws + (k + 1) * kKT;
        if (more && jn + kKT > wave_lim_min) tile_mask(sn, jn, lim, lane);
        tile_pv<DT, D>(smem + cur, pb, oacc, lane);
        store_tile<D>(smem + nn, f.tk0, cc, rg);  // past the last tile: a stage nobody reads
        fetch_tile<D, SAME, PO2>(f, k + 3, rg);
        tile_max(sn, qk_scale, st, oacc, more);
        __syncthreads();
        const int t = cur;
        cur = nxt;
        nxt = nn;
        nn = t;
      };
      for (int k = 0; k < nk; k += 2) {
        step(k, sa, sb);
        if (k + 1 >= nk) break;
        step(k + 1, sb, sa);
      }
    }
  }

  // ---- epilogue: lane (row l32, half h2) holds dims 32dt + 8q + 4h2 + (0..3)
  const float ltot = xor32_sum(st.lsum);
  if (row_t < 0) return;
  const bool empty = !(ltot > 0.f);
  const float scale = empty ? 0.f : p.v_scale / ltot;
  const int64_t rid = row_t * p.num_qo_heads + row_h;
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
    if (p.lse) p.lse[sidx] = empty ? -INFINITY : (st.m + fast_log2(ltot)) * kLn2;
    if (p.mx) p.mx[sidx] = empty ? -INFINITY : st.true_max * kLn2;
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
  // power-of-two pages with equal K/V strides take the table-of-page-addresses fetch
  const bool po2 = same && (p.page_size & (p.page_size - 1)) == 0 && p.ks1 < (int64_t(1) << 24);
  if (po2)
    flash_attn_kernel<DT, D, true, true><<<grid, kThreads, 0, stream>>>(p, tiles_per_batch, num_row_tiles);
  else if (same)
    flash_attn_kernel<DT, D, true, false><<<grid, kThreads, 0, stream>>>(p, tiles_per_batch, num_row_tiles);
  else
    flash_attn_kernel<DT, D, false, false><<<grid, kThreads, 0, stream>>>(p, tiles_per_batch, num_row_tiles);
  return hipGetLastError();
}

}  // namespace

bool flash_attn_supported(const AttnParams& p) {
  // element offsets: page strides fit 32 bits and so does every offset within a page
  const int64_t lim = int64_t(1) << 31;
  const bool offsets32 =
      p.ks0 < lim && p.vs0 < lim &&
      (p.page_size - 1) * p.ks1 + (p.num_kv_heads - 1) * p.ks2 + p.dqk < lim &&
      (p.page_size - 1) * p.vs1 + (p.num_kv_heads - 1) * p.vs2 + p.dvo < lim;
  return p.q_dtype == p.kv_dtype && (p.q_dtype == BF16 || p.q_dtype == F16) && p.dqk == p.dvo &&
         (p.dqk == 64 || p.dqk == 128) && p.group <= kRows && p.page_size <= 2048 && offsets32;
}

hipError_t launch_flash_attn(const AttnParams& p, bool same_strides, hipStream_t stream) {
  if (p.q_dtype == BF16)
    return p.dqk == 128 ? launch_fd<BF16, 128>(p, same_strides, stream)
                        : launch_fd<BF16, 64>(p, same_strides, stream);
  return p.dqk == 128 ? launch_fd<F16, 128>(p, same_strides, stream)
                      : launch_fd<F16, 64>(p, same_strides, stream);
}

}  // namespace pa
