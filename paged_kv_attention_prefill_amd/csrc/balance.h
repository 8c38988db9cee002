// Work-balanced split of a decode launch (library-internal load balancing; the
// pages only fix that split partial states merge through their LSE, which is how
// the pieces below are recombined).
//
// The work is the sequence of items (query batch b, KV head g), b-major; item
// (b, g) has nu(b) = max(1, ceil(L_b / unit)) units of `unit` KV tokens (an
// empty KV batch still has one unit, so that some workgroup writes its empty
// result).  With T units in total and NB shares (as many as there are
// co-resident workgroups, or that many over the row tiles below), share i takes
// units [i Qc, min(T, (i+1) Qc)), Qc = ceil(T / NB): every share streams the
// same number of KV tokens (up to one unit), so all of them finish together
// instead of in rounds of fixed-size chunks.
//
// When the rows of an item span several row tiles (MLA with more than 128 rows
// per request), a share is taken by one workgroup per row tile, placed on one
// XCD and dispatched together: they walk the same KV tokens in the same order,
// so the share's KV is read from HBM once into that XCD's L2.
//
// A share's range crosses items; each crossing closes a segment.  A segment
// that covers a whole item writes the final O / LSE; otherwise it writes a
// partial state (O normalised by its own sum, LSE, max) to workspace slot
// item + i, which is unique because item and share indices both grow along
// the sequence (the row tiles of a share write disjoint rows of the slot).
// The share that takes an item's first unit records the
// first and last share of the item in ws_seg[item], for the merge launch.
#pragma once

#include "device_common.h"

namespace pa {

__device__ __forceinline__ int kv_len_of(const AttnParams& p, int b) {
  const int kb = p.broadcast ? 0 : b;
  const int n = p.kv_indptr[kb + 1] - p.kv_indptr[kb];
  return n ? (n - 1) * p.page_size + p.kv_last[kb] : 0;
}

__device__ __forceinline__ int units_of(int L, int unit) { return L > 0 ? (L + unit - 1) / unit : 1; }

// inclusive prefix sum over the wave's 64 lanes
__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uni64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// A workgroup's walk over its share; every value here is wave-uniform (scalar
// registers).  Usage: if (cur.start(p, i)) do { ... cur.seg ... } while (cur.next(p));
struct BalCursor {
  int b, g;      // current item
  int L, nu;     // KV length and units of batch b
  int u;         // unit offset within the item
  int take;      // units of the current segment
  int64_t pos;   // global unit index of the segment's start
  int64_t left;  // units left for this workgroup, current segment included
  int64_t Qc;    // units per share
  int i;         // this workgroup's share
  int rt;        // and row tile

  __device__ __forceinline__ int j0(const AttnParams& p) const { return min(L, u * p.bal_unit); }
  __device__ __forceinline__ int j1(const AttnParams& p) const { return min(L, (u + take) * p.bal_unit); }
  __device__ __forceinline__ bool whole() const { return u == 0 && take == nu; }
  __device__ __forceinline__ int64_t slot(const AttnParams& p) const {
    return (int64_t)(b * p.num_kv_heads + g) + i;
  }

  // the item's first share (its first row tile) records the item's span for the merge
  __device__ __forceinline__ void open(const AttnParams& p) {
    take = uni(left < nu - u ? (int)left : nu - u);
    if (u == 0 && rt == 0 && threadIdx.x == 0) {
      const int item = b * p.num_kv_heads + g;
      p.ws_seg[2 * item] = i;
      p.ws_seg[2 * item + 1] = (int)((pos + nu - 1) / Qc);
    }
  }

  __device__ __forceinline__ bool start(const AttnParams& p, int wg) {
    const int lane = threadIdx.x & 63;
    const int B = p.batch, H = p.num_kv_heads, unit = p.bal_unit;
    // workgroups are dealt round-robin to the 8 XCDs: with bal_xcd, the virtual
    // workgroups of one XCD are consecutive, and so are the row tiles of a share
    const int nwg = p.bal_blocks * p.bal_co;
    const int v = p.bal_xcd ? (wg % 8) * (nwg / 8) + wg / 8 : wg;
    i = v / p.bal_co;
    rt = v - i * p.bal_co;
    int64_t tot = 0;
    for (int base = 0; base < B; base += 64) {
      const int bb = base + lane;
      const int n = bb < B ? units_of(kv_len_of(p, bb), unit) : 0;
      tot += uni(__shfl(wave_incl_scan(n, lane), 63, 64));
    }
    const int64_t T = tot * H;
    Qc = (T + p.bal_blocks - 1) / p.bal_blocks;
    pos = (int64_t)i * Qc;
    if (pos >= T) return false;
    left = (pos + Qc < T ? pos + Qc : T) - pos;
    // the batch b with H S_b <= pos < H S_{b+1}
    int64_t Sb = 0;  // units before batch b, per KV head
    b = 0;
    for (int base = 0; base < B; base += 64) {
      const int bb = base + lane;
      const int n = bb < B ? units_of(kv_len_of(p, bb), unit) : 0;
      const int incl = wave_incl_scan(n, lane);
      const uint64_t m = __ballot(bb < B && (Sb + incl) * H > pos);
      if (m) {
        const int l = __builtin_ctzll(m);
        b = uni(base + l);
        Sb += uni(__shfl(incl - n, l, 64));
        break;
      }
      Sb += uni(__shfl(incl, 63, 64));
    }
    L = uni(kv_len_of(p, b));
    nu = units_of(L, unit);
    const int64_t in_b = pos - Sb * H;  // units into batch b's items
    g = (int)(in_b / nu);
    u = (int)(in_b - (int64_t)g * nu);
    open(p);
    return true;
  }

  __device__ __forceinline__ bool next(const AttnParams& p) {
    left -= take;
    if (left <= 0) return false;
    pos += take;
    u += take;
    if (u == nu) {
      u = 0;
      if (++g == p.num_kv_heads) {
        g = 0;
        ++b;
        L = uni(kv_len_of(p, b));
        nu = units_of(L, p.bal_unit);
      }
    }
    open(p);
    return true;
  }
};

}  // namespace pa
