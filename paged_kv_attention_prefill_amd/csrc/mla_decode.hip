// MLA paged decode: every query head and every query token of a request reads
// one shared latent KV row per token (576 dims: K is the whole row, V its first
// 512 dims) — the shared latent KV of the FlashInfer PR #3309 analysis (code
// section 1), where q_len is folded into the head dimension because the KV is
// shared by all heads and queries.  Here all q_len x H rows of a request form
// row blocks (r = token*H + head), so one KV tile in LDS feeds every row.
//
// Four kernels by rows per request and query type, all streaming tiles of whole
// latent rows HBM -> LDS with direct-to-LDS loads (bf16 rows, or fp8 e4m3 codes
// with a per-tensor scale):
//   mla_narrow_kernel (<= 16 rows): the 576-dim contraction is split over the
//     waves and the partial scores are summed in LDS; 32-token tiles;
//   mla_mid_kernel (17..64 rows, bf16 queries): the same scheme for two or four
//     16-row blocks;
//   mla_rows_kernel (> 64 rows, bf16 queries): the flash-attention shape, 16
//     rows per wave, 32-token tiles;
//   mla_rows8_kernel (> 16 rows, fp8 queries over an fp8 cache): the same shape
//     with both products on the fp8 matrix cores, 128-token tiles.
// Balanced shares of long KV batches leave partial states (O normalised by the
// piece's own sum, LSE, max) in the workspace for the merge launch.
#include "balance.h"
#include "mfma_common.h"

namespace pa {
namespace {

constexpr int kDqk = 576, kDvo = 512;
constexpr int kPageWinM = 256;               // page ids staged in LDS at a time
// Cache policy of the KV tile loads: non-temporal (the nt bit).  Every latent
// row is read once per launch (the row tiles of a share read it together), and
// streaming it past the caches measured 9% faster on a bf16 cache of 16-row
// requests (H16 q1: 139 -> 126 us by events), within 1-2% on the other shapes,
// and 3% slower only on the fp8 page-size-1 row gather (576-byte rows that
// share 128-byte lines).
constexpr int kKvCpol = 2;

// ---------------------------------------------------------------------------
// Many rows per request (q_len x H > 64, bf16 KV): the flash-attention shape.
// A workgroup = (request, 128-row tile, KV range) with 8 waves of 16 rows each;
// every wave keeps its rows' Q^T (16 x 576) in registers and its rows' whole
// O^T (512 x 16, fp32) in accumulation registers, so a KV tile in LDS feeds all
// 128 rows with no exchange between waves.  Per 32-token tile:
//   the tile's rows go HBM -> LDS by direct-to-LDS loads (global_load_lds, 16
//   bytes per lane, a wave instruction filling 1 KB of LDS), double-buffered so
//   the next tile streams in during this tile's math;
//   S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (K from LDS as the A operand);
//   online softmax with a lazily re-based running max (as in the prefill kernel);
//   O^T += V^T P^T with V^T read transposed (ds_read_b64_tr_b16) from the same
//   LDS rows (V is the first 512 dims of a row) and P^T straight from the
//   score registers.
constexpr int kNW2 = 8;                  // waves per workgroup
constexpr int kRW = 16;                  // rows per wave
constexpr int kRT2 = kNW2 * kRW;         // rows per workgroup
constexpr int kTK2 = 32;                 // KV tokens per tile
constexpr int kPieces = kDqk / 8;       // 16-byte pieces per latent row (72)
constexpr int kKP2 = kPieces * 16;       // LDS row pitch (bytes), unpadded
static_assert(16 * kKP2 == 18432, "the asm LDS reads address row r + 16 with offset:18432");
constexpr int kDma = kTK2 * kPieces / 64;  // 1-KB direct-load instructions per tile (36)
constexpr int kStage2 = kDma * 1024;     // one tile in LDS
static_assert(kTK2 * kPieces % 64 == 0, "a tile is a whole number of 1-KB wave loads");

// Workgroup barrier for the LDS hand-offs of the narrow kernel's streaming loop.
// The fence of __syncthreads makes every wave wait for all of its outstanding
// vector-memory operations, which includes the direct-to-LDS loads of the tiles
// still in flight (their LDS writes fall under the fence), so the pipeline
// would drain at every barrier.  Here the LDS operations are completed
// explicitly (lgkmcnt(0): writes visible to the other waves after the barrier),
// the loads of the tile being handed over are waited for by the caller (vmcnt),
// and the memory clobbers keep the compiler from moving LDS accesses across the
// barrier.  (The many-rows kernel measured faster with __syncthreads.)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt: no wait
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t lds_off(const void* p) {
  return (uint32_t)(uintptr_t)(const PA_LDS void*)p;
}

// Reads of a stage that direct loads filled.  The caller has waited for the
// tile's loads (vmcnt, then a barrier); the compiler cannot see that and, where
// its tracking of direct-to-LDS loads loses the stages (at loop heads), waits
// for every load in flight before such a read.  These reads are written in
// inline asm, each block waiting for its own reads before it returns.
__device__ __forceinline__ void lds_read6_b128(uint32_t a0, uint32_t a1, uint32_t a2, i32x4_t (&r)[6]) {
  asm volatile(
      "ds_read_b128 %0, %6\n\t"
      "ds_read_b128 %1, %6 offset:18432\n\t"
      "ds_read_b128 %2, %7\n\t"
      "ds_read_b128 %3, %7 offset:18432\n\t"
      "ds_read_b128 %4, %8\n\t"
      "ds_read_b128 %5, %8 offset:18432\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5])
      : "v"(a0), "v"(a1), "v"(a2)
      : "memory");
}
// Eight transposed 4x16 reads (ds_read_b64_tr_b16) at b_d and b_d + 18432.
__device__ __forceinline__ void lds_read8_tr(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3,
                                             i32x2_t (&r)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:18432\n\t"
      "ds_read_b64_tr_b16 %2, %9\n\t"
      "ds_read_b64_tr_b16 %3, %9 offset:18432\n\t"
      "ds_read_b64_tr_b16 %4, %10\n\t"
      "ds_read_b64_tr_b16 %5, %10 offset:18432\n\t"
      "ds_read_b64_tr_b16 %6, %11\n\t"
      "ds_read_b64_tr_b16 %7, %11 offset:18432\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
        "=&v"(r[7])
      : "v"(b0), "v"(b1), "v"(b2), "v"(b3)
      : "memory");
}
// Writes of 16-byte pieces into the widened tile (not a direct-load target, but
// the compiler's tracking would order them after every load in flight),
// completed before returning.
__device__ __forceinline__ void lds_write4_b128(uint32_t a0, i32x4_t v0, uint32_t a1, i32x4_t v1,
                                                uint32_t a2, i32x4_t v2, uint32_t a3, i32x4_t v3) {
  asm volatile(
      "ds_write_b128 %0, %1\n\t"
      "ds_write_b128 %2, %3\n\t"
      "ds_write_b128 %4, %5\n\t"
      "ds_write_b128 %6, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      :
      : "v"(a0), "v"(v0), "v"(a1), "v"(v1), "v"(a2), "v"(v2), "v"(a3), "v"(v3)
      : "memory");
}
__device__ __forceinline__ void lds_write2_b128(uint32_t a0, i32x4_t v0, uint32_t a1, i32x4_t v1) {
  asm volatile(
      "ds_write_b128 %0, %1\n\t"
      "ds_write_b128 %2, %3\n\t"
      "s_waitcnt lgkmcnt(0)"
      :
      : "v"(a0), "v"(v0), "v"(a1), "v"(v1)
      : "memory");
}
// Four 16-byte reads at a0, a0 + 18432, a1, a1 + 18432.
__device__ __forceinline__ void lds_read4_b128(uint32_t a0, uint32_t a1, i32x4_t (&r)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:18432\n\t"
      "ds_read_b128 %2, %5\n\t"
      "ds_read_b128 %3, %5 offset:18432\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(a0), "v"(a1)
      : "memory");
}
// Two 16-byte reads at a0, a0 + 18432.
__device__ __forceinline__ void lds_read2x_b128(uint32_t a0, i32x4_t (&r)[2]) {
  asm volatile(
      "ds_read_b128 %0, %2\n\t"
      "ds_read_b128 %1, %2 offset:18432\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1])
      : "v"(a0)
      : "memory");
}
// Partial-score reads of a row block: 2 KS 16-byte reads at base + S k + 1024 st
// (k < KS, st < 2), completed on return.
template <int KS, int S>
__device__ __forceinline__ void lds_read_parts(uint32_t base, f32x4_t (&r)[KS][2]) {
  if constexpr (KS == 2) {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %4 offset:1024\n\t"
        "ds_read_b128 %2, %4 offset:%5\n\t"
        "ds_read_b128 %3, %4 offset:%6\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0][0]), "=&v"(r[0][1]), "=&v"(r[1][0]), "=&v"(r[1][1])
        : "v"(base), "i"(S), "i"(S + 1024)
        : "memory");
  } else {
    static_assert(KS == 4, "2 or 4 slices");
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %8 offset:1024\n\t"
        "ds_read_b128 %2, %8 offset:%9\n\t"
        "ds_read_b128 %3, %8 offset:%10\n\t"
        "ds_read_b128 %4, %8 offset:%11\n\t"
        "ds_read_b128 %5, %8 offset:%12\n\t"
        "ds_read_b128 %6, %8 offset:%13\n\t"
        "ds_read_b128 %7, %8 offset:%14\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0][0]), "=&v"(r[0][1]), "=&v"(r[1][0]), "=&v"(r[1][1]), "=&v"(r[2][0]), "=&v"(r[2][1]),
          "=&v"(r[3][0]), "=&v"(r[3][1])
        : "v"(base), "i"(S), "i"(S + 1024), "i"(2 * S), "i"(2 * S + 1024), "i"(3 * S), "i"(3 * S + 1024)
        : "memory");
  }
}

// A wave's partial scores: 16 bytes per lane at a and a + 1024, completed on return.
__device__ __forceinline__ void lds_write_part(uint32_t a, f32x4_t v0, f32x4_t v1) {
  asm volatile(
      "ds_write_b128 %0, %1\n\t"
      "ds_write_b128 %0, %2 offset:1024\n\t"
      "s_waitcnt lgkmcnt(0)"
      :
      : "v"(a), "v"(v0), "v"(v1)
      : "memory");
}

// One 4-byte write (an exchange word next to the stages), completed on return.
__device__ __forceinline__ void lds_write_b32(uint32_t a, int v) {
  asm volatile(
      "ds_write_b32 %0, %1\n\t"
      "s_waitcnt lgkmcnt(0)"
      :
      : "v"(a), "v"(v)
      : "memory");
}
// P^T block (16 bytes), one row's rescale factor and the flag word, in one round trip.
__device__ __forceinline__ void lds_read_pv(uint32_t apb, uint32_t aal, uint32_t afl, i32x4_t& pb, float& al,
                                            int& fl) {
  asm volatile(
      "ds_read_b128 %0, %3\n\t"
      "ds_read_b32 %1, %4\n\t"
      "ds_read_b32 %2, %5\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(pb), "=&v"(al), "=&v"(fl)
      : "v"(apb), "v"(aal), "v"(afl)
      : "memory");
}
// The PV inputs of NRB row blocks in one round trip: P^T blocks at apb + 1024 rb,
// rescale factors at aal + 64 rb, and the NRB flag words at afl.
template <int NRB>
__device__ __forceinline__ void lds_read_pv_blocks(uint32_t apb, uint32_t aal, uint32_t afl, i32x4_t (&pb)[NRB],
                                                   float (&al)[NRB], int (&fl)[NRB]) {
  static_assert(NRB == 2 || NRB == 4, "two or four row blocks");
  if constexpr (NRB == 4) {
    i32x4_t f;
    asm volatile(
        "ds_read_b128 %0, %9\n\t"
        "ds_read_b128 %1, %9 offset:1024\n\t"
        "ds_read_b128 %2, %9 offset:2048\n\t"
        "ds_read_b128 %3, %9 offset:3072\n\t"
        "ds_read_b32 %4, %10\n\t"
        "ds_read_b32 %5, %10 offset:64\n\t"
        "ds_read_b32 %6, %10 offset:128\n\t"
        "ds_read_b32 %7, %10 offset:192\n\t"
        "ds_read_b128 %8, %11\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(pb[0]), "=&v"(pb[1]), "=&v"(pb[2]), "=&v"(pb[3]), "=&v"(al[0]), "=&v"(al[1]),
          "=&v"(al[2]), "=&v"(al[3]), "=&v"(f)
        : "v"(apb), "v"(aal), "v"(afl)
        : "memory");
    fl[0] = f.x;
    fl[1] = f.y;
    fl[2] = f.z;
    fl[3] = f.w;
  } else {
    i32x2_t f;
    asm volatile(
        "ds_read_b128 %0, %5\n\t"
        "ds_read_b128 %1, %5 offset:1024\n\t"
        "ds_read_b32 %2, %6\n\t"
        "ds_read_b32 %3, %6 offset:64\n\t"
        "ds_read_b64 %4, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(pb[0]), "=&v"(pb[1]), "=&v"(al[0]), "=&v"(al[1]), "=&v"(f)
        : "v"(apb), "v"(aal), "v"(afl)
        : "memory");
    fl[0] = f.x;
    fl[1] = f.y;
  }
}
// Twelve 16-byte reads at a + 1024 k, k = 0..11 (the partial-score blocks).
__device__ __forceinline__ void lds_read12_b128(uint32_t a, i32x4_t (&r)[12]) {
  asm volatile(
      "ds_read_b128 %0, %12\n\t"
      "ds_read_b128 %1, %12 offset:1024\n\t"
      "ds_read_b128 %2, %12 offset:2048\n\t"
      "ds_read_b128 %3, %12 offset:3072\n\t"
      "ds_read_b128 %4, %12 offset:4096\n\t"
      "ds_read_b128 %5, %12 offset:5120\n\t"
      "ds_read_b128 %6, %12 offset:6144\n\t"
      "ds_read_b128 %7, %12 offset:7168\n\t"
      "ds_read_b128 %8, %12 offset:8192\n\t"
      "ds_read_b128 %9, %12 offset:9216\n\t"
      "ds_read_b128 %10, %12 offset:10240\n\t"
      "ds_read_b128 %11, %12 offset:11264\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
        "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11])
      : "v"(a)
      : "memory");
}
// fp8 direct path: six 8-byte reads (three addresses, each also at +9216 = 16 rows).
__device__ __forceinline__ void lds_read6_b64(uint32_t a0, uint32_t a1, uint32_t a2, i32x2_t (&r)[6]) {
  asm volatile(
      "ds_read_b64 %0, %6\n\t"
      "ds_read_b64 %1, %6 offset:9216\n\t"
      "ds_read_b64 %2, %7\n\t"
      "ds_read_b64 %3, %7 offset:9216\n\t"
      "ds_read_b64 %4, %8\n\t"
      "ds_read_b64 %5, %8 offset:9216\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5])
      : "v"(a0), "v"(a1), "v"(a2)
      : "memory");
}
// fp8 direct path: four / two 8-byte reads (each address also at +9216 = 16 rows).
__device__ __forceinline__ void lds_read4_b64(uint32_t a0, uint32_t a1, i32x2_t (&r)[4]) {
  asm volatile(
      "ds_read_b64 %0, %4\n\t"
      "ds_read_b64 %1, %4 offset:9216\n\t"
      "ds_read_b64 %2, %5\n\t"
      "ds_read_b64 %3, %5 offset:9216\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(a0), "v"(a1)
      : "memory");
}
__device__ __forceinline__ void lds_read2_b64(uint32_t a0, i32x2_t (&r)[2]) {
  asm volatile(
      "ds_read_b64 %0, %2\n\t"
      "ds_read_b64 %1, %2 offset:9216\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1])
      : "v"(a0)
      : "memory");
}
// fp8 direct path: four transposed 8-bit reads.  In each 16-lane group, lane 2j + h
// gives the address of bytes 8h..8h+7 of its group's row j; lane c receives byte c
// of the group's rows 0..7 (checked on the device).
__device__ __forceinline__ void lds_read4_tr8(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,
                                              i32x2_t (&r)[4]) {
  asm volatile(
      "ds_read_b64_tr_b8 %0, %4\n\t"
      "ds_read_b64_tr_b8 %1, %5\n\t"
      "ds_read_b64_tr_b8 %2, %6\n\t"
      "ds_read_b64_tr_b8 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3)
      : "memory");
}
// Eight e4m3 codes (two words, code k in byte k) -> eight bf16 in order, exactly
// (every e4m3 value is a bf16 value).  Written in asm: the compiler's builtin for
// this instruction mis-packs the two halves of its result.
__device__ __forceinline__ i16x8_t fp8x8_to_bf16(i32x2_t x) {
  uint32_t o0, o1, o2, o3;
  asm("v_cvt_scalef32_pk_bf16_fp8 %0, %1, 1.0" : "=v"(o0) : "v"(x.x));
  asm("v_cvt_scalef32_pk_bf16_fp8 %0, %1, 1.0 op_sel:[1,0,0]" : "=v"(o1) : "v"(x.x));
  asm("v_cvt_scalef32_pk_bf16_fp8 %0, %1, 1.0" : "=v"(o2) : "v"(x.y));
  asm("v_cvt_scalef32_pk_bf16_fp8 %0, %1, 1.0 op_sel:[1,0,0]" : "=v"(o3) : "v"(x.y));
  return as_i16x8(make_uint4(o0, o1, o2, o3));
}
// Eight query elements at element offset e of Q as bf16 bits: bf16 queries, or
// fp8 codes widened exactly (the query scale is in the score scale).
__device__ __forceinline__ i16x8_t load_q8(const AttnParams& p, int64_t e) {
  if (p.q_dtype == FP8)
    return fp8x8_to_bf16(*reinterpret_cast<const i32x2_t*>(static_cast<const uint8_t*>(p.q) + e));
  return *reinterpret_cast<const i16x8_t*>(static_cast<const uint16_t*>(p.q) + e);
}
// Two 16-byte reads.
__device__ __forceinline__ void lds_read2_b128(uint32_t a0, uint32_t a1, i32x4_t& r0, i32x4_t& r1) {
  asm volatile(
      "ds_read_b128 %0, %2\n\t"
      "ds_read_b128 %1, %3\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1)
      : "v"(a0), "v"(a1)
      : "memory");
}
__device__ __forceinline__ i32x4_t lds_read_b128(uint32_t a0) {
  i32x4_t r;
  asm volatile(
      "ds_read_b128 %0, %1\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r)
      : "v"(a0)
      : "memory");
  return r;
}

// LDS swizzle: piece p of row r sits at slot p ^ swz(r) of the row (the XOR stays
// within p's aligned group of 8 pieces).  gfx950's LDS, as measured with
// bank-conflict counters on single read patterns: 64 four-byte banks (256 bytes
// per cycle); a 16-byte read (ds_read_b128) takes four cycles of 16 lanes, the
// lanes of a cycle being those with equal lane / 32 and equal parity of the
// quad index (lane / 4) mod 8; an 8-byte transposed read takes two cycles of 32
// consecutive lanes.  With the 1152-byte pitch (72 16-byte units), row r
// starts at unit 8 (r mod 2) of the 16 units of a bank row.  swz(r) = r & 6
// makes the K operand reads (rows 0-3 and 12-15 at piece p with rows 4-11 at
// piece p + 1 in one cycle, and the other three cycles alike) and the
// transposed V reads (rows 4 lg + 0..3, two pieces, per 32 lanes) hit distinct
// banks; it depends on bits 1 and 2 only, so rows r and r + 16 share it.
__device__ __forceinline__ int mla_swz(int r) { return r & 6; }

// Direct HBM -> LDS load of tile rows [jb, jb + kTK2) (clamped into [.., we)):
// instruction i of the tile fills LDS bytes [1024 i, 1024 i + 1024); lane l
// fills slot 64 i + l = (row, slot q) with piece q ^ swz(row) of that row.
__device__ __forceinline__ void dma_tile(const AttnParams& p, const int* s_pages, uint8_t* stage,
                                         int jb, int we, int wbP, int g, int w, int lane) {
  const uint16_t* kbase = static_cast<const uint16_t*>(p.k);
  const uint32_t ks0 = (uint32_t)p.ks0, ks1 = (uint32_t)p.ks1;
  const uint32_t kc = (uint32_t)(g * p.ks2);
  // recomputed per call (cheap) rather than hoisted and held across the loop
  int ln = lane;
  asm volatile("" : "+v"(ln));
#pragma unroll
  for (int i0 = 0; i0 < kDma; i0 += kNW2) {
    const int i = i0 + w;
    const int slot = 64 * i + ln;
    const int row = slot / kPieces, q = slot - row * kPieces;
    const int piece = q ^ mla_swz(row);
    const int j = jb + row;
    const uint32_t jj = (j < we ? j : we - 1) - wbP;  // a valid token, window-relative
    const uint32_t pi = div_by_magic(jj, p.page_magic);
    const uint32_t pslot = jj - pi * (uint32_t)p.page_size;
    const uint32_t page = s_pages[pi];
    const uint64_t off = (uint64_t)page * ks0 + (pslot * ks1 + kc + 8 * piece);
    if (i < kDma)
      __builtin_amdgcn_global_load_lds(kbase + off, (PA_LDS void*)(stage + 1024 * i), 16, 0, kKvCpol);
  }
}

// fp8 KV: a tile is 32 rows x 576 one-byte codes (36 pieces of 16 codes per row,
// 18 wave instructions).  The narrow and mid kernels read the codes in place from
// a swizzled layout (swz8) and widen them in registers; the many-rows kernel loads
// them linearly and widens the tile into the bf16 layout above (convert_tile).
constexpr int kPieces8 = kDqk / 16;                // 16-byte pieces of an fp8 row (36)
constexpr int kDma8 = kTK2 * kPieces8 / 64;        // 1-KB direct loads per fp8 tile (18)
constexpr int kStage8 = kDma8 * 1024;
static_assert(kTK2 * kPieces8 % 64 == 0, "an fp8 tile is a whole number of 1-KB wave loads");

// fp8 stage layout read in place by the narrow and mid kernels: piece p of row r at slot
// p ^ swz8(r), within p's aligned group of four (36 pieces per row).  With the
// bank model above, the 8-byte K operand reads (32 lanes: rows 0..15, two
// halves) fall on distinct banks; the transposed V reads of a 32-lane cycle
// hold rows t and t + 16 (the token order of P^T), which sit on the same banks
// for any swizzle of bits 0..3, so they take two cycles; a swizzle with bit 4
// would cost the K reads their shared +16-row offset, for four V reads per
// wave and tile.
__device__ __forceinline__ int swz8(int r) { return (r >> 2) & 3; }

// Stage layout of the many-rows kernel for fp8 queries: piece p of row r at slot
// p ^ swzq(r) within p's aligned group of four.  Rows are 576 bytes (36 16-byte
// units), so row r starts at unit 4 r mod 16 of a 256-byte bank row (the bank
// model above).  swzq(r) = r2 + 2 r4 (r_i: bit i of r) puts the K operand reads
// (four cycles of 16 lanes: rows 16 st + 0..15, pieces by lane group) and the
// transposed 8-bit V reads (32 lanes: rows 4q + 0..3 and 16 + 4q + 0..3 of two
// lane groups q, 8 bytes each) on distinct banks.
__device__ __forceinline__ int swzq(int r) { return ((r >> 2) & 1) | (((r >> 4) & 1) << 1); }

// fp8 stage swizzle by layout: 0 linear, 1 swz8, 2 swzq
template <int SW>
__device__ __forceinline__ int fp8_swz(int r) {
  if constexpr (SW == 1) return swz8(r);
  else if constexpr (SW == 2) return swzq(r);
  else return 0;
}

template <int SW = 0>
__device__ __forceinline__ void dma_tile8(const AttnParams& p, const int* s_pages, uint8_t* stage,
                                          int jb, int we, int wbP, int g, int w, int lane) {
  const uint8_t* kbase = static_cast<const uint8_t*>(p.k);
  const uint32_t ks0 = (uint32_t)p.ks0, ks1 = (uint32_t)p.ks1;
  const uint32_t kc = (uint32_t)(g * p.ks2);
  int ln = lane;
  asm volatile("" : "+v"(ln));
#pragma unroll
  for (int i0 = 0; i0 < kDma8; i0 += kNW2) {
    const int i = i0 + w;
    const int slot = 64 * i + ln;
    const int row = slot / kPieces8, piece = slot - row * kPieces8;
    const int j = jb + row;
    const uint32_t jj = (j < we ? j : we - 1) - wbP;
    const uint32_t pi = div_by_magic(jj, p.page_magic);
    const uint32_t pslot = jj - pi * (uint32_t)p.page_size;
    const uint32_t page = s_pages[pi];
    const uint64_t off = (uint64_t)page * ks0 + (pslot * ks1 + kc + 16 * (piece ^ fp8_swz<SW>(row)));
    if (i < kDma8)
      __builtin_amdgcn_global_load_lds(kbase + off, (PA_LDS void*)(stage + 1024 * i), 16, 0, kKvCpol);
  }
}

// Tiles that lie within one page (the page size a multiple of the tile): the
// page's offset is uniform, and the (row, piece) each lane loads is fixed per
// load instruction, so the per-lane part is precomputed once (PageLanes) and a
// load costs a clamp, a multiply-add and the address add.
template <bool FP8, int SW = 0>
struct PageLanes {
  static constexpr int N = ((FP8 ? kDma8 : kDma) + kNW2 - 1) / kNW2;  // load rounds
  int row[N];       // tile row of this lane's piece in round r
  uint32_t off[N];  // element offset of the piece within the row (+ KV head)
  __device__ __forceinline__ void init(const AttnParams& p, int g, int w, int lane) {
#pragma unroll
    for (int r = 0; r < N; ++r) {
      const int i = r * kNW2 + w;
      const int slot = 64 * i + lane;
      if constexpr (FP8) {
        row[r] = slot / kPieces8;
        const int q = slot - row[r] * kPieces8;
        off[r] = (uint32_t)(g * p.ks2) + 16 * (q ^ fp8_swz<SW>(row[r]));
      } else {
        row[r] = slot / kPieces;
        const int q = slot - row[r] * kPieces;
        off[r] = (uint32_t)(g * p.ks2) + 8 * (q ^ mla_swz(row[r]));
      }
    }
  }
};

// (plain functions, one per storage type: a template holding these builtins
// fails to instantiate in the host compilation pass)
#define PA_DMA_PAGE_BODY(E, KD, LANES)                                                        \
  const E* kbase = static_cast<const E*>(p.k);                                                 \
  const uint32_t rel = (uint32_t)(jb - wbP);                                                  \
  const uint32_t pi = div_by_magic(rel, p.page_magic);                                        \
  const uint64_t base = (uint64_t)(uint32_t)page * (uint64_t)p.ks0 +                          \
                        (uint64_t)((rel - pi * (uint32_t)p.page_size) * (uint32_t)p.ks1);     \
  const int last = we - 1 - jb; /* rows past the range load the last valid row */            \
  const uint32_t ks1 = (uint32_t)p.ks1;                                                       \
  _Pragma("unroll") for (int r = 0; r < LANES::N; ++r) {                                      \
    const int i = r * kNW2 + w;                                                               \
    const uint32_t off = (uint32_t)min(pl.row[r], last) * ks1 + pl.off[r];                    \
    if (i < KD)                                                                               \
      __builtin_amdgcn_global_load_lds(kbase + base + off, (PA_LDS void*)(stage + 1024 * i), 16, 0, kKvCpol); \
  }
__device__ __forceinline__ void dma_page_bf16(const AttnParams& p, int page, uint8_t* stage, int jb,
                                              int we, int wbP, const PageLanes<false>& pl, int w) {
  PA_DMA_PAGE_BODY(uint16_t, kDma, PageLanes<false>)
}
__device__ __forceinline__ void dma_page_fp8(const AttnParams& p, int page, uint8_t* stage, int jb,
                                             int we, int wbP, const PageLanes<true>& pl, int w) {
  PA_DMA_PAGE_BODY(uint8_t, kDma8, PageLanes<true>)
}
using PageLanesQ = PageLanes<true, 2>;  // fp8 stages of the fp8-query kernel
// The same with the per-lane part computed per call from a laundered lane index
// (not held in registers across the caller's loop): the many-rows kernels, whose
// registers are taken by Q^T and O^T.
__device__ __forceinline__ void dma_page_bf16_inl(const AttnParams& p, int page, uint8_t* stage, int jb,
                                                  int we, int wbP, int g, int w, int lane) {
  int ln = lane;
  asm volatile("" : "+v"(ln));
  PageLanes<false> pl;
  pl.init(p, g, w, ln);
  PA_DMA_PAGE_BODY(uint16_t, kDma, PageLanes<false>)
}
__device__ __forceinline__ void dma_page_fp8q_inl(const AttnParams& p, int page, uint8_t* stage, int jb,
                                                  int we, int wbP, int g, int w, int lane) {
  int ln = lane;
  asm volatile("" : "+v"(ln));
  PageLanesQ pl;
  pl.init(p, g, w, ln);
  PA_DMA_PAGE_BODY(uint8_t, kDma8, PageLanesQ)
}
__device__ __forceinline__ void dma_page_fp8_inl(const AttnParams& p, int page, uint8_t* stage, int jb,
                                                 int we, int wbP, int g, int w, int lane) {
  int ln = lane;
  asm volatile("" : "+v"(ln));
  PageLanes<true> pl;
  pl.init(p, g, w, ln);
  PA_DMA_PAGE_BODY(uint8_t, kDma8, PageLanes<true>)
}
using PageLanes8S = PageLanes<true, 1>;  // swizzled fp8 stages
__device__ __forceinline__ void dma_page_fp8s(const AttnParams& p, int page, uint8_t* stage, int jb,
                                              int we, int wbP, const PageLanes8S& pl, int w) {
  PA_DMA_PAGE_BODY(uint8_t, kDma8, PageLanes8S)
}
#undef PA_DMA_PAGE_BODY

// fp8 stage -> bf16 tile (swizzled layout of the bf16 path); e4m3 codes widen
// exactly to bf16.  Every thread converts whole 16-code pieces.
// One piece (16 codes of row q / kPieces8) -> its two 16-byte bf16 pieces and
// their LDS addresses in the swizzled tile at dst.
struct WidePiece {
  uint32_t a0, a1;
  i32x4_t v0, v1;
};
__device__ __forceinline__ WidePiece convert_piece(i32x4_t x, int q, uint32_t dst) {
  const int row = q / kPieces8, piece = q - row * kPieces8;
  const uint32_t wv[4] = {(uint32_t)x.x, (uint32_t)x.y, (uint32_t)x.z, (uint32_t)x.w};
  int o[8];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const auto lo2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)wv[h], false);
    const auto hi2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)wv[h], true);
    o[2 * h] = (int)((__float_as_uint(lo2[0]) >> 16) | (__float_as_uint(lo2[1]) & 0xffff0000u));
    o[2 * h + 1] = (int)((__float_as_uint(hi2[0]) >> 16) | (__float_as_uint(hi2[1]) & 0xffff0000u));
  }
  const int sw = mla_swz(row);
  const uint32_t drow = dst + row * kKP2;
  return WidePiece{drow + 16 * ((2 * piece) ^ sw), drow + 16 * ((2 * piece + 1) ^ sw),
                   i32x4_t{o[0], o[1], o[2], o[3]}, i32x4_t{o[4], o[5], o[6], o[7]}};
}

// Widening of a whole tile by the workgroup's threads (three rounds at most: two
// pieces, then a third for the first threads).
__device__ __forceinline__ void convert_tile(const uint8_t* src, uint8_t* dst, int tid_in) {
  constexpr int n = 64 * kNW2;
  static_assert(kTK2 * kPieces8 > 2 * n && kTK2 * kPieces8 <= 3 * n, "three rounds");
  // the per-thread addresses are recomputed per call (cheap) rather than hoisted
  // out of the tile loop, where they were spilled and reloaded behind a wait
  // that also drained the tiles in flight
  int tid = tid_in;
  asm volatile("" : "+v"(tid));
  const uint32_t a = lds_off(src) + 16 * tid;
  const uint32_t d = lds_off(dst);
  i32x4_t x0, x1;
  lds_read2_b128(a, a + 16 * n, x0, x1);
  const WidePiece p0 = convert_piece(x0, tid, d);
  const WidePiece p1 = convert_piece(x1, tid + n, d);
  lds_write4_b128(p0.a0, p0.v0, p0.a1, p0.v1, p1.a0, p1.v0, p1.a1, p1.v1);
  if (tid + 2 * n < kTK2 * kPieces8) {
    const WidePiece p2 = convert_piece(lds_read_b128(a + 2 * 16 * n), tid + 2 * n, d);
    lds_write2_b128(p2.a0, p2.v0, p2.a1, p2.v1);
  }
}

// Token range of explicit split c of request b (pages [c n / S, (c + 1) n / S)).
__device__ __forceinline__ void mla_item_range(const AttnParams& p, int b, int c, int& L, int& j0, int& j1) {
  const int kb = p.broadcast ? 0 : b;
  const int n = p.kv_indptr[kb + 1] - p.kv_indptr[kb];
  L = n ? (n - 1) * p.page_size + p.kv_last[kb] : 0;
  j0 = (int)(((int64_t)c * n / p.num_splits) * p.page_size);
  j1 = min((int)(((int64_t)(c + 1) * n / p.num_splits) * p.page_size), L);
}

struct MlaRow {
  float m;         // reference max (log2 units, scaled); re-based lazily
  float lsum;      // this lane's partial sum
  float true_max;  // running row max
};

// One 32-token tile of math for this wave's 16 rows (lane: row l16, group lg).
__device__ __forceinline__ void mla_rows_tile(const uint8_t* kv, int jb, int lim, bool need_mask,
                                              const i16x8_t (&qreg)[kDqk / 32], float qk_scale,
                                              MlaRow& st, f32x4_t (&oacc)[kDvo / 16], int lane) {
  constexpr int KK = kDqk / 32, NDT = kDvo / 16;
  int ln = lane;  // per-lane offsets recomputed per tile, not held across the loop
  asm volatile("" : "+v"(ln));
  const int l16 = ln & 15, lg = ln >> 4;
  // S^T[token][row] = K Q^T: two 16-token blocks.  The 36 K operands (k-step
  // kk, block st: f = 2 kk + st) are read kPF ahead of their MFMAs from a ring
  // of registers; the scheduling barriers keep that order.
  constexpr int kPF = 4;
  f32x4_t sacc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
  // K operand of k-step kk, block st: row 16 st + l16, piece 4 kk + lg, whose
  // low three bits are 4 (kk % 2) + lg; swz(row) is the same for both blocks
  const int sw = mla_swz(l16);
  const int kq0 = l16 * kKP2 + 16 * (lg ^ sw);        // even k-steps (byte offsets)
  const int kq1 = l16 * kKP2 + 16 * ((lg + 4) ^ sw);  // odd k-steps
  auto kfrag = [&](int f) __attribute__((always_inline)) {
    const int kk = f >> 1;
    return *reinterpret_cast<const i16x8_t*>(kv + (kk & 1 ? kq1 : kq0) + 16 * (f & 1) * kKP2 +
                                             128 * (kk >> 1));
  };
  i16x8_t ring[kPF];
#pragma unroll
  for (int f = 0; f < kPF; ++f) ring[f] = kfrag(f);
#pragma unroll
  for (int f = 0; f < 2 * KK; ++f) {
    const i16x8_t a = ring[f % kPF];
    if (f + kPF < 2 * KK) ring[f % kPF] = kfrag(f + kPF);
    sacc[f & 1] = mfma16<BF16>(a, qreg[f >> 1], sacc[f & 1]);
    __builtin_amdgcn_sched_barrier(0);
  }
  // lane holds row l16, tokens jb + 16st + 4lg + i
  float sv[2][4];
  float tmax = -INFINITY;
  if (need_mask) {
    const int rel = lim - jb - 4 * lg;  // token 16 st + 4 lg + i is in range iff 16 st + i < rel
#pragma unroll
    for (int st2 = 0; st2 < 2; ++st2)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[st2][i] = 16 * st2 + i < rel ? sacc[st2][i] : -INFINITY;
        tmax = fmaxf(tmax, sv[st2][i]);
      }
  } else {
#pragma unroll
    for (int st2 = 0; st2 < 2; ++st2)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[st2][i] = sacc[st2][i];
        tmax = fmaxf(tmax, sv[st2][i]);
      }
  }
  tmax = xor32_max(xor16_max(tmax)) * qk_scale;
  st.true_max = fmaxf(st.true_max, tmax);
  // lazily re-based reference max: O is rescaled only when a row max grows by
  // more than 2^8 (P <= 2^8 stays well inside bf16 and fp32 sums)
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
  const float nmref = -(st.m == -INFINITY ? 0.f : st.m);
  float e[8];
#pragma unroll
  for (int st2 = 0; st2 < 2; ++st2)
#pragma unroll
    for (int i = 0; i < 4; ++i) e[4 * st2 + i] = fast_exp2(fmaf(sv[st2][i], qk_scale, nmref));
  const uint4 bits = make_uint4(pack2<BF16>(e[0], e[1]), pack2<BF16>(e[2], e[3]),
                                pack2<BF16>(e[4], e[5]), pack2<BF16>(e[6], e[7]));
  const i16x8_t pb = as_i16x8(bits);
  st.lsum = sum2<BF16>(bits.x, sum2<BF16>(bits.y, sum2<BF16>(bits.z, sum2<BF16>(bits.w, st.lsum))));
  // O^T += V^T P^T: V^T 16 dims x (tokens 4lg..4lg+3, 16+4lg..16+4lg+3) by two
  // transposed 4x16 reads, matching the token order of P^T above
  // lane reads 4 dims (8 bytes) of row rr = 4 lg + l16/4 (and rr + 16, same
  // swizzle): dims 16 d + 4 (l16 % 4) = piece 2 d + (l16 % 4) / 2, half l16 % 2;
  // the piece's low three bits are 2 (d % 4) + (l16 % 4) / 2
  const int rr = 4 * lg + (l16 >> 2);
  const int vsw = mla_swz(rr);
  const int vb = rr * kKP2 + 8 * (l16 & 1);
  const int hp = (l16 & 3) >> 1;
  const int vq[4] = {vb + 16 * ((0 + hp) ^ vsw), vb + 16 * ((2 + hp) ^ vsw),
                     vb + 16 * ((4 + hp) ^ vsw), vb + 16 * ((6 + hp) ^ vsw)};
  constexpr int kPV = 3;  // V^T operands in flight
  i16x8_t vring[kPV];
  auto vfrag = [&](int d) __attribute__((always_inline)) {
    const uint16_t* a0 = reinterpret_cast<const uint16_t*>(kv + vq[d & 3] + 128 * (d >> 2));
    const i16x4_t lo4 = lds_read_tr(a0);
    const i16x4_t hi4 = lds_read_tr(a0 + 16 * (kKP2 / 2));
    return i16x8_t{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
  };
#pragma unroll
  for (int d = 0; d < kPV; ++d) vring[d] = vfrag(d);
#pragma unroll
  for (int d = 0; d < NDT; ++d) {
    const i16x8_t va = vring[d % kPV];
    if (d + kPV < NDT) vring[d % kPV] = vfrag(d + kPV);
    oacc[d] = mfma16<BF16>(va, pb, oacc[d]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One (request b, KV head g, row tile from row0) token range [j0, j1) of the
// many-rows kernel; output as for the narrow kernel.  Called by every thread.
template <bool FP8>
__device__ __forceinline__ void mla_rows_range(const AttnParams& p, int b, int g, int rt, int L, int j0,
                                               int j1, bool to_ws, int64_t wslot, int c, uint8_t* s_kv0,
                                               uint8_t* s_kv1, uint8_t* s_kv2, uint8_t* s_kv3,
                                               uint8_t* s_wide, int* s_pages) {
  constexpr int KK = kDqk / 32;   // 18 k-steps of Q.K (16x16x32)
  constexpr int NDT = kDvo / 16;  // 32 16-dim tiles of O
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar registers
  const int l16 = lane & 15, lg = lane >> 4;
  // the range is the workgroup's: scalar registers
  b = uni(b);
  g = uni(g);
  L = uni(L);
  j0 = uni(j0);
  j1 = uni(j1);
  const int kb = p.broadcast ? 0 : b;
  const int pbeg = p.kv_indptr[kb];
  const int R = p.q_len * p.group;
  const int row0 = rt * kRT2;

  // ---- this lane's row (B-operand column / C column): wave w rows 16w..16w+15
  const int row = row0 + kRW * w + l16;
  const bool row_ok = row < R;
  int lim = j1;
  if (row_ok && p.causal) lim = min(lim, L - p.q_len + row / p.group + 1);
  if (!row_ok) lim = INT_MIN;
  int lo = row_ok ? lim : INT_MAX;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) lo = min(lo, __shfl_xor(lo, off, 64));
  const int wave_lim_min = __builtin_amdgcn_readfirstlane(lo);
  const bool wave_live = wave_lim_min != INT_MAX;  // the wave has a valid row
  int jhi = j1;  // workgroup's last visible token
  if (p.causal) jhi = min(j1, L - p.q_len + (min(row0 + kRT2, R) - 1) / p.group + 1);

  i16x8_t qreg[KK];
  {
    const int qi = row_ok ? row / p.group : 0, qh = row_ok ? row % p.group : 0;
    const int64_t qe =
        ((int64_t)(b * p.q_len + qi) * p.num_qo_heads + (int64_t)g * p.group + qh) * kDqk + 8 * lg;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qreg[kk] = row_ok ? load_q8(p, qe + 32 * kk) : i16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
  }

  MlaRow st{-INFINITY, 0.f, -INFINITY};
  f32x4_t oacc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) oacc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const float qk_scale = p.sm_scale * p.k_scale * kLog2e;
  const int P = p.page_size;

  if (jhi > j0) {
    const int pfirst = j0 / P, plast = (jhi - 1) / P;
    for (int wb = pfirst; wb <= plast; wb += kPageWinM) {
      const int npw = min(kPageWinM, plast - wb + 1);
      __syncthreads();  // the previous window's readers are done
      for (int i = tid; i < npw; i += 64 * kNW2) s_pages[i] = p.kv_indices[pbeg + wb + i];
      __syncthreads();
      const int ws = max(j0, wb * P), we = min(jhi, (wb + npw) * P);
      const int nk = (we - ws + kTK2 - 1) / kTK2;
      // tile k lives in stage k % 4; tiles k+1..k+3 are in flight during the
      // math of tile k.  A wave issues kMinDma direct loads per tile, so
      // vmcnt(2 kMinDma) after issuing tile k+2 means tile k's loads are done;
      // the barrier then covers every wave's loads, and every wave is done with
      // tile k-1, whose stage takes tile k+3.
      constexpr int kMinDma = (FP8 ? kDma8 : kDma) / kNW2;  // direct loads per wave per tile
      constexpr int kWait = 2 * kMinDma;     // vmcnt that leaves only tiles k+1, k+2 in flight
      static_assert(kWait < 64, "vmcnt field");
      constexpr int kWaitImm = (kWait & 0xF) | ((kWait >> 4) << 14) | 0x70 | 0xF00;
      const int wbP = wb * P;
      auto tile_at = [&](int k) { return ws + min(k, nk - 1) * kTK2; };
      // tiles within one page (page size a multiple of the tile, page-aligned
      // range): lane i of ptab holds the page id of tile 64 (k / 64) + i, and a
      // tile's loads take it with one uniform lane read (tiles are issued in
      // order 0, 1, 2, ...) instead of a per-lane page-table walk through LDS
      const bool page_tiles = P % kTK2 == 0 && ws % kTK2 == 0;
      int ptab = 0;
      auto dma = [&](uint8_t* stage, int k) __attribute__((always_inline)) {
        const int jb = tile_at(k);
        if (page_tiles) {
          if ((k & 63) == 0) ptab = s_pages[div_by_magic((uint32_t)(tile_at(k + lane) - wbP), p.page_magic)];
          const int page = __builtin_amdgcn_readlane(ptab, k & 63);
          if constexpr (FP8)
            dma_page_fp8_inl(p, page, stage, jb, we, wbP, g, w, lane);
          else
            dma_page_bf16_inl(p, page, stage, jb, we, wbP, g, w, lane);
        } else if constexpr (FP8) {
          dma_tile8(p, s_pages, stage, jb, we, wbP, g, w, lane);
        } else {
          dma_tile(p, s_pages, stage, jb, we, wbP, g, w, lane);
        }
      };
      dma(s_kv0, 0);
      dma(s_kv1, 1);
      dma(s_kv2, 2);
      // fp8: the landed stage is widened into s_wide (a second barrier publishes
      // it; the first one also says every wave is done with the previous tile)
#define PA_MLA_STEP(K, CUR, NEXT3)                                                            \
  {                                                                                         \
    __builtin_amdgcn_s_waitcnt(kWaitImm); /* this wave's loads of tile K are done */        \
    lds_barrier(); /* every wave's; no wait for the tiles behind it */                      \
    dma(NEXT3, (K) + 3);                                                                    \
    const uint8_t* src = CUR;                                                               \
    if constexpr (FP8) {                                                                    \
      convert_tile(CUR, s_wide, tid);                                                       \
      lds_barrier();                                                                         \
      src = s_wide;                                                                         \
    }                                                                                       \
    const int jb = ws + (K) * kTK2;                                                         \
    if (wave_live)                                                                          \
      mla_rows_tile(src, jb, lim, jb + kTK2 > wave_lim_min, qreg, qk_scale, st, oacc, lane); \
  }
      for (int k = 0; k < nk; k += 4) {
        PA_MLA_STEP(k, s_kv0, s_kv3);
        if (k + 1 >= nk) break;
        PA_MLA_STEP(k + 1, s_kv1, s_kv0);
        if (k + 2 >= nk) break;
        PA_MLA_STEP(k + 2, s_kv2, s_kv1);
        if (k + 3 >= nk) break;
        PA_MLA_STEP(k + 3, s_kv3, s_kv2);
      }
#undef PA_MLA_STEP
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no loads in flight into the stages
      __syncthreads();
    }
  }

  // ---- epilogue: lane (row l16, group lg) holds dims 16d + 4lg + (0..3)
  const float ltot = xor32_sum(xor16_sum(st.lsum));
  if (!row_ok) return;
  const bool empty = !(ltot > 0.f);
  const float scale = empty ? 0.f : p.v_scale / ltot;
  const int64_t rid = (int64_t)(b * p.q_len + row / p.group) * p.num_qo_heads + (int64_t)g * p.group +
                      row % p.group;
  const int64_t wrow = wslot * p.ws_rows + row;  // workspace row (balanced split)
#pragma unroll
  for (int d = 0; d < NDT; ++d) {
    const int dim = 16 * d + 4 * lg;
    const float x0 = oacc[d][0] * scale, x1 = oacc[d][1] * scale;
    const float x2 = oacc[d][2] * scale, x3 = oacc[d][3] * scale;
    if (to_ws) {
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.ws_o) + wrow * kDvo + dim) =
          make_uint2(pack2<BF16>(x0, x1), pack2<BF16>(x2, x3));  // bf16 partial state
    } else if (p.o_dtype == F32) {
      *reinterpret_cast<float4*>(static_cast<float*>(p.o) + c * p.o_split_stride + rid * kDvo + dim) =
          make_float4(x0, x1, x2, x3);
    } else {
      const uint2 v = p.o_dtype == F16 ? make_uint2(pack2<F16>(x0, x1), pack2<F16>(x2, x3))
                                       : make_uint2(pack2<BF16>(x0, x1), pack2<BF16>(x2, x3));
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.o) + c * p.o_split_stride + rid * kDvo + dim) = v;
    }
  }
  if (lg == 0) {
    const float lse = empty ? -INFINITY : (st.m + fast_log2(ltot)) * kLn2;
    const float mx = empty ? -INFINITY : st.true_max * kLn2;
    if (to_ws) {
      p.ws_lse[wrow] = lse;
      p.ws_mx[wrow] = mx;
    } else {
      const int64_t sidx = c * p.s_split_stride + rid;
      if (p.lse) p.lse[sidx] = lse;
      if (p.mx) p.mx[sidx] = mx;
    }
  }
}

// Workgroups: (request, KV head, row tile, explicit split) items, the row tiles
// of one item on one XCD so its KV range is read once into that L2; or, under
// the balanced split, equal shares of the (request, KV head, 32-token unit)
// sequence, each taken by one workgroup per row tile on one XCD.
template <bool FP8>
__global__ __launch_bounds__(64 * kNW2, 1) void mla_rows_kernel(AttnParams p, int nrt, int ngroups) {
  // four stages (distinct LDS objects, so the compiler's wait counting tells
  // the direct loads into one stage from the reads of another)
  constexpr int STAGE = FP8 ? kStage8 : kStage2;
  __shared__ __align__(16) uint8_t s_kv0[STAGE];
  __shared__ __align__(16) uint8_t s_kv1[STAGE];
  __shared__ __align__(16) uint8_t s_kv2[STAGE];
  __shared__ __align__(16) uint8_t s_kv3[STAGE];
  __shared__ __align__(16) uint8_t s_wide[FP8 ? kStage2 : 16];  // fp8: the widened tile
  __shared__ int s_pages[kPageWinM];
  if (p.bal_blocks > 0) {
    BalCursor cur;
    if (!cur.start(p, blockIdx.x)) return;
    do {
      mla_rows_range<FP8>(p, cur.b, cur.g, cur.rt, cur.L, cur.j0(p), cur.j1(p),
                          !cur.whole(), cur.slot(p), 0, s_kv0, s_kv1, s_kv2, s_kv3, s_wide, s_pages);
    } while (cur.next(p));
    return;
  }
  const int lam = blockIdx.x;
  const int xcd = lam % 8, k8 = lam / 8;
  const int rt = k8 % nrt;
  const int gi = (k8 / nrt) * 8 + xcd;
  if (gi >= ngroups) return;
  const int b = gi / (p.num_kv_heads * p.num_splits);
  const int g = (gi / p.num_splits) % p.num_kv_heads;
  const int c = gi % p.num_splits;
  int L, j0, j1;
  mla_item_range(p, b, c, L, j0, j1);
  mla_rows_range<FP8>(p, b, g, rt, L, j0, j1, false, 0,
                      c, s_kv0, s_kv1, s_kv2, s_kv3, s_wide, s_pages);
}

// ---------------------------------------------------------------------------
// fp8 queries over an fp8 cache, more than 16 rows per request: both products
// on the fp8 matrix cores (the FP8 MLA decode that the FlashInfer PR #3309
// analysis targets, introduction).  The workgroup shape is that of the many-rows
// kernel (8 waves x 16 rows), but a tile is 128 tokens, one k-step of the fp8
// MFMA along the tokens, kept as fp8 codes in LDS (swzq layout) in two stages of
// 72 KB fed by direct loads (the load of tile k + 1 runs during the math of
// tile k); nothing is widened:
//   S^T = K Q^T on v_mfma_scale_f32_16x16x128_f8f6f4 with unit block scales
//   (the per-tensor query and cache scales are in the score scale): K codes
//   from LDS as the A operand (32 per lane, two 16-byte reads), the rows' Q^T
//   codes in registers as the B operand (40 registers); the 576 dims are four
//   128-dim k-steps and one of 64 dims, whose other half is zero in Q^T;
//   online softmax as in mla_rows_tile, over 128 tokens at a time;
//   O^T += V^T P^T on the same MFMA, V^T read by transposed 8-bit reads
//   (ds_read_b64_tr_b8, four per operand) in P^T's token order.  P in e4m3
//   alone (4 significant bits) is too coarse for the fp8-KV error bar when a
//   few tokens dominate a row, so P = hi + lo / 16 with hi = e4m3(P) and
//   lo = e4m3(16 (P - hi)), two MFMAs per 16-dim block of O, the second with
//   the block scale 2^-4 on P^T: about 8 significant bits, as bf16.
// The two operands of the fp8 MFMA pair their (lane group, byte) positions
// identically (checked on the device), so a lane group's 32 bytes may hold any
// 32 dims (or tokens) as long as both operands hold the same ones in the same
// places.
typedef int i32x8_t __attribute__((ext_vector_type(8)));
constexpr int kKS8 = 5;  // k-steps of 128 dims (the last one half used)
constexpr int kTKQ = 128;                       // KV tokens per tile
constexpr int kDmaQ = kTKQ * kPieces8 / 64;     // 1-KB direct loads per tile (72)
constexpr int kStageQ = kDmaQ * 1024;           // 73728 bytes
constexpr int kRoundsQ = kDmaQ / kNW2;          // loads per wave per tile (9)
constexpr int kQuarterQ = 32 * kPieces8 * 16;   // bytes of 32 token rows
static_assert(kDmaQ % kNW2 == 0, "every wave issues the same number of tile loads");
static_assert(kRoundsQ * 1024 == 16 * kPieces8 * 16, "each wave's loads fill 16 whole rows");

// Block scales (E8M0) of the fp8 MFMAs: byte 0 = 127 (2^0), byte 1 = 123 (2^-4),
// one register for both (the instruction picks a byte of its scale operands).
constexpr int kScales = 127 | (123 << 8);
__device__ __forceinline__ f32x4_t mfma_fp8(const i32x8_t& a, const i32x8_t& b, f32x4_t c) {
  // format 0 (e4m3) for both operands, block scales 2^0
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, kScales, 0, kScales);
}
__device__ __forceinline__ f32x4_t mfma_fp8_b16th(const i32x8_t& a, const i32x8_t& b, f32x4_t c) {
  // the same with the B operand's block scale 2^-4
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, kScales, 1, kScales);
}

// One direct HBM -> LDS load of 16 bytes per lane (lane l fills LDS bytes
// [lds + 16 l, lds + 16 l + 16)), issued in asm: the compiler does not count it,
// so it inserts no waits for it before LDS reads that it cannot tell apart from
// the stage being filled (the caller waits with an explicit vmcnt(0) and a
// barrier before a stage is read).  M0 holds the LDS address; one wait state
// between its write and the load; non-temporal, as kKvCpol.
__device__ __forceinline__ void lds_dma16(const void* gaddr, uint8_t* lds) {
  const uint32_t a = (uint32_t)(uintptr_t)(PA_LDS uint8_t*)lds;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :
               : "v"(gaddr), "s"(a)
               : "memory", "m0");
}

// Direct loads of tile rows [jb, jb + 128) (rows past `we` load row we - 1):
// wave w fills LDS bytes [9216 w, 9216 w + 9216), tile rows 16 w .. 16 w + 15,
// with nine loads; lane l of load r fills slot v = 64 r + l of those rows, i.e.
// row 16 w + v / 36, slot v mod 36, with piece (v mod 36) ^ swzq(row).  PAGED:
// the page size and the window-relative tile start are multiples of 64, so
// each 64-row half of the tile (waves 0..3, waves 4..7) lies in one page, whose
// base comes from scalar registers; otherwise every lane looks up its row's page.
template <bool PAGED>
__device__ __forceinline__ void dma_tileq(const AttnParams& p, const int* s_pages, uint8_t* stage,
                                          int jb, int we, int wbP, int g, int w, int lane) {
  const uint8_t* kbase = static_cast<const uint8_t*>(p.k);
  const uint32_t ks0 = (uint32_t)p.ks0, ks1 = (uint32_t)p.ks1;
  const uint32_t kc = (uint32_t)(g * p.ks2);
  const int last = we - 1 - jb;
  int ln = lane;  // recomputed per call rather than held across the tile loop
  asm volatile("" : "+v"(ln));
  uint64_t hbase = 0;
  int hdelta = 0;
  if constexpr (PAGED) {
    // the 64-token block holding the wave's half's first row (or row we - 1)
    const uint32_t rel = (uint32_t)(min(jb + (w >= 4 ? 64 : 0), we - 1) - wbP) & ~63u;
    const uint32_t pi = div_by_magic(rel, p.page_magic);
    const uint32_t page = (uint32_t)s_pages[pi];
    hbase = (uint64_t)page * ks0 + (uint64_t)((rel - pi * (uint32_t)p.page_size) * ks1 + kc);
    hdelta = jb - wbP - (int)rel;  // tile row + delta: row within the block
  }
  const int sw4 = (w & 1) << 1;  // bit 4 of row 16 w + lr (lr < 16), as swzq's bit 1
#pragma unroll
  for (int r = 0; r < kRoundsQ; ++r) {
    const int v = 64 * r + ln;
    const int lr = (v * 1821) >> 16;  // v / 36 for v < 576
    const int q = v - 36 * lr;
    const int row = 16 * w + lr;
    const uint32_t pc = 16 * (q ^ (((lr >> 2) & 1) | sw4));
    const int rr = min(row, last);
    uint64_t off;
    if constexpr (PAGED) {
      off = hbase + (uint32_t)((rr + hdelta) * (int)ks1) + pc;
    } else {
      const uint32_t jj = (uint32_t)(jb + rr - wbP);
      const uint32_t pi = div_by_magic(jj, p.page_magic);
      const uint32_t pslot = jj - pi * (uint32_t)p.page_size;
      const uint32_t page = (uint32_t)s_pages[pi];
      off = (uint64_t)page * ks0 + (pslot * ks1 + kc + pc);
    }
    lds_dma16(kbase + off, stage + 1024 * (kRoundsQ * w + r));
  }
}

// Splits four probabilities (one lane's tokens of a 16-token block) into one
// e4m3 word each: hi = e4m3(p), lo = e4m3(16 (p - hi)) (p - hi exact in fp32).
__device__ __forceinline__ void split_p8(const float (&p)[4], int& hi, int& lo) {
  // (the first conversion of a word keeps the other half of its third operand:
  // any live value, overwritten by the second)
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], __float_as_int(p[0]), false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], hi, true);
  // 16 hi, exactly (e4m3 values times a power of two)
  const auto a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi, 16.f, false);
  const auto b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi, 16.f, true);
  const float r0 = fmaf(p[0], 16.f, -a[0]), r1 = fmaf(p[1], 16.f, -a[1]);
  const float r2 = fmaf(p[2], 16.f, -b[0]), r3 = fmaf(p[3], 16.f, -b[1]);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(r0, r1, __float_as_int(r0), false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(r2, r3, lo, true);
}

// One 128-token tile of math for this wave's 16 rows (lane: row l16, group lg).
__device__ __forceinline__ void mla_rows8_tile(const uint8_t* kv, int jb, int lim, bool need_mask,
                                               const i32x8_t (&qreg)[kKS8], float qk_scale,
                                               MlaRow& st, f32x4_t (&oacc)[kDvo / 16], int lane) {
  constexpr int NDT = kDvo / 16;
  constexpr int kPitch = kPieces8 * 16;  // 576-byte fp8 rows
  constexpr int NB = kTKQ / 16;          // 16-token blocks (8)
  int ln = lane;  // per-lane offsets recomputed per tile, not held across the loop
  asm volatile("" : "+v"(ln));
  const int l16 = ln & 15, lg = ln >> 4;
  // K operand of k-step ks, block t: row 16 t + l16, pieces 8 ks + 2 lg + e
  // (e = 0, 1), i.e. slot 8 ks + 4 (lg >> 1) + ((2 (lg & 1) + e) ^ swzq(row)).
  // swzq depends on row bits 2 and 4 only: four per-lane bases (t & 1, e), the
  // block pair t >> 1 adding 32 rows and the k-step 128 bytes.  K-step 4 has
  // pieces 32..35 only (lane groups 0 and 1); lane groups 2 and 3 read pieces
  // 32..35 of their row again (in bounds, finite codes) against zero Q^T codes.
  // (Addresses stay pointers into the stage, so the compiler's wait counting
  // sees which stage a read touches and does not wait for the loads in flight
  // into the other one.)
  const int sw0 = swzq(l16);  // odd blocks: sw0 ^ 2
  int kb[2][2];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int e = 0; e < 2; ++e)
      kb[tb][e] = (16 * tb + l16) * kPitch + 64 * (lg >> 1) + 16 * ((2 * (lg & 1) + e) ^ (sw0 ^ (2 * tb)));
  // fragment f: k-step f / NB, block f % NB (the blocks' accumulators independent)
  auto kfrag = [&](int f) __attribute__((always_inline)) {
    const int ks = f / NB, t = f % NB;
    int b0 = kb[t & 1][0], b1 = kb[t & 1][1];
    if (ks == kKS8 - 1) {
      // lane groups 2 and 3: back by 64 bytes (computed here, per read, rather
      // than kept as per-lane offset constants)
      const int back = ln & 32 ? 64 : 0;
      b0 -= back;
      b1 -= back;
      asm volatile("" : "+v"(b0), "+v"(b1));
    }
    const int o = kQuarterQ * (t >> 1) + 128 * ks;
    const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(kv + b0 + o);
    const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(kv + b1 + o);
    return i32x8_t{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  };
  constexpr int NF = NB * kKS8;
  constexpr int kPF = 2;  // K operands in flight
  f32x4_t sacc[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) sacc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  i32x8_t ring[kPF];
#pragma unroll
  for (int f = 0; f < kPF; ++f) ring[f] = kfrag(f);
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const i32x8_t a = ring[f % kPF];
    if (f + kPF < NF) ring[f % kPF] = kfrag(f + kPF);
    sacc[f % NB] = mfma_fp8(a, qreg[f / NB], sacc[f % NB]);
    __builtin_amdgcn_sched_barrier(0);
  }
  // lane holds row l16, tokens jb + 16 t + 4 lg + i
  float sv[NB][4];
  float tmax = -INFINITY;
  if (need_mask) {
    const int rel = lim - jb - 4 * lg;  // token 16 t + 4 lg + i is in range iff 16 t + i < rel
#pragma unroll
    for (int t = 0; t < NB; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[t][i] = 16 * t + i < rel ? sacc[t][i] : -INFINITY;
        tmax = fmaxf(tmax, sv[t][i]);
      }
  } else {
#pragma unroll
    for (int t = 0; t < NB; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[t][i] = sacc[t][i];
        tmax = fmaxf(tmax, sv[t][i]);
      }
  }
  tmax = xor32_max(xor16_max(tmax)) * qk_scale;
  st.true_max = fmaxf(st.true_max, tmax);
  // lazily re-based reference max (as in mla_rows_tile): P <= 2^8, inside e4m3
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
  const float nmref = -(st.m == -INFINITY ? 0.f : st.m);
  // P^T operands: byte 4 t + i of lane (row, lg) is token 16 t + 4 lg + i
  i32x8_t phi, plo;
  float psum = 0.f;
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    float e[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) e[i] = fast_exp2(fmaf(sv[t][i], qk_scale, nmref));
    psum += (e[0] + e[1]) + (e[2] + e[3]);
    int hw, lw;
    split_p8(e, hw, lw);
    phi[t] = hw;
    plo[t] = lw;
  }
  st.lsum += psum;
  // O^T += V^T P^T: V^T operand of dim block d, read r (bytes 8r..8r+7 = blocks
  // 2r, 2r + 1): in each 16-lane group q, lane 2j + h addresses bytes 8h..8h+7 of
  // the dim block's piece in token row 32 r + trow(q, j), and lane c receives dim
  // c of the group's eight rows: tokens 32 r + 4q + j (j < 4) and
  // 32 r + 16 + 4q + (j - 4), the token order of P^T above
  const int q = ln >> 4, jr = (ln & 15) >> 1, h = ln & 1;
  const int trow = jr < 4 ? 4 * q + jr : 12 + 4 * q + jr;
  const int tsw = swzq(trow);  // = swzq(trow + 32 r)
  // dim block d sits at slot 4 (d >> 2) + ((d & 3) ^ tsw): four per-lane bases
  // (d mod 4), the block group adding 64 (d >> 2) bytes
  int vb[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) vb[u] = trow * kPitch + 8 * h + 16 * (u ^ tsw);
  auto vfrag = [&](int d) __attribute__((always_inline)) {
    const uint8_t* a = kv + vb[d & 3] + 64 * (d >> 2);
    const i32x2_t x0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((PA_LDS i32x2_t*)(a));
    const i32x2_t x1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((PA_LDS i32x2_t*)(a + kQuarterQ));
    const i32x2_t x2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((PA_LDS i32x2_t*)(a + 2 * kQuarterQ));
    const i32x2_t x3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((PA_LDS i32x2_t*)(a + 3 * kQuarterQ));
    return i32x8_t{x0.x, x0.y, x1.x, x1.y, x2.x, x2.y, x3.x, x3.y};
  };
  constexpr int kPV = 2;  // V^T operands in flight
  i32x8_t vring[kPV];
#pragma unroll
  for (int d = 0; d < kPV; ++d) vring[d] = vfrag(d);
#pragma unroll
  for (int d = 0; d < NDT; ++d) {
    const i32x8_t va = vring[d % kPV];
    if (d + kPV < NDT) vring[d % kPV] = vfrag(d + kPV);
    oacc[d] = mfma_fp8(va, phi, oacc[d]);
    oacc[d] = mfma_fp8_b16th(va, plo, oacc[d]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One (request b, KV head g, row tile rt) token range [j0, j1) of the fp8-query
// many-rows kernel; output as for the narrow kernel.  Called by every thread.
__device__ __forceinline__ void mla_rows8_range(const AttnParams& p, int b, int g, int rt, int L, int j0,
                                                int j1, bool to_ws, int64_t wslot, int c, uint8_t* s_kv0,
                                                uint8_t* s_kv1, int* s_pages) {
  constexpr int NDT = kDvo / 16;  // 32 16-dim tiles of O
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar registers
  const int l16 = lane & 15, lg = lane >> 4;
  b = uni(b);
  g = uni(g);
  L = uni(L);
  j0 = uni(j0);
  j1 = uni(j1);
  const int kb = p.broadcast ? 0 : b;
  const int pbeg = p.kv_indptr[kb];
  const int R = p.q_len * p.group;
  const int row0 = rt * kRT2;

  const int row = row0 + kRW * w + l16;
  const bool row_ok = row < R;
  int lim = j1;
  if (row_ok && p.causal) lim = min(lim, L - p.q_len + row / p.group + 1);
  if (!row_ok) lim = INT_MIN;
  int lo = row_ok ? lim : INT_MAX;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) lo = min(lo, __shfl_xor(lo, off, 64));
  const int wave_lim_min = __builtin_amdgcn_readfirstlane(lo);
  const bool wave_live = wave_lim_min != INT_MAX;
  int jhi = j1;
  if (p.causal) jhi = min(j1, L - p.q_len + (min(row0 + kRT2, R) - 1) / p.group + 1);

  // Q^T codes: k-step ks, lane group lg holds dims 128 ks + 32 lg .. + 31 of row
  // (k-step 4: dims 512..575 in lane groups 0 and 1, zeros in 2 and 3)
  i32x8_t qreg[kKS8];
  {
    const int qi = row_ok ? row / p.group : 0, qh = row_ok ? row % p.group : 0;
    const uint8_t* qp = static_cast<const uint8_t*>(p.q) +
                        ((int64_t)(b * p.q_len + qi) * p.num_qo_heads + (int64_t)g * p.group + qh) * kDqk +
                        32 * lg;
#pragma unroll
    for (int ks = 0; ks < kKS8; ++ks) {
      const bool ok = row_ok && (ks < kKS8 - 1 || lg < 2);
      const i32x4_t z = {0, 0, 0, 0};
      const i32x4_t a = ok ? *reinterpret_cast<const i32x4_t*>(qp + 128 * ks) : z;
      const i32x4_t bq = ok ? *reinterpret_cast<const i32x4_t*>(qp + 128 * ks + 16) : z;
      qreg[ks] = i32x8_t{a.x, a.y, a.z, a.w, bq.x, bq.y, bq.z, bq.w};
    }
  }

  MlaRow st{-INFINITY, 0.f, -INFINITY};
  f32x4_t oacc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) oacc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const float qk_scale = p.sm_scale * p.k_scale * kLog2e;
  const int P = p.page_size;

  if (jhi > j0) {
    const int pfirst = j0 / P, plast = (jhi - 1) / P;
    for (int wb = pfirst; wb <= plast; wb += kPageWinM) {
      const int npw = min(kPageWinM, plast - wb + 1);
      __syncthreads();  // the previous window's readers are done
      for (int i = tid; i < npw; i += 64 * kNW2) s_pages[i] = p.kv_indices[pbeg + wb + i];
      __syncthreads();
      const int ws = max(j0, wb * P), we = min(jhi, (wb + npw) * P);
      const int nk = (we - ws + kTKQ - 1) / kTKQ;
      const int wbP = wb * P;
      // tile k in stage k % 2; the load of tile k + 1 runs during the math of
      // tile k (one step per loop iteration, the stages picked at run time: the
      // loads are issued in asm, so no wait is inserted for them)
      // tile k in stage k % 2; the load of tile k + 1 runs during the math of
      // tile k (one step per loop iteration, the stages picked at run time: the
      // loads are issued in asm, so no wait is inserted for them)
      const bool paged = P % 64 == 0 && (ws - wbP) % 64 == 0;
      auto dma = [&](uint8_t* stage, int jb) __attribute__((always_inline)) {
        if (paged)
          dma_tileq<true>(p, s_pages, stage, jb, we, wbP, g, w, lane);
        else
          dma_tileq<false>(p, s_pages, stage, jb, we, wbP, g, w, lane);
      };
      dma(s_kv0, ws);
      for (int k = 0; k < nk; ++k) {
        uint8_t* cur = k & 1 ? s_kv1 : s_kv0;
        uint8_t* nxt = k & 1 ? s_kv0 : s_kv1;
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of tile k are done
        lds_barrier();                       // every wave's; the other stage's readers are done
        const int jb = ws + k * kTKQ;
        if (k + 1 < nk) dma(nxt, jb + kTKQ);
        __builtin_amdgcn_sched_barrier(0);  // the loads' addresses die before the math
        if (wave_live) mla_rows8_tile(cur, jb, lim, jb + kTKQ > wave_lim_min, qreg, qk_scale, st, oacc, lane);
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no loads in flight into the stages
      __syncthreads();
    }
  }

  // ---- epilogue: lane (row l16, group lg) holds dims 16d + 4lg + (0..3)
  const float ltot = xor32_sum(xor16_sum(st.lsum));
  if (!row_ok) return;
  const bool empty = !(ltot > 0.f);
  const float scale = empty ? 0.f : p.v_scale / ltot;
  // (the row's indices recomputed here, not kept in registers across the loop)
  int rw = row;
  asm volatile("" : "+v"(rw));
  const int64_t rid = (int64_t)(b * p.q_len + rw / p.group) * p.num_qo_heads + (int64_t)g * p.group +
                      rw % p.group;
  const int64_t wrow = wslot * p.ws_rows + rw;  // workspace row (balanced split)
#pragma unroll
  for (int d = 0; d < NDT; ++d) {
    const int dim = 16 * d + 4 * lg;
    const float x0 = oacc[d][0] * scale, x1 = oacc[d][1] * scale;
    const float x2 = oacc[d][2] * scale, x3 = oacc[d][3] * scale;
    if (to_ws) {
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.ws_o) + wrow * kDvo + dim) =
          make_uint2(pack2<BF16>(x0, x1), pack2<BF16>(x2, x3));  // bf16 partial state
    } else if (p.o_dtype == F32) {
      *reinterpret_cast<float4*>(static_cast<float*>(p.o) + c * p.o_split_stride + rid * kDvo + dim) =
          make_float4(x0, x1, x2, x3);
    } else {
      const uint2 v = p.o_dtype == F16 ? make_uint2(pack2<F16>(x0, x1), pack2<F16>(x2, x3))
                                       : make_uint2(pack2<BF16>(x0, x1), pack2<BF16>(x2, x3));
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.o) + c * p.o_split_stride + rid * kDvo + dim) = v;
    }
  }
  if (lg == 0) {
    const float lse = empty ? -INFINITY : (st.m + fast_log2(ltot)) * kLn2;
    const float mx = empty ? -INFINITY : st.true_max * kLn2;
    if (to_ws) {
      p.ws_lse[wrow] = lse;
      p.ws_mx[wrow] = mx;
    } else {
      const int64_t sidx = c * p.s_split_stride + rid;
      if (p.lse) p.lse[sidx] = lse;
      if (p.mx) p.mx[sidx] = mx;
    }
  }
}

// Workgroups as for the many-rows kernel.
__global__ __launch_bounds__(64 * kNW2, 1) void mla_rows8_kernel(AttnParams p, int nrt, int ngroups) {
  __shared__ __align__(16) uint8_t s_kv0[kStageQ];
  __shared__ __align__(16) uint8_t s_kv1[kStageQ];
  __shared__ int s_pages[kPageWinM];
  if (p.bal_blocks > 0) {
    BalCursor cur;
    if (!cur.start(p, blockIdx.x)) return;
    do {
      mla_rows8_range(p, cur.b, cur.g, cur.rt, cur.L, cur.j0(p), cur.j1(p),
                      !cur.whole(), cur.slot(p), 0, s_kv0, s_kv1, s_pages);
    } while (cur.next(p));
    return;
  }
  const int lam = blockIdx.x;
  const int xcd = lam % 8, k8 = lam / 8;
  const int rt = k8 % nrt;
  const int gi = (k8 / nrt) * 8 + xcd;
  if (gi >= ngroups) return;
  const int b = gi / (p.num_kv_heads * p.num_splits);
  const int g = (gi / p.num_splits) % p.num_kv_heads;
  const int c = gi % p.num_splits;
  int L, j0, j1;
  mla_item_range(p, b, c, L, j0, j1);
  mla_rows8_range(p, b, g, rt, L, j0, j1, false, 0, c, s_kv0, s_kv1, s_pages);
}

// ---------------------------------------------------------------------------
// Up to 16 rows per request (q_len x H <= 16): one row block is too little MFMA
// work for one wave to keep up with HBM, so the tile is shared out by dims.
// Per 32-token tile (LDS stages fed by direct loads, as above):
//   S^T = K Q^T is split over the 576 dims: waves 0..5 each take three 32-dim
//   k-steps (one 16x16x32 MFMA per k-step and 16-token block) and leave their
//   partial scores in LDS; wave 6 adds the six partials for all 16 rows x 32
//   tokens, runs the online softmax and publishes P^T and the rows' rescale
//   factors;
//   O^T += V^T P^T is split over the 512 V dims: wave w owns dims [64w, 64w+64).
// bf16 tiles are read in place from four stages, two barriers per tile; fp8
// tiles too (codes widened in registers), pipelined one tile deep over double-
// buffered partial scores and P^T with one barrier per tile (mla_narrow_range).
constexpr int kNS = kDqk / 32 / 3;  // waves that compute partial scores (6); wave kNS reduces
static_assert(kNS < kNW2, "a wave beyond the partial-score waves does the softmax");
// exchange from the reducing wave to the others
struct NarrowX {
  i16x8_t pb[64];      // P^T in the PV B-operand layout
  float alpha[16];     // rows' rescale factors of the current tile (valid when flag)
  float stat[16][3];   // final: row sum, reference max, running max
  int flag;            // some row's reference max moved in this tile
};
// LDS stages (tiles in flight + 1): as many as fit next to the score exchange
// (bf16: 4 x 36 KB; fp8: 7 x 18 KB next to the double-buffered scores and P^T)
template <bool FP8>
constexpr int kNarrowStages = FP8 ? 7 : 4;

// One (request b, KV head g) token range [j0, j1) of the narrow kernel; the
// result goes to the final O / LSE (split c_out) or to workspace slot wslot.
// Called by every thread of the workgroup.
template <bool FP8>
__device__ __forceinline__ void mla_narrow_range(const AttnParams& p, int b, int g, int L, int j0, int j1,
                                                 bool to_ws, int64_t wslot, int c, uint8_t* s_kv0,
                                                 uint8_t* s_kv1, uint8_t* s_kv2, uint8_t* s_kv3,
                                                 f32x4_t (*s_part)[2][64], NarrowX* s_x, int* s_pages) {
  constexpr int NST = kNarrowStages<FP8>;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;
  const int kb = p.broadcast ? 0 : b;
  const int pbeg = p.kv_indptr[kb];
  const int R = p.q_len * p.group;
  const int row = l16;  // every wave covers the same 16 rows
  const bool row_ok = row < R;
  int lim = j1;
  if (row_ok && p.causal) lim = min(lim, L - p.q_len + row / p.group + 1);
  if (!row_ok) lim = INT_MIN;
  int lo = row_ok ? lim : INT_MAX;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) lo = min(lo, __shfl_xor(lo, off, 64));
  const int wave_lim_min = __builtin_amdgcn_readfirstlane(lo);
  int jhi = j1;
  if (p.causal) jhi = min(j1, L - p.q_len + (R - 1) / p.group + 1);

  // Q^T operands of this wave's three k-steps (waves 0..5)
  i16x8_t qreg[3];
  {
    const int qi = row_ok ? row / p.group : 0, qh = row_ok ? row % p.group : 0;
    const int64_t qe =
        ((int64_t)(b * p.q_len + qi) * p.num_qo_heads + (int64_t)g * p.group + qh) * kDqk + 8 * lg;
#pragma unroll
    for (int u = 0; u < 3; ++u)
      qreg[u] = row_ok && w < kNS ? load_q8(p, qe + 32 * (3 * w + u)) : i16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
  }

  // softmax state: kept by the reducing wave (kNS) only
  float m = -INFINITY, lsum = 0.f, true_max = -INFINITY;
  f32x4_t oacc[4];  // dims 64w + 16d + 4lg + i, row l16
#pragma unroll
  for (int d = 0; d < 4; ++d) oacc[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const float qk_scale = p.sm_scale * p.k_scale * kLog2e;
  const int P = p.page_size;

  // One tile of a (bf16, swizzled) tile buffer kv in four parts: waves
  // 0..kNS-1 compute the partial scores (part_s) and every wave reads its V^T
  // operands (part_v); after a barrier wave kNS sums the partials, runs the
  // online softmax and publishes P^T (16-bit, in the PV B-operand layout) and
  // the rows' rescale factors (part_r); after another barrier every wave does
  // PV for its 64 dims (part_pv).
  auto part_s = [&](const uint8_t* kv) __attribute__((always_inline)) {
    if (w < kNS) {
      f32x4_t sacc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
      const int sw = mla_swz(l16);  // rows l16 and 16 + l16 share the swizzle
      uint32_t ka[3];
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        const int piece = 4 * (3 * w + u) + lg;
        ka[u] = lds_off(kv) + l16 * kKP2 + 16 * ((piece & ~7) | ((piece & 7) ^ sw));
      }
      i32x4_t kr[6];  // (k-step u, block st2) at 2u + st2
      lds_read6_b128(ka[0], ka[1], ka[2], kr);
#pragma unroll
      for (int u = 0; u < 3; ++u)
#pragma unroll
        for (int st2 = 0; st2 < 2; ++st2)
          sacc[st2] = mfma16<BF16>(__builtin_bit_cast(i16x8_t, kr[2 * u + st2]), qreg[u], sacc[st2]);
      lds_write_part(lds_off(&s_part[w][0][lane]), sacc[0], sacc[1]);
    }
  };
  // V^T operands of dims 64w + 16d: two transposed 4x16 reads each (row rr and
  // rr + 16, same swizzle), lane quad l16 % 4 = dims 4 (l16 % 4)..+3
  auto part_v = [&](const uint8_t* kv, i32x2_t (&vr)[8]) __attribute__((always_inline)) {
    const int rr = 4 * lg + (l16 >> 2);
    const int vsw = mla_swz(rr);
    const int hp = (l16 & 3) >> 1;
    uint32_t vb[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int piece = 2 * (4 * w + d) + hp;
      vb[d] = lds_off(kv) + rr * kKP2 + 16 * ((piece & ~7) | ((piece & 7) ^ vsw)) + 8 * (l16 & 1);
    }
    lds_read8_tr(vb[0], vb[1], vb[2], vb[3], vr);
  };
  auto part_r = [&](int jb, f32x4_t (*sp)[2][64], NarrowX* sx) __attribute__((always_inline)) {
    // the kNS x 2 partial blocks of this lane, all read in one round trip
    static_assert(kNS == 6, "twelve partial blocks");
    i32x4_t pr[12];
    lds_read12_b128(lds_off(&sp[0][0][lane]), pr);
    f32x4_t ssum[2] = {__builtin_bit_cast(f32x4_t, pr[0]), __builtin_bit_cast(f32x4_t, pr[1])};
#pragma unroll
    for (int v = 1; v < kNS; ++v) {
      ssum[0] += __builtin_bit_cast(f32x4_t, pr[2 * v]);
      ssum[1] += __builtin_bit_cast(f32x4_t, pr[2 * v + 1]);
    }
    // lane holds row l16, tokens jb + 16st + 4lg + i; the mask only on boundary tiles
    if (jb + kTK2 > wave_lim_min) {
#pragma unroll
      for (int st2 = 0; st2 < 2; ++st2)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (jb + 16 * st2 + 4 * lg + i >= lim) ssum[st2][i] = -INFINITY;
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int st2 = 0; st2 < 2; ++st2)
#pragma unroll
      for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, ssum[st2][i]);
    tmax = xor32_max(xor16_max(tmax)) * qk_scale;
    true_max = fmaxf(true_max, tmax);
    const bool grow = tmax > m + 8.f;
    const bool any = __ballot(grow) != 0;
    if (any) {
      const float mnew = grow ? tmax : m;
      const float alpha = fast_exp2((m == -INFINITY ? -INFINITY : m) - (mnew == -INFINITY ? 0.f : mnew));
      const float a = grow ? alpha : 1.f;
      lsum *= a;
      m = mnew;
      if (lg == 0) sx->alpha[l16] = a;
    }
    const float nmref = -(m == -INFINITY ? 0.f : m);
    float e[8];
#pragma unroll
    for (int st2 = 0; st2 < 2; ++st2)
#pragma unroll
      for (int i = 0; i < 4; ++i) e[4 * st2 + i] = fast_exp2(fmaf(ssum[st2][i], qk_scale, nmref));
    const uint4 bits = make_uint4(pack2<BF16>(e[0], e[1]), pack2<BF16>(e[2], e[3]),
                                  pack2<BF16>(e[4], e[5]), pack2<BF16>(e[6], e[7]));
    lsum = sum2<BF16>(bits.x, sum2<BF16>(bits.y, sum2<BF16>(bits.z, sum2<BF16>(bits.w, lsum))));
    sx->pb[lane] = as_i16x8(bits);
    if (lane == 0) lds_write_b32(lds_off(&sx->flag), any);
  };
  auto part_pv = [&](const i32x2_t (&vr)[8]) __attribute__((always_inline)) {
    // P^T, the row's rescale factor (meaningful when the flag is set) and the flag
    i32x4_t pbv;
    float a;
    int flag;
    lds_read_pv(lds_off(&s_x->pb[lane]), lds_off(&s_x->alpha[l16]), lds_off(&s_x->flag), pbv, a, flag);
    if (__builtin_amdgcn_readfirstlane(flag)) {
#pragma unroll
      for (int d = 0; d < 4; ++d) oacc[d] *= a;
    }
    const i16x8_t pb = __builtin_bit_cast(i16x8_t, pbv);
    // O^T += V^T P^T for dims 64w + 16d
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const i32x4_t v4 = {vr[2 * d].x, vr[2 * d].y, vr[2 * d + 1].x, vr[2 * d + 1].y};
      oacc[d] = mfma16<BF16>(__builtin_bit_cast(i16x8_t, v4), pb, oacc[d]);
    }
  };

  // fp8, read in place from the swizzled stages (see swz8): waves 0..kNS-1 read
  // their K operands with 8-byte reads and widen them in registers (part_s8);
  // every wave reads its V^T operands with transposed 8-bit reads whose rows
  // follow P^T's token order (part_v8)
  constexpr int kPitch8 = kPieces8 * 16;  // 576-byte fp8 rows
  auto part_s8 = [&](const uint8_t* kv, f32x4_t (*sp)[2][64]) __attribute__((always_inline)) {
    f32x4_t sacc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
    const uint32_t base = lds_off(kv) + l16 * kPitch8 + 8 * (lg & 1);  // rows l16 and 16 + l16
    const int sw = swz8(l16);                                           // (same swizzle)
    uint32_t ka[3];
#pragma unroll
    for (int u = 0; u < 3; ++u) ka[u] = base + 16 * ((2 * (3 * w + u) + (lg >> 1)) ^ sw);
    i32x2_t kr[6];  // (k-step u, block st2) at 2u + st2
    lds_read6_b64(ka[0], ka[1], ka[2], kr);
#pragma unroll
    for (int u = 0; u < 3; ++u)
#pragma unroll
      for (int st2 = 0; st2 < 2; ++st2)
        sacc[st2] = mfma16<BF16>(fp8x8_to_bf16(kr[2 * u + st2]), qreg[u], sacc[st2]);
    lds_write_part(lds_off(&sp[w][0][lane]), sacc[0], sacc[1]);
  };
  auto part_v8 = [&](const uint8_t* kv, i16x8_t (&va)[4]) __attribute__((always_inline)) {
    // lane group q holds P^T's k = 8q + j, i.e. tokens 4q + j (j < 4) and 12 + 4q + j
    const int q = lane >> 4, j = (lane & 15) >> 1, h = lane & 1;
    const int trow = j < 4 ? 4 * q + j : 12 + 4 * q + j;
    const int sw = swz8(trow);
    const uint32_t rb = lds_off(kv) + trow * kPitch8 + 8 * h;
    i32x2_t vr[4];
    lds_read4_tr8(rb + 16 * ((4 * w + 0) ^ sw), rb + 16 * ((4 * w + 1) ^ sw), rb + 16 * ((4 * w + 2) ^ sw),
                  rb + 16 * ((4 * w + 3) ^ sw), vr);
#pragma unroll
    for (int d = 0; d < 4; ++d) va[d] = fp8x8_to_bf16(vr[d]);
  };
  // PV of one tile from stage kv (wave w: dims 64w..64w+63)
  auto part_pv8 = [&](const uint8_t* kv, const NarrowX* sx) __attribute__((always_inline)) {
    i16x8_t va[4];
    part_v8(kv, va);
    i32x4_t pbv;
    float a;
    int flag;
    lds_read_pv(lds_off(&sx->pb[lane]), lds_off(&sx->alpha[l16]), lds_off(&sx->flag), pbv, a, flag);
    if (__builtin_amdgcn_readfirstlane(flag)) {
#pragma unroll
      for (int d = 0; d < 4; ++d) oacc[d] *= a;
    }
    const i16x8_t pb = __builtin_bit_cast(i16x8_t, pbv);
#pragma unroll
    for (int d = 0; d < 4; ++d) oacc[d] = mfma16<BF16>(va[d], pb, oacc[d]);
  };

  // tiles never straddle a page when the page size is a multiple of the tile
  // (range starts are multiples of the tile or of the page)
  const bool page_tiles = P % kTK2 == 0 && j0 % kTK2 == 0;
  PageLanes<FP8, FP8 ? 1 : 0> plane;
  if (page_tiles) plane.init(p, g, w, lane);
  if (jhi > j0) {
    const int pfirst = j0 / P, plast = (jhi - 1) / P;
    for (int wb = pfirst; wb <= plast; wb += kPageWinM) {
      const int npw = min(kPageWinM, plast - wb + 1);
      __syncthreads();  // the previous window's readers are done
      for (int i = tid; i < npw; i += 64 * kNW2) s_pages[i] = p.kv_indices[pbeg + wb + i];
      __syncthreads();
      const int ws = max(j0, wb * P), we = min(jhi, (wb + npw) * P);
      const int nk = (we - ws + kTK2 - 1) / kTK2;
      // tile k in stage k % NST; tiles k+1 .. k+NST-1 in flight during tile k
      // (a wave issues at least kMinDma direct loads per tile, so vmcnt(kWait)
      // after issuing tile k+NST-2 means tile k has landed)
      constexpr int kMinDma = (FP8 ? kDma8 : kDma) / kNW2;  // loads per wave per tile
      constexpr int kWait = (NST - 2) * kMinDma;
      static_assert(kWait < 64, "vmcnt field");
      constexpr int kWaitImm = (kWait & 0xF) | ((kWait >> 4) << 14) | 0x70 | 0xF00;
      const int wbP = wb * P;
      auto tile_at = [&](int k) { return ws + min(k, nk - 1) * kTK2; };
      // page-aligned tiles: lane i of ptab holds the page id of tile 64 (k / 64) + i,
      // so the loads of tile k take its page with one uniform lane read instead of
      // an LDS round trip per tile (tiles are issued in order 0, 1, 2, ...)
      int ptab = 0;
      auto dma = [&](uint8_t* stage, int k) __attribute__((always_inline)) {
        const int jb = tile_at(k);
        if (page_tiles) {
          if ((k & 63) == 0) ptab = s_pages[div_by_magic((uint32_t)(tile_at(k + lane) - wbP), p.page_magic)];
          const int page = __builtin_amdgcn_readlane(ptab, k & 63);
          if constexpr (FP8)
            dma_page_fp8s(p, page, stage, jb, we, wbP, plane, w);
          else
            dma_page_bf16(p, page, stage, jb, we, wbP, plane, w);
        } else {
          if constexpr (FP8)
            dma_tile8<1>(p, s_pages, stage, jb, we, wbP, g, w, lane);
          else
            dma_tile(p, s_pages, stage, jb, we, wbP, g, w, lane);
        }
      };
      if constexpr (!FP8) {
        dma(s_kv0, 0);
        dma(s_kv1, 1);
        dma(s_kv2, 2);
      }
      // Two barriers per tile.  Step K: scores and V operands of tile K | barrier |
      // loads of tile K+NST-1 into the stage of tile K-1 (read before the barrier),
      // softmax of tile K, wait for this wave's loads of tile K+1 | barrier (so
      // P^T and the whole of tile K+1 are visible) | PV of tile K.
      if constexpr (!FP8) {
        // tile K read in place from its stage
        __builtin_amdgcn_s_waitcnt(kWaitImm);  // tile 0's direct loads are done
        lds_barrier();
#define PA_MLA_NSTEP(K, CUR, NEXT)                                                            \
  {                                                                                         \
    part_s(CUR);                                                                            \
    i32x2_t vr[8];                                                                          \
    part_v(CUR, vr);                                                                        \
    lds_barrier();                                                                           \
    dma(NEXT, (K) + NST - 1);                                                               \
    if (w == kNS) part_r(ws + (K) * kTK2, s_part, s_x);                                     \
    __builtin_amdgcn_s_waitcnt(kWaitImm); /* tile K+1's direct loads are done */            \
    lds_barrier();                                                                           \
    part_pv(vr);                                                                            \
  }
        static_assert(NST == 4, "bf16 stage rotation");
        for (int k = 0; k < nk; k += 4) {
          PA_MLA_NSTEP(k, s_kv0, s_kv3);
          if (k + 1 >= nk) break;
          PA_MLA_NSTEP(k + 1, s_kv1, s_kv0);
          if (k + 2 >= nk) break;
          PA_MLA_NSTEP(k + 2, s_kv2, s_kv1);
          if (k + 3 >= nk) break;
          PA_MLA_NSTEP(k + 3, s_kv3, s_kv2);
        }
#undef PA_MLA_NSTEP
      } else {
        // fp8 read in place, one barrier per tile: step K computes the partial
        // scores of tile K+1 (waves 0..kNS-1) while wave kNS runs the softmax of
        // tile K, then every wave does the PV of tile K-1.  Partial scores and P^T
        // are double-buffered; stage t % NST holds tile t, tiles K+3..K+NST-2 are
        // in flight at the end of step K.
        static_assert(NST == 7, "fp8 stages");
        constexpr int kWait3 = (NST - 3) * kMinDma, kWait4 = (NST - 4) * kMinDma;
        static_assert(kWait3 < 16, "vmcnt field");
        constexpr int kWaitImm3 = kWait3 | 0x70 | 0xF00, kWaitImm4 = kWait4 | 0x70 | 0xF00;
        auto stage = [&](int t) { return s_kv0 + kStage8 * (t % NST); };
#pragma unroll
        for (int t = 0; t < NST - 2; ++t) dma(stage(t), t);
        __builtin_amdgcn_s_waitcnt(kWaitImm3);  // tile 0 has landed
        lds_barrier();
        if (w < kNS) part_s8(stage(0), s_part);
        __builtin_amdgcn_s_waitcnt(kWaitImm4);  // tile 1 has landed
        lds_barrier();
        for (int k = 0; k < nk; ++k) {
          dma(stage(k + NST - 2), k + NST - 2);  // the stage of tile k-2, read before the last barrier
          if (w < kNS)
            part_s8(stage(k + 1), s_part + kNS * ((k + 1) & 1));  // past the last tile: unused
          else if (w == kNS)
            part_r(ws + k * kTK2, s_part + kNS * (k & 1), s_x + (k & 1));
          if (k > 0) part_pv8(stage(k - 1), s_x + ((k - 1) & 1));
          __builtin_amdgcn_s_waitcnt(kWaitImm4);  // tile k+2 has landed
          lds_barrier();
        }
        part_pv8(stage(nk - 1), s_x + ((nk - 1) & 1));
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no loads in flight into the stages
      __syncthreads();
    }
  }

  // ---- epilogue: the reducing wave publishes the rows' sums and maxima; wave w
  // writes dims [64w, 64w+64) of the R rows, the reducing wave the stats
  if (w == kNS) {
    const float lt = xor32_sum(xor16_sum(lsum));
    if (lg == 0) {
      s_x->stat[l16][0] = lt;
      s_x->stat[l16][1] = m;
      s_x->stat[l16][2] = true_max;
    }
  }
  __syncthreads();
  const float ltot = s_x->stat[l16][0];
  const float mref = s_x->stat[l16][1], tmx = s_x->stat[l16][2];
  __syncthreads();  // the stats are read before the next range overwrites them
  if (!row_ok) return;
  const bool empty = !(ltot > 0.f);
  const float scale = empty ? 0.f : p.v_scale / ltot;
  const int64_t rid = (int64_t)(b * p.q_len + row / p.group) * p.num_qo_heads + (int64_t)g * p.group +
                      row % p.group;
  const int64_t wrow = wslot * p.ws_rows + row;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int dim = 64 * w + 16 * d + 4 * lg;
    const float x0 = oacc[d][0] * scale, x1 = oacc[d][1] * scale;
    const float x2 = oacc[d][2] * scale, x3 = oacc[d][3] * scale;
    if (to_ws) {
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.ws_o) + wrow * kDvo + dim) =
          make_uint2(pack2<BF16>(x0, x1), pack2<BF16>(x2, x3));  // bf16 partial state
    } else if (p.o_dtype == F32) {
      *reinterpret_cast<float4*>(static_cast<float*>(p.o) + c * p.o_split_stride + rid * kDvo + dim) =
          make_float4(x0, x1, x2, x3);
    } else {
      const uint2 v = p.o_dtype == F16 ? make_uint2(pack2<F16>(x0, x1), pack2<F16>(x2, x3))
                                       : make_uint2(pack2<BF16>(x0, x1), pack2<BF16>(x2, x3));
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.o) + c * p.o_split_stride + rid * kDvo + dim) = v;
    }
  }
  if (w == kNS && lg == 0) {
    const float lse = empty ? -INFINITY : (mref + fast_log2(ltot)) * kLn2;
    const float mx = empty ? -INFINITY : tmx * kLn2;
    if (to_ws) {
      p.ws_lse[wrow] = lse;
      p.ws_mx[wrow] = mx;
    } else {
      const int64_t sidx = c * p.s_split_stride + rid;
      if (p.lse) p.lse[sidx] = lse;
      if (p.mx) p.mx[sidx] = mx;
    }
  }
}

// Workgroups: (request, KV head, explicit split) items, or, under the
// balanced split, equal shares of the (request, KV head, 32-token unit) sequence.
template <bool FP8>
__global__ __launch_bounds__(64 * kNW2, 1) void mla_narrow_kernel(AttnParams p, int ngroups) {
  // bf16: four stages; fp8: the NST stages contiguous from s_kv0, and the partial
  // scores and the P^T exchange double-buffered
  constexpr int NST = kNarrowStages<FP8>;
  static_assert(FP8 || NST == 4, "bf16 stages");
  __shared__ __align__(16) uint8_t s_kv0[FP8 ? NST * kStage8 : kStage2];
  __shared__ __align__(16) uint8_t s_kv1[FP8 ? 16 : kStage2];
  __shared__ __align__(16) uint8_t s_kv2[FP8 ? 16 : kStage2];
  __shared__ __align__(16) uint8_t s_kv3[FP8 ? 16 : kStage2];
  __shared__ __align__(16) f32x4_t s_part[(FP8 ? 2 : 1) * kNS][2][64];  // partial scores
  __shared__ __align__(16) NarrowX s_xb[FP8 ? 2 : 1];
  NarrowX* const s_x = s_xb;
  __shared__ int s_pages[kPageWinM];
  if (p.bal_blocks > 0) {
    BalCursor cur;
    if (!cur.start(p, blockIdx.x)) return;
    do {
      mla_narrow_range<FP8>(p, cur.b, cur.g, cur.L, cur.j0(p), cur.j1(p), !cur.whole(), cur.slot(p), 0,
                            s_kv0, s_kv1, s_kv2, s_kv3, s_part, s_x, s_pages);
    } while (cur.next(p));
    return;
  }
  const int gi = blockIdx.x;
  if (gi >= ngroups) return;
  const int b = gi / (p.num_kv_heads * p.num_splits);
  const int g = (gi / p.num_splits) % p.num_kv_heads;
  const int c = gi % p.num_splits;
  int L, j0, j1;
  mla_item_range(p, b, c, L, j0, j1);
  mla_narrow_range<FP8>(p, b, g, L, j0, j1, false, 0,
                        c, s_kv0, s_kv1, s_kv2, s_kv3, s_part, s_x, s_pages);
}

// ---------------------------------------------------------------------------
// 17..64 rows per request: NRB = 2 or 4 row blocks of 16 rows.  Wave w takes
// row block w % NRB and k-step slice w / NRB of the 576-dim contraction
// (KS = 8 / NRB slices), so every wave computes partial scores; waves
// 0..NRB-1 then each sum one row block's partials and run its online softmax;
// every wave does PV for its 64 V dims over all row blocks.  The KV stream is
// the narrow kernel's (direct loads, bare barriers, stage reads in asm); three
// bf16 stages fit next to the 16 KB of partial scores, and fp8 is read in place
// from six stages next to double-buffered partial scores and P^T.
template <int NRB>
struct MidX {
  i16x8_t pb[NRB][64];    // P^T of each row block in the PV B-operand layout
  float alpha[NRB][16];   // rescale factors of the current tile (valid when flag)
  float stat[NRB][16][3]; // final: row sum, reference max, running max
  alignas(16) int flag[NRB];
};
template <bool FP8>
constexpr int kMidStages = FP8 ? 6 : 3;

template <bool FP8, int NRB>
__device__ __forceinline__ void mla_mid_range(const AttnParams& p, int b, int g, int L, int j0, int j1,
                                              bool to_ws, int64_t wslot, int c, uint8_t* s_kv0,
                                              uint8_t* s_kv1, uint8_t* s_kv2,
                                              f32x4_t (*s_part)[2][64], MidX<NRB>* s_x, int* s_pages) {
  constexpr int NST = kMidStages<FP8>;
  constexpr int KS = kNW2 / NRB;                  // k-step slices per row block
  constexpr int KK = kDqk / 32;                   // 18 k-steps
  constexpr int KMAX = (KK + KS - 1) / KS;        // k-steps of the largest slice
  static_assert(KS * NRB == kNW2 && KMAX >= 3, "wave split");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;
  const int rbw = w % NRB, ksw = w / NRB;
  const int k0 = ksw * KK / KS, nks = (ksw + 1) * KK / KS - k0;  // this wave's k-steps
  const int kb = p.broadcast ? 0 : b;
  const int pbeg = p.kv_indptr[kb];
  const int R = p.q_len * p.group;
  // row of this lane in its wave's row block (scores, softmax)
  const int row = 16 * rbw + l16;
  const bool row_ok = row < R;
  int lim = j1;
  if (row_ok && p.causal) lim = min(lim, L - p.q_len + row / p.group + 1);
  if (!row_ok) lim = INT_MIN;
  int lo = row_ok ? lim : INT_MAX;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) lo = min(lo, __shfl_xor(lo, off, 64));
  const int wave_lim_min = __builtin_amdgcn_readfirstlane(lo);
  int jhi = j1;
  if (p.causal) jhi = min(j1, L - p.q_len + (R - 1) / p.group + 1);

  // Q^T operands of this wave's k-steps k0 .. k0 + nks - 1
  i16x8_t qreg[KMAX];
  {
    const int qi = row_ok ? row / p.group : 0, qh = row_ok ? row % p.group : 0;
    const int64_t qe =
        ((int64_t)(b * p.q_len + qi) * p.num_qo_heads + (int64_t)g * p.group + qh) * kDqk + 8 * lg;
#pragma unroll
    for (int u = 0; u < KMAX; ++u)
      qreg[u] = row_ok && u < nks ? load_q8(p, qe + 32 * (k0 + u)) : i16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
  }

  // softmax state of row block w, kept by wave w < NRB
  float m = -INFINITY, lsum = 0.f, true_max = -INFINITY;
  f32x4_t oacc[NRB][4];  // row block rb: dims 64w + 16d + 4lg + i, row 16 rb + l16
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int d = 0; d < 4; ++d) oacc[rb][d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const float qk_scale = p.sm_scale * p.k_scale * kLog2e;
  const int P = p.page_size;

  auto part_s = [&](const uint8_t* kv) __attribute__((always_inline)) {
    f32x4_t sacc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
    const int sw = mla_swz(l16);
    const uint32_t kbase = lds_off(kv) + l16 * kKP2;
    auto kaddr = [&](int kk) {
      const int piece = 4 * kk + lg;
      return kbase + 16 * ((piece & ~7) | ((piece & 7) ^ sw));
    };
    // whole groups of three k-steps, then a rest of one or two
#pragma unroll
    for (int j = 0; j + 3 <= KMAX; j += 3) {
      if (j + 3 <= nks) {
        i32x4_t kr[6];
        lds_read6_b128(kaddr(k0 + j), kaddr(k0 + j + 1), kaddr(k0 + j + 2), kr);
#pragma unroll
        for (int u = 0; u < 3; ++u)
#pragma unroll
          for (int st2 = 0; st2 < 2; ++st2)
            sacc[st2] = mfma16<BF16>(__builtin_bit_cast(i16x8_t, kr[2 * u + st2]), qreg[j + u], sacc[st2]);
      }
    }
    if constexpr (KMAX % 3 != 0) {
      constexpr int j = KMAX / 3 * 3;
      if (nks - j == 2) {
        i32x4_t kr[4];
        lds_read4_b128(kaddr(k0 + j), kaddr(k0 + j + 1), kr);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int st2 = 0; st2 < 2; ++st2)
            sacc[st2] = mfma16<BF16>(__builtin_bit_cast(i16x8_t, kr[2 * u + st2]), qreg[j + u], sacc[st2]);
      } else if (nks - j == 1) {
        i32x4_t kr[2];
        lds_read2x_b128(kaddr(k0 + j), kr);
#pragma unroll
        for (int st2 = 0; st2 < 2; ++st2)
          sacc[st2] = mfma16<BF16>(__builtin_bit_cast(i16x8_t, kr[st2]), qreg[j], sacc[st2]);
      }
    }
    lds_write_part(lds_off(&s_part[w][0][lane]), sacc[0], sacc[1]);
  };
  auto part_v = [&](const uint8_t* kv, i32x2_t (&vr)[8]) __attribute__((always_inline)) {
    const int rr = 4 * lg + (l16 >> 2);
    const int vsw = mla_swz(rr);
    const int hp = (l16 & 3) >> 1;
    uint32_t vb[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int piece = 2 * (4 * w + d) + hp;
      vb[d] = lds_off(kv) + rr * kKP2 + 16 * ((piece & ~7) | ((piece & 7) ^ vsw)) + 8 * (l16 & 1);
    }
    lds_read8_tr(vb[0], vb[1], vb[2], vb[3], vr);
  };
  // wave w < NRB: row block w
  auto part_r = [&](int jb, f32x4_t (*sp)[2][64], MidX<NRB>* sx) __attribute__((always_inline)) {
    // sp[w + NRB k][st][lane] for the KS slices k (2 KB per wave)
    f32x4_t pr[KS][2];
    lds_read_parts<KS, 2048 * NRB>(lds_off(&sp[w][0][lane]), pr);
    f32x4_t ssum[2] = {pr[0][0], pr[0][1]};
#pragma unroll
    for (int k = 1; k < KS; ++k) {
      ssum[0] += pr[k][0];
      ssum[1] += pr[k][1];
    }
    if (jb + kTK2 > wave_lim_min) {
#pragma unroll
      for (int st2 = 0; st2 < 2; ++st2)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (jb + 16 * st2 + 4 * lg + i >= lim) ssum[st2][i] = -INFINITY;
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int st2 = 0; st2 < 2; ++st2)
#pragma unroll
      for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, ssum[st2][i]);
    tmax = xor32_max(xor16_max(tmax)) * qk_scale;
    true_max = fmaxf(true_max, tmax);
    const bool grow = tmax > m + 8.f;
    const bool any = __ballot(grow) != 0;
    if (any) {
      const float mnew = grow ? tmax : m;
      const float alpha = fast_exp2((m == -INFINITY ? -INFINITY : m) - (mnew == -INFINITY ? 0.f : mnew));
      const float a = grow ? alpha : 1.f;
      lsum *= a;
      m = mnew;
      if (lg == 0) sx->alpha[w][l16] = a;
    }
    const float nmref = -(m == -INFINITY ? 0.f : m);
    float e[8];
#pragma unroll
    for (int st2 = 0; st2 < 2; ++st2)
#pragma unroll
      for (int i = 0; i < 4; ++i) e[4 * st2 + i] = fast_exp2(fmaf(ssum[st2][i], qk_scale, nmref));
    const uint4 bits = make_uint4(pack2<BF16>(e[0], e[1]), pack2<BF16>(e[2], e[3]),
                                  pack2<BF16>(e[4], e[5]), pack2<BF16>(e[6], e[7]));
    lsum = sum2<BF16>(bits.x, sum2<BF16>(bits.y, sum2<BF16>(bits.z, sum2<BF16>(bits.w, lsum))));
    sx->pb[w][lane] = as_i16x8(bits);
    if (lane == 0) lds_write_b32(lds_off(&sx->flag[w]), any);
  };
  auto part_pv = [&](const i32x2_t (&vr)[8]) __attribute__((always_inline)) {
    // every row block's P^T, rescale factor and flag in one LDS round trip
    static_assert(sizeof(s_x->pb[0]) == 1024 && sizeof(s_x->alpha[0]) == 64, "exchange layout");
    i32x4_t pbs[NRB];
    float al[NRB];
    int fl[NRB];
    lds_read_pv_blocks<NRB>(lds_off(&s_x->pb[0][lane]), lds_off(&s_x->alpha[0][l16]), lds_off(&s_x->flag[0]), pbs,
                            al, fl);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      if (__builtin_amdgcn_readfirstlane(fl[rb])) {
#pragma unroll
        for (int d = 0; d < 4; ++d) oacc[rb][d] *= al[rb];
      }
      const i16x8_t pb = __builtin_bit_cast(i16x8_t, pbs[rb]);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const i32x4_t v4 = {vr[2 * d].x, vr[2 * d].y, vr[2 * d + 1].x, vr[2 * d + 1].y};
        oacc[rb][d] = mfma16<BF16>(__builtin_bit_cast(i16x8_t, v4), pb, oacc[rb][d]);
      }
    }
  };

  // fp8, read in place from the swizzled stages (as in the narrow kernel)
  constexpr int kPitch8 = kPieces8 * 16;
  auto part_s8 = [&](const uint8_t* kv, f32x4_t (*sp)[2][64]) __attribute__((always_inline)) {
    f32x4_t sacc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
    const uint32_t base = lds_off(kv) + l16 * kPitch8 + 8 * (lg & 1);  // rows l16 and 16 + l16
    const int sw = swz8(l16);
    auto kaddr = [&](int kk) { return base + 16 * ((2 * kk + (lg >> 1)) ^ sw); };
#pragma unroll
    for (int j = 0; j + 3 <= KMAX; j += 3) {
      if (j + 3 <= nks) {
        i32x2_t kr[6];
        lds_read6_b64(kaddr(k0 + j), kaddr(k0 + j + 1), kaddr(k0 + j + 2), kr);
#pragma unroll
        for (int u = 0; u < 3; ++u)
#pragma unroll
          for (int st2 = 0; st2 < 2; ++st2)
            sacc[st2] = mfma16<BF16>(fp8x8_to_bf16(kr[2 * u + st2]), qreg[j + u], sacc[st2]);
      }
    }
    if constexpr (KMAX % 3 != 0) {
      constexpr int j = KMAX / 3 * 3;
      if (nks - j == 2) {
        i32x2_t kr[4];
        lds_read4_b64(kaddr(k0 + j), kaddr(k0 + j + 1), kr);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int st2 = 0; st2 < 2; ++st2)
            sacc[st2] = mfma16<BF16>(fp8x8_to_bf16(kr[2 * u + st2]), qreg[j + u], sacc[st2]);
      } else if (nks - j == 1) {
        i32x2_t kr[2];
        lds_read2_b64(kaddr(k0 + j), kr);
#pragma unroll
        for (int st2 = 0; st2 < 2; ++st2)
          sacc[st2] = mfma16<BF16>(fp8x8_to_bf16(kr[st2]), qreg[j], sacc[st2]);
      }
    }
    lds_write_part(lds_off(&sp[w][0][lane]), sacc[0], sacc[1]);
  };
  auto part_v8 = [&](const uint8_t* kv, i16x8_t (&va)[4]) __attribute__((always_inline)) {
    // lane group q holds P^T's k = 8q + j, i.e. tokens 4q + j (j < 4) and 12 + 4q + j
    const int q = lane >> 4, j = (lane & 15) >> 1, h = lane & 1;
    const int trow = j < 4 ? 4 * q + j : 12 + 4 * q + j;
    const int sw = swz8(trow);
    const uint32_t rb = lds_off(kv) + trow * kPitch8 + 8 * h;
    i32x2_t vr[4];
    lds_read4_tr8(rb + 16 * ((4 * w + 0) ^ sw), rb + 16 * ((4 * w + 1) ^ sw), rb + 16 * ((4 * w + 2) ^ sw),
                  rb + 16 * ((4 * w + 3) ^ sw), vr);
#pragma unroll
    for (int d = 0; d < 4; ++d) va[d] = fp8x8_to_bf16(vr[d]);
  };
  auto part_pv8 = [&](const uint8_t* kv, MidX<NRB>* sx) __attribute__((always_inline)) {
    i16x8_t va[4];
    part_v8(kv, va);
    i32x4_t pbs[NRB];
    float al[NRB];
    int fl[NRB];
    lds_read_pv_blocks<NRB>(lds_off(&sx->pb[0][lane]), lds_off(&sx->alpha[0][l16]), lds_off(&sx->flag[0]), pbs,
                            al, fl);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      if (__builtin_amdgcn_readfirstlane(fl[rb])) {
#pragma unroll
        for (int d = 0; d < 4; ++d) oacc[rb][d] *= al[rb];
      }
      const i16x8_t pb = __builtin_bit_cast(i16x8_t, pbs[rb]);
#pragma unroll
      for (int d = 0; d < 4; ++d) oacc[rb][d] = mfma16<BF16>(va[d], pb, oacc[rb][d]);
    }
  };

  const bool page_tiles = P % kTK2 == 0 && j0 % kTK2 == 0;
  PageLanes<FP8, FP8 ? 1 : 0> plane;
  if (page_tiles) plane.init(p, g, w, lane);
  if (jhi > j0) {
    const int pfirst = j0 / P, plast = (jhi - 1) / P;
    for (int wb = pfirst; wb <= plast; wb += kPageWinM) {
      const int npw = min(kPageWinM, plast - wb + 1);
      __syncthreads();  // the previous window's readers are done
      for (int i = tid; i < npw; i += 64 * kNW2) s_pages[i] = p.kv_indices[pbeg + wb + i];
      __syncthreads();
      const int ws = max(j0, wb * P), we = min(jhi, (wb + npw) * P);
      const int nk = (we - ws + kTK2 - 1) / kTK2;
      // tile k in stage k % NST; a wave issues at least kMinDma direct loads per
      // tile, so vmcnt(kWait) leaves at most NST - 2 tiles in flight
      constexpr int kMinDma = (FP8 ? kDma8 : kDma) / kNW2;
      constexpr int kWait = (NST - 2) * kMinDma;
      static_assert(kWait < 64, "vmcnt field");
      constexpr int kWaitImm = (kWait & 0xF) | ((kWait >> 4) << 14) | 0x70 | 0xF00;
      const int wbP = wb * P;
      auto tile_at = [&](int k) { return ws + min(k, nk - 1) * kTK2; };
      // page-aligned tiles: lane i of ptab holds the page id of tile 64 (k / 64) + i,
      // so the loads of tile k take its page with one uniform lane read instead of
      // an LDS round trip per tile (tiles are issued in order 0, 1, 2, ...)
      int ptab = 0;
      auto dma = [&](uint8_t* stage, int k) __attribute__((always_inline)) {
        const int jb = tile_at(k);
        if (page_tiles) {
          if ((k & 63) == 0) ptab = s_pages[div_by_magic((uint32_t)(tile_at(k + lane) - wbP), p.page_magic)];
          const int page = __builtin_amdgcn_readlane(ptab, k & 63);
          if constexpr (FP8)
            dma_page_fp8s(p, page, stage, jb, we, wbP, plane, w);
          else
            dma_page_bf16(p, page, stage, jb, we, wbP, plane, w);
        } else {
          if constexpr (FP8)
            dma_tile8<1>(p, s_pages, stage, jb, we, wbP, g, w, lane);
          else
            dma_tile(p, s_pages, stage, jb, we, wbP, g, w, lane);
        }
      };
      if constexpr (!FP8) {
        dma(s_kv0, 0);
        dma(s_kv1, 1);
#define PA_MLA_MSTEP(K, CUR, NEXT)                                                            \
  {                                                                                         \
    __builtin_amdgcn_s_waitcnt(kWaitImm); /* tile K's direct loads are done */              \
    lds_barrier();                                                                           \
    dma(NEXT, (K) + NST - 1);                                                               \
    part_s(CUR);                                                                            \
    i32x2_t vr[8];                                                                          \
    part_v(CUR, vr);                                                                        \
    lds_barrier();                                                                           \
    if (w < NRB) part_r(ws + (K) * kTK2, s_part, s_x);                                      \
    lds_barrier();                                                                           \
    part_pv(vr);                                                                            \
  }
        static_assert(NST == 3, "bf16 stage rotation");
        for (int k = 0; k < nk; k += 3) {
          PA_MLA_MSTEP(k, s_kv0, s_kv2);
          if (k + 1 >= nk) break;
          PA_MLA_MSTEP(k + 1, s_kv1, s_kv0);
          if (k + 2 >= nk) break;
          PA_MLA_MSTEP(k + 2, s_kv2, s_kv1);
        }
#undef PA_MLA_MSTEP
      } else {
        // fp8 read in place, one barrier per tile (as in the narrow kernel): step K
        // computes the partial scores of tile K+1 on every wave, the softmax of tile
        // K on waves 0..NRB-1 and the PV of tile K-1; partial scores and P^T are
        // double-buffered, stage t % NST holds tile t
        static_assert(NST == 6, "fp8 stages");
        constexpr int kWait3 = (NST - 3) * kMinDma, kWait4 = (NST - 4) * kMinDma;
        static_assert(kWait3 < 16, "vmcnt field");
        constexpr int kWaitImm3 = kWait3 | 0x70 | 0xF00, kWaitImm4 = kWait4 | 0x70 | 0xF00;
        auto stage = [&](int t) { return s_kv0 + kStage8 * (t % NST); };
#pragma unroll
        for (int t = 0; t < NST - 2; ++t) dma(stage(t), t);
        __builtin_amdgcn_s_waitcnt(kWaitImm3);  // tile 0 has landed
        lds_barrier();
        part_s8(stage(0), s_part);
        __builtin_amdgcn_s_waitcnt(kWaitImm4);  // tile 1 has landed
        lds_barrier();
        for (int k = 0; k < nk; ++k) {
          dma(stage(k + NST - 2), k + NST - 2);  // the stage of tile k-2, read before the last barrier
          part_s8(stage(k + 1), s_part + kNW2 * ((k + 1) & 1));  // past the last tile: unused
          if (w < NRB) part_r(ws + k * kTK2, s_part + kNW2 * (k & 1), s_x + (k & 1));
          if (k > 0) part_pv8(stage(k - 1), s_x + ((k - 1) & 1));
          __builtin_amdgcn_s_waitcnt(kWaitImm4);  // tile k+2 has landed
          lds_barrier();
        }
        part_pv8(stage(nk - 1), s_x + ((nk - 1) & 1));
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no loads in flight into the stages
      __syncthreads();
    }
  }

  // ---- epilogue: waves 0..NRB-1 publish their row block's sums and maxima;
  // wave w writes dims [64w, 64w+64) of every row
  if (w < NRB) {
    const float lt = xor32_sum(xor16_sum(lsum));
    if (lg == 0) {
      s_x->stat[w][l16][0] = lt;
      s_x->stat[w][l16][1] = m;
      s_x->stat[w][l16][2] = true_max;
    }
  }
  __syncthreads();
  float ltot[NRB], mref[NRB], tmx[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    ltot[rb] = s_x->stat[rb][l16][0];
    mref[rb] = s_x->stat[rb][l16][1];
    tmx[rb] = s_x->stat[rb][l16][2];
  }
  __syncthreads();  // the stats are read before the next range overwrites them
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int orow = 16 * rb + l16;
    if (orow >= R) continue;
    const bool empty = !(ltot[rb] > 0.f);
    const float scale = empty ? 0.f : p.v_scale / ltot[rb];
    const int64_t rid = (int64_t)(b * p.q_len + orow / p.group) * p.num_qo_heads + (int64_t)g * p.group +
                        orow % p.group;
    const int64_t wrow = wslot * p.ws_rows + orow;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int dim = 64 * w + 16 * d + 4 * lg;
      const float x0 = oacc[rb][d][0] * scale, x1 = oacc[rb][d][1] * scale;
      const float x2 = oacc[rb][d][2] * scale, x3 = oacc[rb][d][3] * scale;
      if (to_ws) {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.ws_o) + wrow * kDvo + dim) =
            make_uint2(pack2<BF16>(x0, x1), pack2<BF16>(x2, x3));  // bf16 partial state
      } else if (p.o_dtype == F32) {
        *reinterpret_cast<float4*>(static_cast<float*>(p.o) + c * p.o_split_stride + rid * kDvo + dim) =
            make_float4(x0, x1, x2, x3);
      } else {
        const uint2 v = p.o_dtype == F16 ? make_uint2(pack2<F16>(x0, x1), pack2<F16>(x2, x3))
                                         : make_uint2(pack2<BF16>(x0, x1), pack2<BF16>(x2, x3));
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.o) + c * p.o_split_stride + rid * kDvo + dim) = v;
      }
    }
    if (w == rb && lg == 0) {
      const float lse = empty ? -INFINITY : (mref[rb] + fast_log2(ltot[rb])) * kLn2;
      const float mx = empty ? -INFINITY : tmx[rb] * kLn2;
      if (to_ws) {
        p.ws_lse[wrow] = lse;
        p.ws_mx[wrow] = mx;
      } else {
        const int64_t sidx = c * p.s_split_stride + rid;
        if (p.lse) p.lse[sidx] = lse;
        if (p.mx) p.mx[sidx] = mx;
      }
    }
  }
}

template <bool FP8, int NRB>
__global__ __launch_bounds__(64 * kNW2, 1) void mla_mid_kernel(AttnParams p, int ngroups) {
  // bf16: three stages; fp8: the NST stages contiguous from s_kv0, and the partial
  // scores and the P^T exchange double-buffered
  constexpr int NST = kMidStages<FP8>;
  static_assert(FP8 || NST == 3, "bf16 stages");
  __shared__ __align__(16) uint8_t s_kv0[FP8 ? NST * kStage8 : kStage2];
  __shared__ __align__(16) uint8_t s_kv1[FP8 ? 16 : kStage2];
  __shared__ __align__(16) uint8_t s_kv2[FP8 ? 16 : kStage2];
  __shared__ __align__(16) f32x4_t s_part[(FP8 ? 2 : 1) * kNW2][2][64];  // partial scores
  __shared__ __align__(16) MidX<NRB> s_xb[FP8 ? 2 : 1];
  MidX<NRB>* const s_x = s_xb;
  __shared__ int s_pages[kPageWinM];
  if (p.bal_blocks > 0) {
    BalCursor cur;
    if (!cur.start(p, blockIdx.x)) return;
    do {
      mla_mid_range<FP8, NRB>(p, cur.b, cur.g, cur.L, cur.j0(p), cur.j1(p), !cur.whole(), cur.slot(p), 0,
                              s_kv0, s_kv1, s_kv2, s_part, s_x, s_pages);
    } while (cur.next(p));
    return;
  }
  const int gi = blockIdx.x;
  if (gi >= ngroups) return;
  const int b = gi / (p.num_kv_heads * p.num_splits);
  const int g = (gi / p.num_splits) % p.num_kv_heads;
  const int c = gi % p.num_splits;
  int L, j0, j1;
  mla_item_range(p, b, c, L, j0, j1);
  mla_mid_range<FP8, NRB>(p, b, g, L, j0, j1, false, 0,
                          c, s_kv0, s_kv1, s_kv2, s_part, s_x, s_pages);
}

hipError_t launch_rows(const AttnParams& p, hipStream_t stream) {
  const int R = p.q_len * p.group;
  const int nrt = (R + kRT2 - 1) / kRT2;
  const int ngroups = p.batch * p.num_kv_heads * p.num_splits;
  const int blocks = p.bal_blocks > 0 ? p.bal_blocks * p.bal_co : nrt * 8 * ((ngroups + 7) / 8);
  if (p.q_dtype == FP8 && R > kRW) {
    // fp8 queries, more than 16 rows: both products on the fp8 MFMA (waves
    // without rows only load and wait)
    mla_rows8_kernel<<<blocks, 64 * kNW2, 0, stream>>>(p, nrt, ngroups);
  } else if (R <= kRW) {
    if (p.kv_dtype == FP8)
      mla_narrow_kernel<true><<<blocks, 64 * kNW2, 0, stream>>>(p, ngroups);
    else
      mla_narrow_kernel<false><<<blocks, 64 * kNW2, 0, stream>>>(p, ngroups);
  } else if (R <= 2 * kRW) {
    if (p.kv_dtype == FP8)
      mla_mid_kernel<true, 2><<<blocks, 64 * kNW2, 0, stream>>>(p, ngroups);
    else
      mla_mid_kernel<false, 2><<<blocks, 64 * kNW2, 0, stream>>>(p, ngroups);
  } else if (R <= 4 * kRW) {
    if (p.kv_dtype == FP8)
      mla_mid_kernel<true, 4><<<blocks, 64 * kNW2, 0, stream>>>(p, ngroups);
    else
      mla_mid_kernel<false, 4><<<blocks, 64 * kNW2, 0, stream>>>(p, ngroups);
  } else if (p.kv_dtype == FP8) {
    mla_rows_kernel<true><<<blocks, 64 * kNW2, 0, stream>>>(p, nrt, ngroups);
  } else {
    mla_rows_kernel<false><<<blocks, 64 * kNW2, 0, stream>>>(p, nrt, ngroups);
  }
  return hipGetLastError();
}

}  // namespace

bool mla_rows_path(const AttnParams& p) {
  // the kernels divide tokens within a page-id window by the page size with a
  // 32-bit reciprocal: window-relative tokens (< 256 pages) times the page size
  // below 2^32; page offsets and in-page offsets fit 32 bits
  return (p.kv_dtype == BF16 || p.kv_dtype == FP8) && p.page_size <= 4096 &&
         p.ks0 < (int64_t(1) << 31) &&
         (p.page_size - 1) * p.ks1 + (p.num_kv_heads - 1) * p.ks2 + kDqk < (int64_t(1) << 31);
}

bool mla_decode_supported(const AttnParams& p) {
  // other page sizes and strides go to the generic kernel
  return mla_rows_path(p) && p.qo_indptr == nullptr &&
         ((p.q_dtype == BF16 && (p.kv_dtype == BF16 || p.kv_dtype == FP8)) ||
          (p.q_dtype == FP8 && p.kv_dtype == FP8)) &&
         p.dqk == kDqk && p.dvo == kDvo && p.ks0 == p.vs0 && p.ks1 == p.vs1 && p.ks2 == p.vs2 &&
         p.k == p.v;
}

int mla_rows_per_tile(const AttnParams&) { return kRT2; }

int mla_tile_tokens(const AttnParams& p) {
  return p.q_dtype == FP8 && p.q_len * p.group > kRW ? kTKQ : kTK2;
}


int mla_blocks_per_cu(const AttnParams& p) {
  const bool fp8 = p.kv_dtype == FP8;
  const int R = p.q_len * p.group;
  const void* f = p.q_dtype == FP8 && R > kRW ? reinterpret_cast<const void*>(&mla_rows8_kernel)
                  : R <= kRW       ? (fp8 ? reinterpret_cast<const void*>(&mla_narrow_kernel<true>)
                                        : reinterpret_cast<const void*>(&mla_narrow_kernel<false>))
                  : R <= 2 * kRW ? (fp8 ? reinterpret_cast<const void*>(&mla_mid_kernel<true, 2>)
                                        : reinterpret_cast<const void*>(&mla_mid_kernel<false, 2>))
                  : R <= 4 * kRW ? (fp8 ? reinterpret_cast<const void*>(&mla_mid_kernel<true, 4>)
                                        : reinterpret_cast<const void*>(&mla_mid_kernel<false, 4>))
                  : p.q_dtype == FP8 ? reinterpret_cast<const void*>(&mla_rows8_kernel)
                                 : (fp8 ? reinterpret_cast<const void*>(&mla_rows_kernel<true>)
                                        : reinterpret_cast<const void*>(&mla_rows_kernel<false>));
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, 64 * kNW2, 0) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    n = 1;  // the kernels' LDS stages fill a CU
  }
  return n;
}

hipError_t launch_mla_decode(const AttnParams& p, hipStream_t stream) { return launch_rows(p, stream); }

}  // namespace pa
