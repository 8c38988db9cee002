// Internal kernel parameters of libpaged_attn (host and device).  Not part of
// the C ABI: the entry points in api.cpp translate pa_*_args into this.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

enum Dt : int { F32 = 0, F16 = 1, BF16 = 2, FP8 = 3 };

// One attention launch over "query tokens" t in [0, total_q) and query heads.
// Decode calls arrive with qo_indptr == nullptr and a uniform q_len.
struct AttnParams {
  const void* q;
  const int32_t* qo_indptr;  // device, [batch+1]; nullptr => uniform q_len
  int32_t batch, q_len, total_q, num_qo_heads, num_kv_heads, group;
  const void* k;
  const void* v;
  int64_t ks0, ks1, ks2, vs0, vs1, vs2;
  int32_t page_size, dqk, dvo;
  int32_t page_shift;       // log2(page_size) if a power of two, else -1
  uint32_t page_magic;      // ceil(2^32 / page_size) (page_size >= 2): n / page_size ==
                            // umulhi(n, page_magic) for n * page_size < 2^32; 0 if page_size == 1
  float k_scale, v_scale, sm_scale;
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  const int32_t* kv_last;
  int32_t broadcast, causal;
  int32_t num_splits;       // states written per row (1: final result)
  int32_t partial_out;      // 1: write unnormalised-merge-ready partial states (fp32 O, LSE)
  void* o;                  // [S][total_q][Hq][dvo]
  float* lse;               // [S][total_q][Hq] or nullptr
  float* mx;                // [S][total_q][Hq] or nullptr
  int64_t o_split_stride;   // elements between states
  int64_t s_split_stride;   // elements between states of lse/mx
  int32_t q_dtype, kv_dtype, o_dtype;
  int32_t max_kv_len;       // host hint (0 unknown)
  int32_t max_q_len;        // host hint: >= every q_b
  int32_t ws_rows;          // row slots per workspace slot (balanced split)
  void* ws_o;               // [slots][ws_rows][dvo], elements of type ws_dtype
  int32_t ws_dtype;         // F32 (GQA decode) or BF16 (MLA kernels)
  float* ws_lse;            // [slots][ws_rows]
  float* ws_mx;             // same as ws_lse
  // work-balanced split (decode, when bal_blocks > 0): bal_blocks shares of equal
  // size of the (batch, KV head, unit) sequence, units of bal_unit tokens; partial
  // states go to slot item + share, and ws_seg[2 item], ws_seg[2 item + 1] receive
  // the item's first and last share
  int32_t bal_blocks;
  int32_t bal_unit;
  int32_t* ws_seg;          // [B * Hkv][2]
  // row tiles per share (MLA with more than one 128-row tile, else 1): the launch
  // has bal_blocks * bal_co workgroups, bal_co per share, one per row tile; they
  // stream the same KV range at the same time, so it is read once into their L2
  int32_t bal_co;
  // 1: workgroup w is virtual workgroup (w % 8) * (launch / 8) + w / 8 (share v /
  // bal_co, row tile v % bal_co), so that the row tiles of one share run on one XCD
  int32_t bal_xcd;
};

// Workspace slots of a balanced split: item + share < items + shares - 1.
inline int64_t bal_slots(int64_t items, int blocks) { return items + blocks - 1; }
// Items of a balanced split: (batch, KV head).
inline int64_t bal_items(const AttnParams& p) { return (int64_t)p.batch * p.num_kv_heads; }

// Size of the library-owned scratch array of the allocation-free decode entry
// point (one per GPU); noalloc_scratch() returns its device address on the
// current device (looked up once per device).
constexpr size_t kNoAllocScratchBytes = size_t(128) << 20;
hipError_t noalloc_scratch(void** ptr);

// Launchers (one per kernel family).  Return hipSuccess or the launch error.
hipError_t launch_generic(const AttnParams& p, hipStream_t stream);
bool gqa_decode_supported(const AttnParams& p);
hipError_t launch_gqa_decode(const AttnParams& p, bool same_strides, hipStream_t stream);
int gqa_decode_blocks_per_cu(const AttnParams& p, bool same_strides);
bool mla_decode_supported(const AttnParams& p);
bool mla_rows_path(const AttnParams& p);
int mla_rows_per_tile(const AttnParams& p);
int mla_tile_tokens(const AttnParams& p);  // KV tokens per tile of the kernel taken
int mla_blocks_per_cu(const AttnParams& p);
hipError_t launch_mla_decode(const AttnParams& p, hipStream_t stream);
bool flash_attn_supported(const AttnParams& p);
hipError_t launch_flash_attn(const AttnParams& p, bool same_strides, hipStream_t stream);
// Merge of internal splits; `wide`: one workgroup per row (rows with many states).
hipError_t launch_chunk_merge(const AttnParams& p, bool wide, hipStream_t stream);
hipError_t launch_merge(const void* v, int v_dtype, const float* s, int num_states, int64_t rows,
                        int head_dim, int64_t v_state_stride, int64_t s_state_stride, void* out,
                        int out_dtype, float* s_out, hipStream_t stream);

}  // namespace pa
