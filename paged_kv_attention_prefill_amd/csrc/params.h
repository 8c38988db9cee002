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
  // internal KV chunking (load balance): chunk_tokens > 0 cuts every KV batch into
  // chunks of that many tokens (the last of max_chunks takes the rest); rows with
  // more than one chunk leave partial states in the workspace for a merge launch
  int32_t chunk_tokens;
  int32_t max_chunks;
  int32_t ws_rows;          // row slots per (batch, KV head, chunk) in the workspace
  float* ws_o;              // [B][Hkv][max_chunks][ws_rows][dvo], or [slots][ws_rows][dvo]
  float* ws_lse;            // [B][Hkv][max_chunks][ws_rows], or [slots][ws_rows]
  float* ws_mx;             // same as ws_lse
  // work-balanced split (decode, instead of chunks when bal_blocks > 0): bal_blocks
  // workgroups take equal shares of the (batch, KV head, unit) sequence, units of
  // bal_unit tokens; partial states go to slot item + workgroup, and ws_seg[2 item],
  // ws_seg[2 item + 1] receive the item's first and last workgroup
  int32_t bal_blocks;
  int32_t bal_unit;
  int32_t* ws_seg;          // [B * Hkv][2]
};

// Workspace slots of a balanced split: item + workgroup < items + blocks - 1.
inline int64_t bal_slots(int64_t items, int blocks) { return items + blocks - 1; }

// Number of chunks of a KV batch of L tokens under internal chunking.
__host__ __device__ inline int num_chunks(int L, int chunk_tokens, int max_chunks) {
  const int n = L > 0 ? (L + chunk_tokens - 1) / chunk_tokens : 1;
  return n < max_chunks ? n : max_chunks;
}

// Launchers (one per kernel family).  Return hipSuccess or the launch error.
hipError_t launch_generic(const AttnParams& p, hipStream_t stream);
bool gqa_decode_supported(const AttnParams& p);
hipError_t launch_gqa_decode(const AttnParams& p, bool same_strides, hipStream_t stream);
int gqa_decode_blocks_per_cu(const AttnParams& p, bool same_strides);
bool mla_decode_supported(const AttnParams& p);
bool mla_rows_path(const AttnParams& p);
int mla_rows_per_tile(const AttnParams& p);
bool mla_balanced_ok(const AttnParams& p);
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
