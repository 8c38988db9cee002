/*
 * paged_attn.h — C ABI of libpaged_attn.so: batched attention over a paged KV
 * cache on AMD Instinct MI355X (gfx950).
 *
 * The operation (all entry points): for every query row, the softmax-weighted
 * sum of V over the KV tokens the row may see, plus the row's log-sum-exp
 * (natural log of the scaled scores) and, optionally, its maximum score.
 *   - Paged KV cache with a page table (kv_indptr / kv_indices) and independent
 *     K and V strides: FlashInfer PR #4736 analysis, introduction and code
 *     section 1 (the paged_kv_t constructor receives separate K and V stride
 *     arrays).
 *   - Separate QK and VO head dims: same page, code section 2 (HEAD_DIM_QK /
 *     HEAD_DIM_VO template parameters).
 *   - Shared latent KV (MLA): FlashInfer PR #3309 analysis, code section 1.
 *   - KV batch broadcast: PyTorch 2.14 MPS FlexAttention post, introduction.
 *   - Log-sum-exp and max outputs: the same post, experiment section; the LSE
 *     buffer of the PR #3309 analysis, "why it is good".
 *   - Split-KV partial states merged through their LSE: "Move the Query, Not
 *     the Cache" summary, method section (Route), and the SM110 XQA split
 *     kernel, kernel-design section.
 *
 * Conventions
 *   - Every pointer is a DEVICE pointer unless marked "host".  Strides are in
 *     elements.  The innermost (head-dim) stride of Q, K, V and O is 1.
 *   - Token j of KV batch kb lives in physical page kv_indices[kv_indptr[kb] +
 *     j / page_size], slot j % page_size; element d of KV head g is at
 *       k + page*k_stride[0] + slot*k_stride[1] + g*k_stride[2] + d
 *     (likewise V with v_stride).  kv_len = (n-1)*page_size + last_page_len
 *     for n >= 1 pages, 0 for n == 0.
 *   - A sparse selection of token rows per query (the "Move the Query, Not the
 *     Cache" summary, problem statement: KV picked by a sparse indexer) is a
 *     KV batch per query with page_size 1: kv_indices then lists the selected
 *     token slots, last_page_len is 1, and no causal mask is needed.
 *   - Query head h reads KV head h / (num_qo_heads / num_kv_heads).
 *   - causal: query i of a batch with q_b queries sits at position
 *     kv_len - q_b + i and sees KV tokens j <= that position.
 *   - A row that sees no token gets O = 0, LSE = -inf, max = -inf.
 *   - LSE is the natural log of sum_j exp(sm_scale * q.k_j) (k_scale folded in).
 *   - fp8 queries (e4m3 codes with a per-tensor q_scale, over an fp8 cache): the
 *     MLA shapes with more than 64 rows per request multiply fp8 Q by fp8 K on
 *     the fp8 matrix cores (the FP8 MLA decode target of the PR #3309
 *     analysis, introduction); every e4m3 code is exact in the kernels'
 *     arithmetic, so results match the real-valued definition on those codes
 *     up to fp32 accumulation and 16-bit rounding of P, as for 16-bit queries.
 *
 * Ownership and concurrency
 *   - The caller owns every buffer.  The library allocates nothing on the
 *     compute path and keeps no pointer after a call returns (the one array it
 *     owns, the per-GPU scratch of paged_attn_decode_noalloc, is allocated when
 *     the library loads).
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     null stream).  Buffers must stay alive until the stream passes the call.
 *   - A workspace belongs to one in-flight call; two calls that overlap in
 *     time must not share one (the PR #3309 analysis traces a multi-token
 *     mismatch to exactly such sharing, reviewer-feedback section).
 *   - All entry points are reentrant; calls of paged_attn_decode_noalloc that
 *     overlap in time on one GPU share its scratch array and race (see there).
 *
 * Errors
 *   - Arguments are validated on the host first; a failed check returns a
 *     negative pa_status and enqueues nothing (this replaces the abort-style
 *     stride equality check shown in the PR #4736 analysis, code section 1).
 *   - Contents of device-resident tables (kv_indices in range, monotone
 *     indptrs, 1 <= last_page_len <= page_size for non-empty batches) are
 *     preconditions and are not checked on the compute path;
 *     paged_attn_check_tables() checks host copies.
 *   - A failed kernel launch returns PA_ERR_HIP.
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 2

typedef void* pa_stream_t; /* a hipStream_t */

typedef enum {
  PA_F32 = 0,
  PA_F16 = 1,
  PA_BF16 = 2,
  PA_FP8_E4M3 = 3 /* OCP e4m3fn: bias 7, max 448, S.1111.111 = NaN, no inf */
} pa_dtype;

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = -1,        /* a required pointer is NULL */
  PA_ERR_SHAPE = -2,       /* a size is out of range or inconsistent */
  PA_ERR_DTYPE = -3,       /* dtype value unknown or not allowed for that buffer */
  PA_ERR_ALIGN = -4,       /* pointer or stride not 16-byte aligned */
  PA_ERR_UNSUPPORTED = -5, /* valid request with no kernel for it (head dims, dtype combo) */
  PA_ERR_WORKSPACE = -6,   /* workspace NULL or smaller than the queried size */
  PA_ERR_HIP = -7          /* HIP runtime error while launching */
} pa_status;

/* Test and tuning flags (pa_*_args.flags).  Results do not depend on them
 * beyond floating-point rounding. */
#define PA_FLAG_FORCE_GENERAL_STRIDES 0x1u /* never take the equal-K/V-strides variant */
#define PA_FLAG_FORCE_GENERIC 0x2u         /* use the generic vector kernel */
#define PA_FLAG_NO_INTERNAL_SPLIT 0x4u     /* one pass per row, no internal split + merge */

/* One paged KV cache. */
typedef struct {
  const void* k;            /* K cache base */
  const void* v;            /* V cache base; may equal k (shared latent rows: V is the first
                               head_dim_vo elements of each K row, v_stride == k_stride) */
  int64_t k_stride[3];      /* [page, slot, kv head], elements; each * elem size % 16 == 0 */
  int64_t v_stride[3];
  int32_t num_kv_heads;
  int32_t page_size;        /* tokens per page, >= 1 */
  int32_t head_dim_qk;      /* supported (qk, vo): (64,64) (128,128) (256,256) (576,512) */
  int32_t head_dim_vo;
  pa_dtype kv_dtype;        /* F32, F16, BF16 or FP8_E4M3 */
  float k_scale;            /* real K = k_scale * stored K (fp8 per-tensor scale; 1 otherwise) */
  float v_scale;            /* real V = v_scale * stored V */
  const int32_t* kv_indptr; /* [num_kv_batches + 1], kv_indptr[0] == 0, non-decreasing */
  const int32_t* kv_indices;       /* [kv_indptr[num_kv_batches]] physical page ids */
  const int32_t* kv_last_page_len; /* [num_kv_batches], in [1, page_size] when n >= 1 */
  int32_t num_kv_batches;
  int32_t max_kv_len_hint;  /* host value: >= every kv_len, or 0 if unknown; decides whether
                               a decode splits the KV internally (0: never) and sizes the
                               workspace; it changes results only by rounding */
} pa_paged_kv;

/* Decode: every query batch has the same number of queries, q_len. */
typedef struct {
  const void* q;            /* [batch, q_len, num_qo_heads, head_dim_qk], contiguous */
  pa_dtype q_dtype;         /* F32, F16, BF16, or FP8_E4M3 with an FP8_E4M3 cache (q_scale) */
  int32_t batch;
  int32_t q_len;
  int32_t num_qo_heads;     /* multiple of kv.num_kv_heads */
  pa_paged_kv kv;
  int32_t kv_broadcast;     /* 1: kv.num_kv_batches == 1 and every query batch reads KV batch 0 */
  int32_t causal;
  float sm_scale;
  int32_t num_kv_splits;    /* S = 1: final O/LSE.  S > 1: S partial states, state c covering
                               pages [floor(c*n/S), floor((c+1)*n/S)) of each KV batch, to be
                               merged by merge_states(); O must then be F32 */
  void* o;                  /* [S][batch, q_len, num_qo_heads, head_dim_vo] */
  pa_dtype o_dtype;         /* F32, F16 or BF16 */
  float* lse;               /* [S][batch, q_len, num_qo_heads]; may be NULL only if S == 1 */
  float* row_max;           /* same shape as lse; NULL to skip */
  uint32_t flags;           /* PA_FLAG_* */
  void* timing_events[2];   /* optional hipEvent_t pair recorded on `stream` right before and
                               right after the attention kernel (not around a merge launch);
                               NULL to skip */
  float q_scale;            /* FP8_E4M3 queries only: real Q = q_scale * stored Q (a per-tensor
                               scale, as k_scale); ignored for other query dtypes */
} pa_decode_args;

/* Prefill: ragged query batches; the new tokens' K/V are already in the cache
 * (kv_len counts them), so causal query i of batch b sits at kv_len_b - q_b + i. */
typedef struct {
  const void* q;            /* [total_q, num_qo_heads, head_dim_qk], contiguous */
  pa_dtype q_dtype;
  const int32_t* qo_indptr; /* [batch + 1] device; batch b owns rows qo_indptr[b]..[b+1]) */
  int32_t batch;
  int32_t total_q;          /* host value == qo_indptr[batch] */
  int32_t max_q_len_hint;   /* host value: >= every q_b, or 0 (then total_q is used) */
  int32_t num_qo_heads;
  pa_paged_kv kv;
  int32_t kv_broadcast;
  int32_t causal;
  float sm_scale;
  void* o;                  /* [total_q, num_qo_heads, head_dim_vo] */
  pa_dtype o_dtype;
  float* lse;               /* [total_q, num_qo_heads]; NULL to skip */
  float* row_max;           /* NULL to skip */
  uint32_t flags;
  void* timing_events[2];   /* as in pa_decode_args */
  float q_scale;            /* as in pa_decode_args */
} pa_prefill_args;

int pa_abi_version(void);
const char* pa_status_string(int status);

/* Host-only: name of the kernel plan the call would run (a static string, e.g.
 * "gqa_decode_mfma" or "generic"), or NULL if the arguments are invalid.
 * Enqueues no GPU work (may make the device queries described below). */
const char* paged_attn_decode_plan_name(const pa_decode_args* args);
const char* paged_attn_prefill_plan_name(const pa_prefill_args* args);

/* Host-only: bytes of device workspace the call needs (0 is possible).
 * Enqueues no GPU work.  The size of the internal KV split of a decode depends
 * on the current device (its compute-unit count and the kernels' occupancy,
 * read once per device with HIP device queries): query with the device current
 * that the call will run on. */
int paged_attn_decode_workspace_size(const pa_decode_args* args, size_t* bytes);
int paged_attn_prefill_workspace_size(const pa_prefill_args* args, size_t* bytes);

/* Enqueue one decode / prefill call.  workspace: device buffer of at least the
 * queried size (may be NULL when that size is 0). */
int paged_attn_decode(const pa_decode_args* args, void* workspace, size_t workspace_bytes,
                      pa_stream_t stream);
int paged_attn_prefill(const pa_prefill_args* args, void* workspace, size_t workspace_bytes,
                       pa_stream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): paged_attn_decode with
 * the same arguments, kernels and results, whose workspace is a device array
 * owned by the library instead of a caller buffer.  The caller still passes
 * every input and output.  The array holds PA_NOALLOC_SCRATCH_BYTES per GPU;
 * each GPU the library runs on holds its copy from the time the library loads
 * until the process ends.  A call whose workspace (paged_attn_decode_workspace_
 * size) exceeds that returns PA_ERR_WORKSPACE and enqueues nothing.  The call
 * allocates nothing (no hipMalloc, no allocating library routine).  Every call
 * on one GPU shares that GPU's array, and no kernel expects it to hold anything
 * on entry (each workspace byte read is written earlier in the same call), so
 * calls that overlap in time on one GPU (two streams, two threads) race and
 * must be serialised by the caller.  Returns PA_ERR_HIP if the array's device
 * address cannot be read. */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int paged_attn_decode_noalloc(const pa_decode_args* args, pa_stream_t stream);

/* Merge S partial attention states per row through their LSE:
 *   m = max_c s_c, w_c = exp(s_c - m), out = sum_c w_c v_c / sum_c w_c,
 *   s_out = m + ln sum_c w_c; states with s_c = -inf carry no weight; a row
 *   whose states are all -inf gets out = 0, s_out = -inf.
 * v_states [num_states, rows, head_dim] (F32, F16 or BF16), s_states
 * [num_states, rows] natural-log LSE, v_out [rows, head_dim], s_out [rows]
 * (nullable).  head_dim % 4 == 0, 1 <= num_states <= 1024. */
int merge_states(const void* v_states, pa_dtype v_dtype, const float* s_states,
                 int32_t num_states, int64_t rows, int32_t head_dim, void* v_out,
                 pa_dtype out_dtype, float* s_out, pa_stream_t stream);

/* Host-only check of HOST copies of a page table: indptr[0] == 0 and
 * non-decreasing, every index in [0, num_pool_pages), 1 <= last <= page_size
 * for batches with pages.  Returns PA_OK or PA_ERR_SHAPE. */
int paged_attn_check_tables(const int32_t* h_indptr, const int32_t* h_indices,
                            const int32_t* h_last_page_len, int32_t num_kv_batches,
                            int32_t num_pool_pages, int32_t page_size);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */
