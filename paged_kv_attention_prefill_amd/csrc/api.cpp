// C-ABI entry points of libpaged_attn: host-side validation, kernel choice
// (decided on the host and launched as a specialised kernel rather than
// branching inside the kernel — FlashInfer PR #4736 analysis, "lessons"
// section), workspace planning, launch on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/paged_attn.h"
#include "params.h"

namespace {

using pa::AttnParams;

bool log_enabled() {
  static const bool on = [] {
    const char* e = std::getenv("PA_LOG");
    return e && e[0] == '1';
  }();
  return on;
}

int elem_bytes(int dt) { return dt == PA_F32 ? 4 : dt == PA_FP8_E4M3 ? 1 : 2; }
bool known_dtype(int dt) { return dt >= PA_F32 && dt <= PA_FP8_E4M3; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_dims(int dqk, int dvo) {
  return (dqk == 64 && dvo == 64) || (dqk == 128 && dvo == 128) || (dqk == 256 && dvo == 256) ||
         (dqk == 576 && dvo == 512);
}

bool supported_combo(int qdt, int kvdt) {
  return (qdt == PA_F32 && kvdt == PA_F32) || (qdt == PA_F16 && kvdt == PA_F16) ||
         (qdt == PA_BF16 && kvdt == PA_BF16) || (qdt == PA_BF16 && kvdt == PA_FP8_E4M3) ||
         (qdt == PA_F16 && kvdt == PA_FP8_E4M3) || (qdt == PA_FP8_E4M3 && kvdt == PA_FP8_E4M3);
}

// Checks shared by decode and prefill.  Returns PA_OK or the first failure.
int check_common(const void* q, int q_dtype, int num_qo_heads, const pa_paged_kv& kv,
                 int kv_broadcast, int expect_kv_batches, const void* o, int o_dtype) {
  if (!q || !kv.k || !kv.v || !kv.kv_indptr || !kv.kv_indices || !kv.kv_last_page_len || !o)
    return PA_ERR_NULL;
  if (!known_dtype(q_dtype) || !known_dtype(kv.kv_dtype) || !known_dtype(o_dtype))
    return PA_ERR_DTYPE;
  if (o_dtype == PA_FP8_E4M3) return PA_ERR_DTYPE;
  if (num_qo_heads < 1 || kv.num_kv_heads < 1 || kv.page_size < 1) return PA_ERR_SHAPE;
  if (num_qo_heads % kv.num_kv_heads != 0) return PA_ERR_SHAPE;
  if (kv.num_kv_batches < 1) return PA_ERR_SHAPE;
  if (kv_broadcast ? kv.num_kv_batches != 1 : kv.num_kv_batches != expect_kv_batches)
    return PA_ERR_SHAPE;
  if (kv.max_kv_len_hint < 0) return PA_ERR_SHAPE;
  if (kv.head_dim_qk < 1 || kv.head_dim_vo < 1) return PA_ERR_SHAPE;
  for (int i = 0; i < 3; ++i)
    if (kv.k_stride[i] < 0 || kv.v_stride[i] < 0) return PA_ERR_SHAPE;
  if (kv.k == kv.v) {
    if (kv.head_dim_vo > kv.head_dim_qk) return PA_ERR_SHAPE;
    for (int i = 0; i < 3; ++i)
      if (kv.k_stride[i] != kv.v_stride[i]) return PA_ERR_SHAPE;
  }
  if (!(std::isfinite(kv.k_scale) && std::isfinite(kv.v_scale))) return PA_ERR_SHAPE;
  if (!supported_combo(q_dtype, kv.kv_dtype)) return PA_ERR_UNSUPPORTED;
  if (!supported_dims(kv.head_dim_qk, kv.head_dim_vo)) return PA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(kv.k) || !aligned16(kv.v) || !aligned16(o)) return PA_ERR_ALIGN;
  const int eb = elem_bytes(kv.kv_dtype);
  for (int i = 0; i < 3; ++i)
    if ((kv.k_stride[i] * eb) % 16 != 0 || (kv.v_stride[i] * eb) % 16 != 0) return PA_ERR_ALIGN;
  return PA_OK;
}

void fill_kv(AttnParams& p, const pa_paged_kv& kv) {
  p.k = kv.k;
  p.v = kv.v;
  p.ks0 = kv.k_stride[0]; p.ks1 = kv.k_stride[1]; p.ks2 = kv.k_stride[2];
  p.vs0 = kv.v_stride[0]; p.vs1 = kv.v_stride[1]; p.vs2 = kv.v_stride[2];
  p.page_size = kv.page_size;
  p.page_shift = -1;
  for (int sh = 0; sh < 31; ++sh)
    if ((1 << sh) == kv.page_size) p.page_shift = sh;
  p.page_magic = kv.page_size == 1
                     ? 0u
                     : (uint32_t)(((uint64_t(1) << 32) + kv.page_size - 1) / kv.page_size);
  p.dqk = kv.head_dim_qk;
  p.dvo = kv.head_dim_vo;
  p.k_scale = kv.k_scale;
  p.v_scale = kv.v_scale;
  p.kv_indptr = kv.kv_indptr;
  p.kv_indices = kv.kv_indices;
  p.kv_last = kv.kv_last_page_len;
  p.kv_dtype = kv.kv_dtype;
  p.max_kv_len = kv.max_kv_len_hint;
}

// Query scale folded into the score scale: q_scale for fp8 queries, 1 otherwise.
float query_scale(int q_dtype, float q_scale) { return q_dtype == PA_FP8_E4M3 ? q_scale : 1.f; }

// The kernels scale scores by sm_scale * q_scale * k_scale * log2(e) in fp32;
// that product must be finite (a scale that overflows it has no fp32 result).
bool finite_score_scale(float sm_scale, float q_scale, float k_scale) {
  return std::isfinite(sm_scale) && std::isfinite(q_scale) &&
         std::isfinite(sm_scale * q_scale * k_scale * 1.4426950408889634f);
}

int check_decode(const pa_decode_args* a) {
  if (!a) return PA_ERR_NULL;
  if (a->batch < 1 || a->q_len < 1) return PA_ERR_SHAPE;
  if (a->num_kv_splits < 1 || a->num_kv_splits > 1024) return PA_ERR_SHAPE;
  if (!finite_score_scale(a->sm_scale, query_scale(a->q_dtype, a->q_scale), a->kv.k_scale))
    return PA_ERR_SHAPE;
  int st = check_common(a->q, a->q_dtype, a->num_qo_heads, a->kv, a->kv_broadcast, a->batch, a->o,
                        a->o_dtype);
  if (st != PA_OK) return st;
  if (a->num_kv_splits > 1) {
    if (!a->lse) return PA_ERR_NULL;
    if (a->o_dtype != PA_F32) return PA_ERR_DTYPE;
  }
  if ((int64_t)a->batch * a->q_len > INT32_MAX / 2) return PA_ERR_SHAPE;
  return PA_OK;
}

int check_prefill(const pa_prefill_args* a) {
  if (!a) return PA_ERR_NULL;
  if (!a->qo_indptr) return PA_ERR_NULL;
  if (a->batch < 1 || a->total_q < 0 || a->max_q_len_hint < 0) return PA_ERR_SHAPE;
  if (!finite_score_scale(a->sm_scale, query_scale(a->q_dtype, a->q_scale), a->kv.k_scale))
    return PA_ERR_SHAPE;
  return check_common(a->q, a->q_dtype, a->num_qo_heads, a->kv, a->kv_broadcast, a->batch, a->o,
                      a->o_dtype);
}

AttnParams params_decode(const pa_decode_args* a) {
  AttnParams p{};
  p.q = a->q;
  p.qo_indptr = nullptr;
  p.batch = a->batch;
  p.q_len = a->q_len;
  p.total_q = a->batch * a->q_len;
  p.max_q_len = a->q_len;
  p.num_qo_heads = a->num_qo_heads;
  fill_kv(p, a->kv);
  p.num_kv_heads = a->kv.num_kv_heads;
  p.group = a->num_qo_heads / a->kv.num_kv_heads;
  p.sm_scale = a->sm_scale * query_scale(a->q_dtype, a->q_scale);  // real Q = q_scale * codes
  p.broadcast = a->kv_broadcast ? 1 : 0;
  p.causal = a->causal ? 1 : 0;
  p.num_splits = a->num_kv_splits;
  p.partial_out = a->num_kv_splits > 1;
  p.o = a->o;
  p.lse = a->lse;
  p.mx = a->row_max;
  p.o_split_stride = (int64_t)p.total_q * p.num_qo_heads * p.dvo;
  p.s_split_stride = (int64_t)p.total_q * p.num_qo_heads;
  p.q_dtype = a->q_dtype;
  p.o_dtype = a->o_dtype;
  return p;
}

AttnParams params_prefill(const pa_prefill_args* a) {
  AttnParams p{};
  p.q = a->q;
  p.qo_indptr = a->qo_indptr;
  p.batch = a->batch;
  p.q_len = 0;
  p.total_q = a->total_q;
  p.max_q_len = a->max_q_len_hint > 0 ? a->max_q_len_hint : a->total_q;
  p.num_qo_heads = a->num_qo_heads;
  fill_kv(p, a->kv);
  p.num_kv_heads = a->kv.num_kv_heads;
  p.group = a->num_qo_heads / a->kv.num_kv_heads;
  p.sm_scale = a->sm_scale * query_scale(a->q_dtype, a->q_scale);
  p.broadcast = a->kv_broadcast ? 1 : 0;
  p.causal = a->causal ? 1 : 0;
  p.num_splits = 1;
  p.partial_out = 0;
  p.o = a->o;
  p.lse = a->lse;
  p.mx = a->row_max;
  p.o_split_stride = (int64_t)p.total_q * p.num_qo_heads * p.dvo;
  p.s_split_stride = (int64_t)p.total_q * p.num_qo_heads;
  p.q_dtype = a->q_dtype;
  p.o_dtype = a->o_dtype;
  return p;
}

// The plan of one call: which kernels run and how much workspace they need.
struct Plan {
  enum Kind { GENERIC, GQA_DECODE, FLASH, MLA_DECODE } kind = GENERIC;
  bool same_strides = false;  // V offsets reuse K offsets (equal K/V strides)
  int ws_rows = 16;           // workspace row slots per (batch, KV head, share)
  int ws_dtype = pa::F32;     // element type of the partial O in the workspace
  int bal_blocks = 0;         // balanced split over this many workgroups (0: none)
  int bal_unit = 0;           // its unit of work in KV tokens
  int bal_co = 1;             // workgroups (row tiles) per share of the balanced split
  int bal_xcd = 0;            // the row tiles of a share on one XCD
  size_t workspace = 0;
  const char* name = "generic";
};

bool equal_kv_strides(const AttnParams& p) {
  return p.ks0 == p.vs0 && p.ks1 == p.vs1 && p.ks2 == p.vs2;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Whether the folded-GQA decode splits its KV over workgroups (the balanced
// split): when the longest KV exceeds one piece of about 2048 tokens (less with
// few (batch, head) items, so that there are ~1536 pieces; page aligned).
// Decided from host values only (identical for the size query and the launch),
// never from device state.
bool decode_split_kv(const AttnParams& p, uint32_t flags) {
  if ((flags & PA_FLAG_NO_INTERNAL_SPLIT) || p.num_splits != 1 || p.max_kv_len <= 0) return false;
  const int64_t items = (int64_t)p.batch * p.num_kv_heads;
  int c = 2048;
  while (c > 256 && items * ((p.max_kv_len + c - 1) / c) < 1536) c /= 2;
  c = (c + p.page_size - 1) / p.page_size * p.page_size;
  return p.max_kv_len > c;
}

// Per-device values read once with HIP device queries (compute-unit count,
// kernel occupancies).  Slots are atomics: concurrent first calls may both run
// the query, and both store the same value.
constexpr int kMaxDevices = 64;

int current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return -1;
  }
  return dev;
}

// Cached per-device value: slot[dev] once `query()` has been called there.
template <typename Query>
int per_device(std::atomic<int>* slot, int fallback, Query query) {
  const int dev = current_device();
  if (dev < 0) return fallback;
  int v = slot[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    v = query(dev);
    if (v <= 0) v = fallback;
    slot[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// Compute units of the current device (MI355X: 256).
int device_cus() {
  static std::atomic<int> cache[kMaxDevices];
  return per_device(cache, 256, [](int dev) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
      (void)hipGetLastError();
      n = 0;
    }
    return n;
  });
}

// Workspace of a balanced split over `blocks` shares: partial states in slots
// item + share (O in elements of ws_dtype, LSE and max in fp32), then the
// first/last share of every item ((batch, KV head)).
size_t ws_o_bytes(size_t rows, int dvo, int ws_dtype) {
  return align256(rows * dvo * (ws_dtype == pa::F32 ? 4 : 2));
}
size_t balanced_workspace(const AttnParams& p, int blocks, int ws_rows, int ws_dtype) {
  const int64_t items = (int64_t)p.batch * p.num_kv_heads;
  const size_t rows = (size_t)pa::bal_slots(items, blocks) * ws_rows;
  return ws_o_bytes(rows, p.dvo, ws_dtype) + 2 * align256(rows * 4) + align256((size_t)items * 8);
}

// Whether the MLA decode splits its KV over workgroups (the balanced split):
// when the longest KV exceeds one piece of the largest power of two (512..8192
// tokens, page aligned) that still gives about a thousand (request, row tile,
// piece) work items.
bool mla_split_kv(const AttnParams& p, uint32_t flags) {
  if ((flags & PA_FLAG_NO_INTERNAL_SPLIT) || p.num_splits != 1 || p.max_kv_len <= 0) return false;
  const int R = p.q_len * p.group;
  const int rt = pa::mla_rows_per_tile(p);
  const int64_t tiles = (int64_t)p.batch * p.num_kv_heads * ((R + rt - 1) / rt);
  int c = 8192;
  while (c > 512 && tiles * ((p.max_kv_len + c - 1) / c) < 1024) c /= 2;
  c = (c + p.page_size - 1) / p.page_size * p.page_size;
  return p.max_kv_len > c;
}

// Workgroups per CU of the balanced GQA decode kernel variant, per device.
int gqa_occupancy(const AttnParams& p, bool same) {
  static std::atomic<int> occ[2][3][2][kMaxDevices];
  return per_device(occ[p.q_dtype == PA_BF16][p.dqk == 64 ? 0 : p.dqk == 128 ? 1 : 2][same], 1,
                    [&](int) { return pa::gqa_decode_blocks_per_cu(p, same); });
}

// Workgroups per CU of the MLA decode kernel for this row count, per device.
int mla_occupancy(const AttnParams& p) {
  static std::atomic<int> occ[3][4][kMaxDevices];
  const int R = p.q_len * p.group;
  const int dt = p.q_dtype == PA_FP8_E4M3 ? 2 : p.kv_dtype == PA_FP8_E4M3 ? 1 : 0;
  return per_device(occ[dt][R <= 16 ? 0 : R <= 32 ? 1 : R <= 64 ? 2 : 3], 1,
                    [&](int) { return pa::mla_blocks_per_cu(p); });
}

Plan make_plan(const AttnParams& p, uint32_t flags) {
  Plan pl;
  const bool same = equal_kv_strides(p) && !(flags & PA_FLAG_FORCE_GENERAL_STRIDES);
  if (flags & PA_FLAG_FORCE_GENERIC) return pl;
  // rows that read one KV head's data: q_len x G per query batch, or, under
  // broadcast, those of every query batch together
  const int64_t rows_per_kv = (int64_t)(p.broadcast ? p.total_q : p.max_q_len) * p.group;
  if (pa::gqa_decode_supported(p) && (!p.broadcast || rows_per_kv <= 16)) {
    pl.kind = Plan::GQA_DECODE;
    pl.same_strides = same;
    pl.name = same ? "gqa_decode_mfma_same_strides" : "gqa_decode_mfma";
    // KV long enough to be worth splitting: a balanced split over one wave of
    // co-resident workgroups (every workgroup streams the same number of
    // 32-token tiles, so none idles at the end)
    if (decode_split_kv(p, flags)) {
      pl.bal_unit = 32;
      pl.bal_blocks = gqa_occupancy(p, same) * device_cus();
      pl.workspace = balanced_workspace(p, pl.bal_blocks, 16, pl.ws_dtype);
    }
    return pl;
  }
  // The flash and MLA kernels take the running max of raw scores and apply the
  // score scale afterwards, which orders scores correctly only for a positive
  // scale; a zero or negative scale goes to the generic kernel (it scales
  // every score first).
  const bool positive_scale = p.sm_scale * p.k_scale * 1.4426950408889634f > 0.f;
  if (positive_scale && pa::mla_decode_supported(p)) {
    pl.kind = Plan::MLA_DECODE;
    pl.name = p.q_dtype == PA_FP8_E4M3    ? "mla_decode_mfma_fp8q"
              : p.kv_dtype == PA_FP8_E4M3 ? "mla_decode_mfma_fp8"
                                          : "mla_decode_mfma";
    if (mla_split_kv(p, flags)) {
      // balanced split over one wave of workgroups; with several 128-row tiles
      // per request, a share is taken by one workgroup per row tile, on one XCD
      // (they stream the same KV tokens together, read once into its L2), and
      // the shares are as many as such groups fit, in whole groups per XCD
      const int R = p.q_len * p.group;
      const int rt = pa::mla_rows_per_tile(p);
      const int nrt = (R + rt - 1) / rt;
      const int wgs = mla_occupancy(p) * device_cus();
      pl.bal_co = nrt;
      pl.bal_unit = pa::mla_tile_tokens(p);
      pl.bal_blocks = nrt > 1 && wgs >= 8 * nrt ? wgs / nrt / 8 * 8 : std::max(1, wgs / nrt);
      pl.bal_xcd = nrt > 1 && pl.bal_blocks % 8 == 0;
      pl.ws_rows = R;
      // bf16 partial O: R rows x 512 dims per share are the bulk of the
      // split's extra traffic (written here, read by the merge)
      pl.ws_dtype = pa::BF16;
      pl.workspace = balanced_workspace(p, pl.bal_blocks, pl.ws_rows, pl.ws_dtype);
    }
    return pl;
  }
  if (positive_scale && pa::flash_attn_supported(p)) {
    pl.kind = Plan::FLASH;
    pl.same_strides = same;
    pl.name = same ? "flash_attn_mfma_same_strides" : "flash_attn_mfma";
    return pl;
  }
  return pl;
}

int run_plan(const Plan& pl, AttnParams p, void* ws, size_t ws_bytes, void* const* events,
             hipStream_t stream) {
  if (pl.workspace > 0 && (!ws || ws_bytes < pl.workspace)) return PA_ERR_WORKSPACE;
  if (log_enabled())
    std::fprintf(stderr,
                 "[paged_attn] kernel=%s total_q=%d Hq=%d Hkv=%d dqk=%d dvo=%d splits=%d "
                 "balanced=%d x%d x%d ws=%zu\n",
                 pl.name, p.total_q, p.num_qo_heads, p.num_kv_heads, p.dqk, p.dvo, p.num_splits,
                 pl.bal_blocks, pl.bal_co, pl.bal_unit, pl.workspace);
  p.ws_rows = pl.ws_rows;
  p.ws_dtype = pl.ws_dtype;
  p.bal_blocks = pl.bal_blocks;
  p.bal_unit = pl.bal_unit;
  p.bal_co = pl.bal_co;
  p.bal_xcd = pl.bal_xcd;
  if (pl.bal_blocks > 0) {
    const int64_t items = pa::bal_items(p);
    const size_t rows = (size_t)pa::bal_slots(items, pl.bal_blocks) * pl.ws_rows;
    char* w = static_cast<char*>(ws);
    const size_t ob = ws_o_bytes(rows, p.dvo, pl.ws_dtype);
    p.ws_o = w;
    p.ws_lse = reinterpret_cast<float*>(w + ob);
    p.ws_mx = reinterpret_cast<float*>(w + ob + align256(rows * 4));
    p.ws_seg = reinterpret_cast<int32_t*>(w + ob + 2 * align256(rows * 4));
  }
  const bool timed = events && events[0] && events[1];
  if (timed && hipEventRecord(static_cast<hipEvent_t>(events[0]), stream) != hipSuccess)
    return PA_ERR_HIP;
  hipError_t e = hipSuccess;
  switch (pl.kind) {
    case Plan::GENERIC:
      e = pa::launch_generic(p, stream);
      break;
    case Plan::GQA_DECODE:
      e = pa::launch_gqa_decode(p, pl.same_strides, stream);
      break;
    case Plan::FLASH:
      e = pa::launch_flash_attn(p, pl.same_strides, stream);
      break;
    case Plan::MLA_DECODE:
      e = pa::launch_mla_decode(p, stream);
      break;
  }
  if (e != hipSuccess) return PA_ERR_HIP;
  if (timed && hipEventRecord(static_cast<hipEvent_t>(events[1]), stream) != hipSuccess)
    return PA_ERR_HIP;
  if (pl.bal_blocks > 0) {
    // many states per row (few long items over many shares): split each row's
    // states over the lane groups of a workgroup
    const int64_t items = (int64_t)p.batch * p.num_kv_heads;
    const bool wide = pl.bal_blocks >= 32 * items;
    e = pa::launch_chunk_merge(p, wide, stream);
  }
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace

extern "C" {

int pa_abi_version(void) { return PA_ABI_VERSION; }

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_SHAPE: return "a size is out of range or inconsistent";
    case PA_ERR_DTYPE: return "dtype unknown or not allowed for this buffer";
    case PA_ERR_ALIGN: return "pointer or stride not 16-byte aligned";
    case PA_ERR_UNSUPPORTED: return "no kernel for this head-dim / dtype combination";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP runtime error while launching";
    default: return "unknown status";
  }
}

const char* paged_attn_decode_plan_name(const pa_decode_args* args) {
  if (check_decode(args) != PA_OK) return nullptr;
  return make_plan(params_decode(args), args->flags).name;
}

const char* paged_attn_prefill_plan_name(const pa_prefill_args* args) {
  if (check_prefill(args) != PA_OK) return nullptr;
  return make_plan(params_prefill(args), args->flags).name;
}

int paged_attn_decode_workspace_size(const pa_decode_args* args, size_t* bytes) {
  if (!bytes) return PA_ERR_NULL;
  const int st = check_decode(args);
  if (st != PA_OK) return st;
  *bytes = make_plan(params_decode(args), args->flags).workspace;
  return PA_OK;
}

int paged_attn_prefill_workspace_size(const pa_prefill_args* args, size_t* bytes) {
  if (!bytes) return PA_ERR_NULL;
  const int st = check_prefill(args);
  if (st != PA_OK) return st;
  *bytes = make_plan(params_prefill(args), args->flags).workspace;
  return PA_OK;
}

int paged_attn_decode(const pa_decode_args* args, void* workspace, size_t workspace_bytes,
                      pa_stream_t stream) {
  const int st = check_decode(args);
  if (st != PA_OK) return st;
  const AttnParams p = params_decode(args);
  return run_plan(make_plan(p, args->flags), p, workspace, workspace_bytes, args->timing_events,
                  static_cast<hipStream_t>(stream));
}

int paged_attn_decode_noalloc(const pa_decode_args* args, pa_stream_t stream) {
  const int st = check_decode(args);
  if (st != PA_OK) return st;
  const AttnParams p = params_decode(args);
  const Plan pl = make_plan(p, args->flags);
  if (pl.workspace > pa::kNoAllocScratchBytes) return PA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (pl.workspace > 0 && pa::noalloc_scratch(&ws) != hipSuccess) {
    (void)hipGetLastError();
    return PA_ERR_HIP;
  }
  return run_plan(pl, p, ws, pl.workspace > 0 ? pa::kNoAllocScratchBytes : 0, args->timing_events,
                  static_cast<hipStream_t>(stream));
}

int paged_attn_prefill(const pa_prefill_args* args, void* workspace, size_t workspace_bytes,
                       pa_stream_t stream) {
  const int st = check_prefill(args);
  if (st != PA_OK) return st;
  if (args->total_q == 0) return PA_OK;
  const AttnParams p = params_prefill(args);
  return run_plan(make_plan(p, args->flags), p, workspace, workspace_bytes, args->timing_events,
                  static_cast<hipStream_t>(stream));
}

int merge_states(const void* v_states, pa_dtype v_dtype, const float* s_states,
                 int32_t num_states, int64_t rows, int32_t head_dim, void* v_out,
                 pa_dtype out_dtype, float* s_out, pa_stream_t stream) {
  if (!v_states || !s_states || !v_out) return PA_ERR_NULL;
  if (!known_dtype(v_dtype) || !known_dtype(out_dtype)) return PA_ERR_DTYPE;
  if (v_dtype == PA_FP8_E4M3 || out_dtype == PA_FP8_E4M3) return PA_ERR_DTYPE;
  if (num_states < 1 || num_states > 1024 || rows < 0) return PA_ERR_SHAPE;
  if (head_dim < 4 || head_dim > 1024 || head_dim % 4 != 0) return PA_ERR_SHAPE;
  if (!aligned16(v_states) || !aligned16(v_out)) return PA_ERR_ALIGN;
  if (rows == 0) return PA_OK;
  const hipError_t e =
      pa::launch_merge(v_states, v_dtype, s_states, num_states, rows, head_dim, rows * head_dim,
                       rows, v_out, out_dtype, s_out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int paged_attn_check_tables(const int32_t* h_indptr, const int32_t* h_indices,
                            const int32_t* h_last_page_len, int32_t num_kv_batches,
                            int32_t num_pool_pages, int32_t page_size) {
  if (!h_indptr || !h_last_page_len) return PA_ERR_NULL;
  if (num_kv_batches < 1 || num_pool_pages < 0 || page_size < 1) return PA_ERR_SHAPE;
  if (h_indptr[0] != 0) return PA_ERR_SHAPE;
  for (int b = 0; b < num_kv_batches; ++b) {
    const int n = h_indptr[b + 1] - h_indptr[b];
    if (n < 0) return PA_ERR_SHAPE;
    if (n > 0 && (h_last_page_len[b] < 1 || h_last_page_len[b] > page_size)) return PA_ERR_SHAPE;
  }
  const int total = h_indptr[num_kv_batches];
  if (total > 0 && !h_indices) return PA_ERR_NULL;
  for (int i = 0; i < total; ++i)
    if (h_indices[i] < 0 || h_indices[i] >= num_pool_pages) return PA_ERR_SHAPE;
  return PA_OK;
}

}  // extern "C"
