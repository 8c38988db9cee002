/*
 * CPU oracle for batched attention over a paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * bench's CPU-baseline leg may load this code; the product path never does.
 * It shares no source, header, table or helper with the HIP library: it has
 * its own dtype decoders and its own page-table walk.
 *
 * What it computes (plain definition, fp64 throughout, two-pass softmax):
 *
 *   Paged KV cache (FlashInfer PR #4736 analysis, introduction and code
 *   section 1, the paged_kv_t constructor): KV batch kb owns pages
 *   kv_indices[kv_indptr[kb] .. kv_indptr[kb+1]); token j of it lives in page
 *   kv_indices[kv_indptr[kb] + j / P], slot j % P.  K and V carry independent
 *   element strides (page, slot, head) (same page, code section 1 "After").
 *   L = (n-1)*P + kv_last_page_len[kb] for n >= 1 pages, 0 otherwise.
 *
 *   KV batch broadcast (PyTorch 2.14 MPS FlexAttention post, introduction):
 *   with kv_broadcast every query batch reads KV batch 0, no copy.
 *
 *   For query token i of query batch b (q_b tokens), query head h,
 *   KV head g = h / (Hq/Hkv), allowed set
 *       J = { j : 0 <= j < L  and  (!causal or j <= L - q_b + i) }
 *   s_j = sm_scale * sum_{d<Dqk} q_scale * Q[d] * k_scale * K_j[d]
 *   (q_scale and k_scale: per-tensor scales of fp8 codes, 1 otherwise)
 *   m   = max_j s_j,  Z = sum_j exp(s_j - m)
 *   O   = sum_j exp(s_j - m) * v_scale * V_j[:Dvo] / Z,  LSE = m + ln Z,  max = m
 *   Empty J: O = 0, LSE = -inf, max = -inf.
 *   This is what the online softmax of the pages (the cross-instance "Move
 *   the Query, Not the Cache" summary, method section, and the SM110 XQA
 *   split kernel, kernel-design section) reaches in exact arithmetic.
 *
 *   Shared latent KV (FlashInfer PR #3309 analysis, code section 1: MLA shares
 *   one KV across all heads and queries): the caller passes the same buffer
 *   and strides for K and V; V is the first Dvo dims of each K row.
 *
 *   Split KV (num_kv_splits = S): partial state c restricts J to the tokens of
 *   pages [floor(c*n/S), floor((c+1)*n/S)) of the KV batch.
 *
 *   Merge (cross-instance summary, method section: partial attention results
 *   merged through online softmax): m = max_c LSE_c, w_c = exp(LSE_c - m),
 *   O = sum_c w_c O_c / sum_c w_c, LSE = m + ln sum_c w_c; states with
 *   LSE = -inf carry no weight; all -inf gives O = 0, LSE = -inf.
 *
 * fp8 (KV caches, and queries with their own scale) is OCP e4m3fn: sign,
 * 4-bit exponent (bias 7), 3-bit mantissa,
 * subnormals (m/8)*2^-6, S.1111.111 is NaN, no infinities.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2, OR_FP8 = 3 };

static double dec_f16(uint16_t h) {
    int s = h >> 15, e = (h >> 10) & 0x1f, m = h & 0x3ff;
    double v;
    if (e == 0) v = ldexp((double)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp(1.0 + m / 1024.0, e - 15);
    return s ? -v : v;
}

static double dec_bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static double dec_fp8_e4m3fn(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 0xf, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m / 8.0, -6);
    else v = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

static double elem(const void* base, int dt, int64_t idx) {
    switch (dt) {
    case OR_F32: return (double)((const float*)base)[idx];
    case OR_F16: return dec_f16(((const uint16_t*)base)[idx]);
    case OR_BF16: return dec_bf16(((const uint16_t*)base)[idx]);
    case OR_FP8: return dec_fp8_e4m3fn(((const uint8_t*)base)[idx]);
    }
    return NAN;
}

/* decode n codes of dtype dt into doubles (used by tests to pin the decoders) */
void oracle_decode(const void* src, int dt, int64_t n, double* dst) {
    for (int64_t i = 0; i < n; ++i) dst[i] = elem(src, dt, i);
}

static int batch_of(const int32_t* qo_indptr, int batch, int64_t t) {
    int lo = 0, hi = batch - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if ((int64_t)qo_indptr[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

/*
 * Rows are (query token t, query head h) with id r = t*Hq + h, where query
 * tokens are numbered over all batches in qo_indptr order.  rows == NULL
 * computes every row, in id order.  Outputs o[S][nrows][Dvo], lse[S][nrows],
 * mx[S][nrows] (mx may be NULL).  Returns 0, or -1 on a bad argument.
 */
int oracle_paged_attn(const void* q, int q_dtype, double q_scale, const int32_t* qo_indptr, int batch,
                      int num_qo_heads, const void* k, const void* v, int kv_dtype,
                      const int64_t* k_stride, const int64_t* v_stride, int num_kv_heads,
                      int page_size, int head_dim_qk, int head_dim_vo, double k_scale,
                      double v_scale, const int32_t* kv_indptr, const int32_t* kv_indices,
                      const int32_t* kv_last_page_len, int num_kv_batches, int kv_broadcast,
                      int causal, double sm_scale, int num_kv_splits, const int64_t* rows,
                      int64_t num_rows, double* o, double* lse, double* mx, int num_threads) {
    if (!q || !qo_indptr || !k || !v || !kv_indptr || !kv_last_page_len || !o || !lse) return -1;
    if (batch < 1 || num_qo_heads < 1 || num_kv_heads < 1 || page_size < 1) return -1;
    if (num_qo_heads % num_kv_heads) return -1;
    if (num_kv_splits < 1) return -1;
    if (kv_broadcast ? num_kv_batches != 1 : num_kv_batches != batch) return -1;
    const int64_t total_q = qo_indptr[batch];
    const int64_t nrows = rows ? num_rows : total_q * num_qo_heads;
    const int group = num_qo_heads / num_kv_heads;
    const int S = num_kv_splits;
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#else
    (void)num_threads;
#endif

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ri = 0; ri < nrows; ++ri) {
        const int64_t r = rows ? rows[ri] : ri;
        const int64_t t = r / num_qo_heads;
        const int h = (int)(r % num_qo_heads);
        const int b = batch_of(qo_indptr, batch, t);
        const int64_t i = t - qo_indptr[b];
        const int64_t qb = qo_indptr[b + 1] - qo_indptr[b];
        const int kb = kv_broadcast ? 0 : b;
        const int64_t n = kv_indptr[kb + 1] - kv_indptr[kb];
        const int64_t L = n == 0 ? 0 : (n - 1) * page_size + kv_last_page_len[kb];
        const int64_t pos = L - qb + i;
        const int g = h / group;
        const int64_t qoff = (t * num_qo_heads + h) * (int64_t)head_dim_qk;

        double* s = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
        for (int c = 0; c < S; ++c) {
            const int64_t p0 = (int64_t)c * n / S, p1 = (int64_t)(c + 1) * n / S;
            int64_t j0 = p0 * page_size, j1 = p1 * page_size;
            if (j1 > L) j1 = L;
            if (causal && j1 > pos + 1) j1 = pos + 1;
            double* orow = o + ((int64_t)c * nrows + ri) * head_dim_vo;
            double m = -INFINITY;
            for (int64_t j = j0; j < j1; ++j) {
                const int64_t page = kv_indices[kv_indptr[kb] + j / page_size];
                const int64_t kbase = page * k_stride[0] + (j % page_size) * k_stride[1] + g * k_stride[2];
                double acc = 0.0;
                for (int d = 0; d < head_dim_qk; ++d)
                    acc += (q_scale * elem(q, q_dtype, qoff + d)) * (k_scale * elem(k, kv_dtype, kbase + d));
                s[j - j0] = sm_scale * acc;
                if (s[j - j0] > m) m = s[j - j0];
            }
            if (j1 <= j0) {
                for (int d = 0; d < head_dim_vo; ++d) orow[d] = 0.0;
                lse[(int64_t)c * nrows + ri] = -INFINITY;
                if (mx) mx[(int64_t)c * nrows + ri] = -INFINITY;
                continue;
            }
            double z = 0.0;
            for (int d = 0; d < head_dim_vo; ++d) orow[d] = 0.0;
            for (int64_t j = j0; j < j1; ++j) {
                const double p = exp(s[j - j0] - m);
                z += p;
                const int64_t page = kv_indices[kv_indptr[kb] + j / page_size];
                const int64_t vbase = page * v_stride[0] + (j % page_size) * v_stride[1] + g * v_stride[2];
                for (int d = 0; d < head_dim_vo; ++d)
                    orow[d] += p * (v_scale * elem(v, kv_dtype, vbase + d));
            }
            for (int d = 0; d < head_dim_vo; ++d) orow[d] /= z;
            lse[(int64_t)c * nrows + ri] = m + log(z);
            if (mx) mx[(int64_t)c * nrows + ri] = m;
        }
        free(s);
    }
    return 0;
}

/* v[S][rows][D], s[S][rows] -> vo[rows][D], so[rows] (so may be NULL) */
int oracle_merge_states(const double* v, const double* s, int num_states, int64_t rows, int dim,
                        double* vo, double* so) {
    if (!v || !s || !vo || num_states < 1 || rows < 0 || dim < 1) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double m = -INFINITY;
        for (int c = 0; c < num_states; ++c)
            if (s[(int64_t)c * rows + r] > m) m = s[(int64_t)c * rows + r];
        double* out = vo + r * dim;
        for (int d = 0; d < dim; ++d) out[d] = 0.0;
        if (m == -INFINITY) {
            if (so) so[r] = -INFINITY;
            continue;
        }
        double wsum = 0.0;
        for (int c = 0; c < num_states; ++c) {
            const double lc = s[(int64_t)c * rows + r];
            if (lc == -INFINITY) continue;
            const double w = exp(lc - m);
            wsum += w;
            const double* vin = v + ((int64_t)c * rows + r) * dim;
            for (int d = 0; d < dim; ++d) out[d] += w * vin[d];
        }
        for (int d = 0; d < dim; ++d) out[d] /= wsum;
        if (so) so[r] = m + log(wsum);
    }
    return 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
