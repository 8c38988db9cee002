"""Why the fp8-query many-rows kernel splits P into two e4m3 terms (CPU only).

That kernel multiplies P.V on the fp8 matrix cores.  This test emulates, in
float64, what reaches those MFMAs under two ways of rounding P, on a score-jump
workload of the GPU parity suite, and compares the result with the oracle:

* P rounded to one e4m3 term (4 significant bits) misses the fp8-KV bar of
  6e-2 on O;
* P = hi + lo / 16, hi = e4m3(P), lo = e4m3(16 (P - hi)) -- the kernel's form --
  stays an order of magnitude inside it.

The emulation follows the kernel's order of work: 128-token tiles from the
first token, a reference max moved only when a tile's max exceeds it by more
than 8 (log2 units), P = exp2(s - m) with s the scaled score in log2 units, the
row sum over the unrounded P, O = sum(P_rounded v) / sum(P) times the V scale.
"""
import math

import numpy as np
import torch

from dense_ref import decoded
from oracle import oracle as OR
from paged_kv_attention_prefill_amd import workloads as W

TILE = 128
REBASE = 8.0


def e4m3(x: np.ndarray) -> np.ndarray:
    """Round to the nearest e4m3fn value (every value here is below 448)."""
    return torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def one_term(p):
    return e4m3(p)


def two_terms(p):
    hi = e4m3(p)
    return hi + e4m3(16.0 * (p - hi)) / 16.0


def emulate(w: W.Workload, round_p) -> np.ndarray:
    H, ql, P = w.num_qo_heads, w.q_len, w.page_size
    q = decoded(w.q, w.q_dtype).double().numpy().reshape(-1, H, w.head_dim_qk)
    k = decoded(w.k, w.kv_dtype).double().numpy().reshape(w.num_pool_pages, P, w.head_dim_qk)
    scale = w.sm_scale * w.k_scale * w.q_scale / math.log(2.0)
    out = np.zeros((len(w.kv_lens) * ql * H, w.head_dim_vo))
    for b, L in enumerate(int(x) for x in w.kv_lens):
        if L == 0:
            continue
        pages = w.kv_indices[w.kv_indptr[b]:w.kv_indptr[b + 1]]
        K = k[pages].reshape(-1, w.head_dim_qk)[:L]
        V = K[:, :w.head_dim_vo]
        x = (q[b * ql:(b + 1) * ql].reshape(ql * H, -1) @ K.T) * scale
        r = np.arange(ql * H)
        allowed = np.arange(L)[None, :] < (L - ql + r // H + 1)[:, None]
        x = np.where(allowed, x, -np.inf)
        m = np.full((ql * H, 1), -np.inf)
        lsum = np.zeros((ql * H, 1))
        acc = np.zeros((ql * H, w.head_dim_vo))
        for j0 in range(0, L, TILE):
            xs = x[:, j0:j0 + TILE]
            tmax = xs.max(axis=1, keepdims=True)
            grow = tmax > m + REBASE
            mnew = np.where(grow, tmax, m)
            alpha = np.where(grow & np.isfinite(m), np.exp2(m - np.where(np.isfinite(mnew), mnew, 0.0)),
                             np.where(grow, 0.0, 1.0))
            acc *= alpha
            lsum *= alpha
            m = mnew
            p = np.exp2(xs - np.where(np.isfinite(m), m, 0.0))
            lsum += p.sum(axis=1, keepdims=True)
            acc += round_p(p) @ V[j0:j0 + TILE]
        out[b * ql * H:(b + 1) * ql * H] = acc / lsum * w.v_scale
    return out


def test_p_in_two_e4m3_terms_meets_the_fp8_bar_where_one_term_does_not():
    # the score-jump case of the fp8-query many-rows kernel in tests/test_gpu_edges.py
    rng = np.random.default_rng(410)
    w = W.build(rng, 410, "mla h128 q4 p64", q_lens=[4, 4], kv_lens=[5, 1500], num_qo_heads=128,
                num_kv_heads=1, head_dim_qk=576, head_dim_vo=512, page_size=64,
                q_dtype=W.DT_FP8, kv_dtype=W.DT_FP8, shared_kv=True, causal=True,
                sm_scale=1.0 / np.sqrt(192.0), k_late_gain=(8.0, 512, 576))
    o_ref, _, _ = OR.attention(w, num_kv_splits=1)
    o_ref = o_ref.reshape(-1, w.head_dim_vo)
    err_one = np.abs(emulate(w, one_term) - o_ref).max()
    err_two = np.abs(emulate(w, two_terms) - o_ref).max()
    assert err_one > 6e-2, err_one
    assert err_two < 1e-2, err_two
