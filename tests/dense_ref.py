"""Brute-force dense attention in torch float64 — an independent check of the oracle.

It decodes the storage codes with torch's own dtype casts (not the oracle's
decoders), gathers each KV batch's rows with a vectorised strided view of the
cache (not the oracle's scalar page walk), and computes scores, the mask,
softmax and log-sum-exp with torch library routines on dense tensors.
"""
from __future__ import annotations

import numpy as np
import torch

from paged_kv_attention_prefill_amd import workloads as W


def decoded(raw: np.ndarray, dtype: int) -> torch.Tensor:
    return W.as_torch(raw.reshape(-1), dtype).to(torch.float64)


def logical_cache(flat: torch.Tensor, stride, pool, P, H, D) -> torch.Tensor:
    return torch.as_strided(flat, size=(pool, P, H, D), stride=(stride[0], stride[1], stride[2], 1))


def dense_attention(w: W.Workload, split=None, causal=None):
    """Returns O [total_q, Hq, Dvo], LSE [total_q, Hq], MAX [total_q, Hq] (float64).

    ``split=(c, S)`` restricts every row to the tokens of pages
    [floor(c*n/S), floor((c+1)*n/S)) of its KV batch.
    """
    caus = w.causal if causal is None else causal
    q = decoded(w.q, w.q_dtype).reshape(w.total_q, w.num_qo_heads, w.head_dim_qk) * w.q_scale
    kflat = decoded(w.k, w.kv_dtype)
    kc = logical_cache(kflat, w.k_stride, w.num_pool_pages, w.page_size, w.num_kv_heads,
                       w.head_dim_qk)
    if w.v is None:
        vc = kc[..., : w.head_dim_vo]
    else:
        vc = logical_cache(decoded(w.v, w.kv_dtype), w.v_stride, w.num_pool_pages, w.page_size,
                           w.num_kv_heads, w.head_dim_vo)
    G = w.num_qo_heads // w.num_kv_heads
    O = torch.zeros(w.total_q, w.num_qo_heads, w.head_dim_vo, dtype=torch.float64)
    LSE = torch.full((w.total_q, w.num_qo_heads), -float("inf"), dtype=torch.float64)
    MX = torch.full((w.total_q, w.num_qo_heads), -float("inf"), dtype=torch.float64)
    for b in range(w.batch):
        kb = 0 if w.kv_broadcast else b
        p0, p1 = int(w.kv_indptr[kb]), int(w.kv_indptr[kb + 1])
        n = p1 - p0
        L = 0 if n == 0 else (n - 1) * w.page_size + int(w.kv_last_page_len[kb])
        t0, t1 = int(w.qo_indptr[b]), int(w.qo_indptr[b + 1])
        qb = t1 - t0
        if qb == 0 or L == 0:
            continue
        pages = torch.from_numpy(w.kv_indices[p0:p1].astype(np.int64))
        K = kc[pages].reshape(n * w.page_size, w.num_kv_heads, w.head_dim_qk)[:L] * w.k_scale
        V = vc[pages].reshape(n * w.page_size, w.num_kv_heads, w.head_dim_vo)[:L] * w.v_scale
        K = K.repeat_interleave(G, dim=1)  # [L, Hq, D]: query head h reads KV head h // G
        V = V.repeat_interleave(G, dim=1)
        Q = q[t0:t1]  # [qb, Hq, D]
        scores = torch.matmul(Q.permute(1, 0, 2), K.permute(1, 2, 0).contiguous()) * w.sm_scale
        j = torch.arange(L).view(1, 1, L)
        i = torch.arange(qb).view(1, qb, 1)
        allowed = torch.ones(1, qb, L, dtype=torch.bool)
        if caus:
            allowed = allowed & (j <= (L - qb) + i)
        if split is not None:
            c, S = split
            lo, hi = (c * n // S) * w.page_size, ((c + 1) * n // S) * w.page_size
            allowed = allowed & (j >= lo) & (j < hi)
        scores = scores.masked_fill(~allowed, -float("inf"))
        lse = torch.logsumexp(scores, dim=-1)          # [Hq, qb]
        mx = scores.amax(dim=-1)
        p = torch.softmax(scores, dim=-1)
        p = torch.nan_to_num(p, nan=0.0)               # fully masked rows
        o = torch.matmul(p, V.permute(1, 0, 2).contiguous())  # [Hq, qb, Dvo]
        O[t0:t1] = o.permute(1, 0, 2)
        LSE[t0:t1] = lse.T
        MX[t0:t1] = mx.T
    return O.numpy(), LSE.numpy(), MX.numpy()
