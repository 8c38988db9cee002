"""Comparison helpers for the GPU parity tests (HIP path vs the CPU oracle)."""
from __future__ import annotations

import numpy as np

from paged_kv_attention_prefill_amd import workloads as W

# max abs error bars: fp32 1e-5 on O and LSE; bf16/fp16 2e-2 on O, 1e-2 on LSE;
# fp8 KV 6e-2 on O (LSE: the 16-bit bar, 1e-2, since none is stated for fp8)
def tolerances(w: W.Workload):
    if w.kv_dtype == W.DT_FP8:
        return 6e-2, 1e-2
    if w.q_dtype == W.DT_F32 and w.kv_dtype == W.DT_F32:
        return 1e-5, 1e-5
    return 2e-2, 1e-2


def to64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_rows(w, o_gpu, lse_gpu, o_ref, lse_ref, mx_gpu=None, mx_ref=None, label=""):
    """o_*: [rows, Dvo], lse_*: [rows] (numpy float64).  Asserts the bars and
    returns a dict of error statistics."""
    tol_o, tol_l = tolerances(w)
    o_gpu = o_gpu.reshape(-1, w.head_dim_vo)
    o_ref = o_ref.reshape(-1, w.head_dim_vo)
    lse_gpu = lse_gpu.reshape(-1)
    lse_ref = lse_ref.reshape(-1)
    assert o_gpu.shape == o_ref.shape, (o_gpu.shape, o_ref.shape)
    assert np.isfinite(o_gpu).all(), f"{label}: non-finite O from the GPU"
    empty = np.isneginf(lse_ref)
    np.testing.assert_array_equal(np.isneginf(lse_gpu), empty, err_msg=f"{label}: empty rows")
    assert (o_gpu[empty] == 0).all(), f"{label}: empty rows must have O = 0"
    err_o = np.abs(o_gpu - o_ref).max() if o_ref.size else 0.0
    fin = ~empty
    err_l = np.abs(lse_gpu[fin] - lse_ref[fin]).max() if fin.any() else 0.0
    stats = dict(label=label, max_err_o=float(err_o), max_err_lse=float(err_l),
                 mean_err_o=float(np.abs(o_gpu - o_ref).mean()) if o_ref.size else 0.0,
                 rms_o=float(np.sqrt((o_ref ** 2).mean())) if o_ref.size else 0.0)
    assert err_o <= tol_o, f"{label}: max |dO| {err_o:.3g} > {tol_o}"
    assert err_l <= tol_l, f"{label}: max |dLSE| {err_l:.3g} > {tol_l}"
    if mx_gpu is not None and mx_ref is not None:
        mx_gpu = mx_gpu.reshape(-1)
        mx_ref = mx_ref.reshape(-1)
        np.testing.assert_array_equal(np.isneginf(mx_gpu), np.isneginf(mx_ref))
        err_m = np.abs(mx_gpu[fin] - mx_ref[fin]).max() if fin.any() else 0.0
        stats["max_err_max"] = float(err_m)
        assert err_m <= tol_l, f"{label}: max |dMAX| {err_m:.3g} > {tol_l}"
    print(stats, flush=True)
    return stats


def sample_rows(w: W.Workload, n: int, seed: int = 0) -> np.ndarray:
    """Row ids (t*Hq + h) for sampled parity: random rows plus the first and last
    query token of every batch (ragged ends), all heads of the very last token."""
    rng = np.random.default_rng(seed)
    total = w.total_q * w.num_qo_heads
    rows = set(rng.choice(total, size=min(n, total), replace=False).tolist())
    Hq = w.num_qo_heads
    for b in range(w.batch):
        for t in (int(w.qo_indptr[b]), int(w.qo_indptr[b + 1]) - 1):
            if t >= int(w.qo_indptr[b]):
                rows.add(t * Hq + int(rng.integers(Hq)))
    t = w.total_q - 1
    rows.update(t * Hq + h for h in range(Hq))
    return np.array(sorted(rows), dtype=np.int64)
