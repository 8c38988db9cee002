"""Pins of the CPU oracle against things other than itself (no GPU needed).

* dtype decoders vs torch / numpy casts over every code;
* brute-force dense attention (torch float64, vectorised gather) on small
  instances of every workload family, incl. causal, ragged, empty rows, HND and
  mixed layouts, fp8 shared latent KV and broadcast;
* closed forms: constant V, zero K, single token, fresh causal prefill,
  one-hot V (rows of P sum to one and vanish outside the allowed set);
* invariants named by the pages: split partials merged by LSE equal the unsplit
  result; relabelling physical pages changes nothing; broadcast KV equals
  replicated KV; GQA equals MHA with repeated KV heads; a shared latent row
  equals a separate V copy;
* the merge formula's special cases.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

from oracle import oracle as OR
from paged_kv_attention_prefill_amd import workloads as W
from dense_ref import dense_attention

RT, AT = 1e-11, 1e-12


def close(a, b, rtol=RT, atol=AT):
    np.testing.assert_allclose(a, b, rtol=rtol, atol=atol)


def small_cases():
    return {
        "c1": lambda: W.config1(),
        "c2_small": lambda: W.config2(batch=3, min_len=1, max_len=70),
        "c2_small_hnd": lambda: W.config2(batch=2, min_len=20, max_len=60, num_qo_heads=16,
                                          num_kv_heads=4, k_layout="HND", v_layout="HND"),
        "c2_small_mixed": lambda: W.config2(batch=2, min_len=20, max_len=60, num_qo_heads=16,
                                            num_kv_heads=4, k_layout="NHD", v_layout="HND"),
        "c3_small": lambda: W.config3(batch=3, min_q=1, max_q=40, max_prefix=50),
        "c4_small_bf16": lambda: W.config4(num_heads=16, q_len=2, batch=2, min_len=1, max_len=150),
        "c4_small_fp8": lambda: W.config4(num_heads=16, q_len=4, kv_dtype=W.DT_FP8, batch=3,
                                          min_len=1, max_len=150),
        "c4_small_fp8q": lambda: W.config4(num_heads=16, q_len=2, kv_dtype=W.DT_FP8,
                                           q_dtype=W.DT_FP8, batch=3, min_len=1, max_len=120),
        "c5_small": lambda: W.config5(num_queries=3, kv_len=300, num_kv_splits=4),
        "sparse_mla_bf16": lambda: W.config_sparse(num_heads=16, kv_lens=[1, 40, 129], pool_factor=3),
        "sparse_mla_fp8": lambda: W.config_sparse(num_heads=8, kv_dtype=W.DT_FP8, kv_lens=[3, 77],
                                                  pool_factor=2),
        "sparse_gqa": lambda: W.config_sparse(mla=False, num_qo_heads=8, num_kv_heads=2,
                                              kv_lens=[5, 70, 33], pool_factor=4),
    }


# ---------------------------------------------------------------- decoders

def test_decode_fp8_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = OR.decode(codes, W.DT_FP8)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    m = ~np.isnan(ref)
    np.testing.assert_array_equal(got[m], ref[m])
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and got[0x7E] == 448.0
    assert got[1] == 2.0 ** -9  # smallest subnormal (1/8)*2^-6


def test_decode_bf16_all_codes():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = OR.decode(codes, W.DT_BF16)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    m = ~np.isnan(ref)
    np.testing.assert_array_equal(got[m], ref[m])


def test_decode_f16_all_codes():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = codes.view(np.float16).astype(np.float64)
    got = OR.decode(codes, W.DT_F16)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    m = ~np.isnan(ref)
    np.testing.assert_array_equal(got[m], ref[m])


def test_fp8_encoder_clamps():
    raw = W.round_to_storage(np.array([500.0, -1000.0, 300.0, 0.0], np.float32), W.DT_FP8)
    got = OR.decode(raw, W.DT_FP8)
    np.testing.assert_array_equal(got, [448.0, -448.0, 288.0, 0.0])


# ---------------------------------------------------------- brute force

@pytest.mark.parametrize("name", list(small_cases()))
def test_oracle_matches_dense(name):
    w = small_cases()[name]()
    o, lse, mx = OR.attention(w, num_kv_splits=1)
    ro, rl, rm = dense_attention(w)
    close(o, ro)
    close(lse, rl)
    close(mx, rm)
    assert np.isfinite(o).all()


@pytest.mark.parametrize("name,S", [("c2_small", 3), ("c3_small", 2), ("c5_small", 4),
                                    ("c4_small_fp8", 3)])
def test_oracle_split_partials_match_dense(name, S):
    w = small_cases()[name]()
    o, lse, mx = OR.attention(w, num_kv_splits=S)
    for c in range(S):
        ro, rl, rm = dense_attention(w, split=(c, S))
        close(o[c], ro)
        close(lse[c], rl)
        close(mx[c], rm)


def test_oracle_row_subset():
    w = small_cases()["c3_small"]()
    o, lse, mx = OR.attention(w)
    rows = np.array([0, 5, w.total_q * w.num_qo_heads - 1, 17], dtype=np.int64)
    so, sl, sm = OR.attention(w, rows=rows)
    flat_o = o.reshape(-1, w.head_dim_vo)
    np.testing.assert_array_equal(so, flat_o[rows])
    np.testing.assert_array_equal(sl, lse.reshape(-1)[rows])


def test_empty_rows_are_zero_and_neg_inf():
    # q_len 4 with KV lengths down to 1: causal rows i with L - 4 + i < 0 see nothing
    w = W.config4(num_heads=16, q_len=4, batch=6, min_len=1, max_len=3)
    o, lse, mx = OR.attention(w)
    L = w.kv_lens
    for b in range(w.batch):
        for i in range(4):
            t = b * 4 + i
            if L[b] - 4 + i < 0:
                assert (o[t] == 0).all() and np.isneginf(lse[t]).all() and np.isneginf(mx[t]).all()
            else:
                assert np.isfinite(lse[t]).all()


# ---------------------------------------------------------- closed forms

def _set_v_const(w, c):
    v = np.empty_like(w.v)
    v[...] = W.round_to_storage(np.array([c], np.float32), w.kv_dtype)[0]
    return dataclasses.replace(w, v=v)


@pytest.mark.parametrize("name", ["c1", "c3_small", "c5_small"])
def test_constant_v_gives_constant_o(name):
    w = _set_v_const(small_cases()[name](), 0.75)
    o, lse, _ = OR.attention(w, num_kv_splits=1)
    finite = np.isfinite(lse)
    close(o[finite], np.full_like(o[finite], 0.75), rtol=1e-15, atol=1e-15)


def _gather_v(w, b):
    """Logical V rows of KV batch b, [L, Hkv, Dvo] float64 (vectorised gather)."""
    from dense_ref import decoded, logical_cache
    flat = decoded(w.v if w.v is not None else w.k, w.kv_dtype)
    st = w.v_stride if w.v is not None else w.k_stride
    D = w.head_dim_vo if w.v is not None else w.head_dim_qk
    vc = logical_cache(flat, st, w.num_pool_pages, w.page_size, w.num_kv_heads, D)
    p0, p1 = int(w.kv_indptr[b]), int(w.kv_indptr[b + 1])
    L = int(w.kv_lens[b])
    pages = torch.from_numpy(w.kv_indices[p0:p1].astype(np.int64))
    return (vc[pages].reshape(-1, w.num_kv_heads, D)[:L, :, : w.head_dim_vo] * w.v_scale).numpy()


def test_zero_k_gives_mean_v_and_log_count():
    w = small_cases()["c3_small"]()
    w = dataclasses.replace(w, k=np.zeros_like(w.k))
    o, lse, mx = OR.attention(w)
    G = w.num_qo_heads // w.num_kv_heads
    for b in range(w.batch):
        V = _gather_v(w, b)
        L = V.shape[0]
        qb = int(w.qo_indptr[b + 1] - w.qo_indptr[b])
        for i in range(qb):
            t = int(w.qo_indptr[b]) + i
            n_allowed = L - qb + i + 1
            for h in range(w.num_qo_heads):
                close(o[t, h], V[:n_allowed, h // G].mean(axis=0), rtol=1e-13, atol=1e-14)
                assert lse[t, h] == pytest.approx(math.log(n_allowed), abs=1e-13)
                assert mx[t, h] == 0.0


def test_single_token_gives_that_v():
    w = W.config2(batch=4, min_len=1, max_len=1, num_qo_heads=8, num_kv_heads=2)
    o, lse, mx = OR.attention(w)
    for b in range(w.batch):
        V = _gather_v(w, b)
        for h in range(8):
            np.testing.assert_array_equal(o[b, h], V[0, h // 4])
    np.testing.assert_array_equal(lse, mx)


def test_fresh_causal_prefill_first_query_sees_first_token():
    w = W.config3(batch=3, min_q=2, max_q=30, max_prefix=0)
    o, lse, mx = OR.attention(w)
    G = w.num_qo_heads // w.num_kv_heads
    for b in range(w.batch):
        V = _gather_v(w, b)
        t = int(w.qo_indptr[b])
        for h in range(w.num_qo_heads):
            np.testing.assert_array_equal(o[t, h], V[0, h // G])
        assert (lse[t] == mx[t]).all()


@pytest.mark.parametrize("causal", [False, True])
def test_one_hot_v_rows_sum_to_one(causal):
    # V_j = e_j: O[d] is the softmax weight of token d, so rows of P are visible
    rng = np.random.default_rng(7)
    q_lens = [3, 5, 1]
    kv_lens = [20, 64, 9]
    w = W.build(rng, 7, "onehot", q_lens=q_lens, kv_lens=kv_lens, num_qo_heads=4,
                num_kv_heads=2, head_dim_qk=32, head_dim_vo=64, page_size=8,
                q_dtype=W.DT_F32, kv_dtype=W.DT_F32, causal=causal, pool_pages=20,
                uniform_q_len=False)
    v = np.full_like(w.v, np.nan)
    v4 = v.reshape(w.num_pool_pages, 8, 2, 64)
    for b in range(3):
        pages = w.kv_indices[w.kv_indptr[b]:w.kv_indptr[b + 1]]
        for j in range(kv_lens[b]):
            v4[pages[j // 8], j % 8, :, :] = 0.0
            v4[pages[j // 8], j % 8, :, j] = 1.0
    w = dataclasses.replace(w, v=v)
    o, lse, _ = OR.attention(w)
    assert np.isfinite(o).all()
    close(o.sum(axis=-1), np.ones(o.shape[:2]), rtol=0, atol=1e-14)
    for b in range(3):
        for i in range(q_lens[b]):
            t = int(w.qo_indptr[b]) + i
            last = kv_lens[b] - q_lens[b] + i if causal else kv_lens[b] - 1
            assert (o[t, :, : last + 1] > 0).all()
            assert (o[t, :, last + 1:] == 0).all()


# ---------------------------------------------------------- invariants

@pytest.mark.parametrize("name,S", [("c2_small", 3), ("c3_small", 4), ("c5_small", 4),
                                    ("c4_small_bf16", 2), ("c4_small_fp8", 5)])
def test_split_then_merge_equals_unsplit(name, S):
    w = small_cases()[name]()
    o, lse, _ = OR.attention(w, num_kv_splits=1)
    po, pl, _ = OR.attention(w, num_kv_splits=S)
    rows = o.shape[0] * o.shape[1]
    mo, ml = OR.merge_states(po.reshape(S, rows, -1), pl.reshape(S, rows))
    close(mo, o.reshape(rows, -1))
    close(ml, lse.reshape(rows))


def select_subset(w, keep):
    """The same queries over a subset of each query's selected token slots
    (page size 1): ``keep(b, i)`` says whether the i-th selected slot of query
    batch b stays."""
    assert w.page_size == 1
    idx, indptr = [], [0]
    for b in range(w.batch):
        sel = w.kv_indices[w.kv_indptr[b]:w.kv_indptr[b + 1]]
        part = [int(x) for i, x in enumerate(sel) if keep(b, i)]
        idx += part
        indptr.append(len(idx))
    n = np.diff(indptr)
    return dataclasses.replace(w, kv_indices=np.asarray(idx, dtype=np.int32),
                               kv_indptr=np.asarray(indptr, dtype=np.int32),
                               kv_last_page_len=np.where(n > 0, 1, 0).astype(np.int32),
                               kv_lens=n.astype(np.int64))


@pytest.mark.parametrize("name", ["sparse_mla_bf16", "sparse_mla_fp8", "sparse_gqa"])
def test_sparse_selection_routed_halves_merge_to_whole(name):
    """Partial attention over two disjoint halves of every query's selected rows
    (interleaved, as two holders of a sparsely selected cache would see them),
    merged through their LSE, equals attention over the whole selection; a
    query whose half is empty contributes a -inf state."""
    w = small_cases()[name]()
    o, lse, _ = OR.attention(w)
    halves = [select_subset(w, lambda b, i, r=r: i % 2 == r) for r in (0, 1)]
    parts = [OR.attention(h) for h in halves]
    rows = o.shape[0] * o.shape[1]
    po = np.stack([p[0].reshape(rows, -1) for p in parts])
    pl = np.stack([p[1].reshape(rows) for p in parts])
    if (w.kv_lens == 1).any():
        assert np.isneginf(pl[1]).any()  # a one-row selection leaves half 1 empty
    mo, ml = OR.merge_states(po, pl)
    close(mo, o.reshape(rows, -1))
    close(ml, lse.reshape(rows))


def _permute_pages(w, seed):
    rng = np.random.default_rng(seed)
    pi = rng.permutation(w.num_pool_pages)
    def move(arr, stride):
        out = np.empty_like(arr)
        page_elems = stride[0]
        a = arr.reshape(w.num_pool_pages, page_elems) if stride[0] * w.num_pool_pages == arr.size \
            else None
        assert a is not None
        o2 = out.reshape(w.num_pool_pages, page_elems)
        o2[pi] = a
        return out
    k = move(w.k, w.k_stride)
    v = None if w.v is None else move(w.v, w.v_stride)
    return dataclasses.replace(w, k=k, v=v, kv_indices=pi[w.kv_indices].astype(np.int32))


@pytest.mark.parametrize("name", ["c1", "c3_small", "c4_small_fp8", "c5_small"])
def test_page_permutation_invariance_bitwise(name):
    w = small_cases()[name]()
    o, lse, mx = OR.attention(w)
    o2, lse2, mx2 = OR.attention(_permute_pages(w, 11))
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)
    np.testing.assert_array_equal(mx, mx2)


def test_broadcast_equals_replicated():
    w = small_cases()["c5_small"]()
    r = W.replicate_broadcast(w)
    for S in (1, 4):
        a = OR.attention(w, num_kv_splits=S)
        b = OR.attention(r, num_kv_splits=S)
        for x, y in zip(a, b):
            np.testing.assert_array_equal(x, y)


def test_gqa_equals_mha_with_repeated_heads():
    w = W.config2(batch=3, min_len=5, max_len=90, num_qo_heads=8, num_kv_heads=2)
    G = 4
    def rep(arr):
        a = arr.reshape(w.num_pool_pages, w.page_size, 2, 128)
        return np.ascontiguousarray(np.repeat(a, G, axis=2))
    st = (w.page_size * 8 * 128, 8 * 128, 128)
    m = dataclasses.replace(w, k=rep(w.k), v=rep(w.v), num_kv_heads=8, k_stride=st, v_stride=st)
    for x, y in zip(OR.attention(w), OR.attention(m)):
        np.testing.assert_array_equal(x, y)


def test_shared_latent_equals_separate_v_copy():
    w = small_cases()["c4_small_fp8"]()
    k4 = w.k.reshape(w.num_pool_pages, w.page_size, 1, 576)
    v = np.ascontiguousarray(k4[..., :512])
    s = dataclasses.replace(w, v=v, v_stride=(w.page_size * 512, 512, 512))
    for x, y in zip(OR.attention(w), OR.attention(s)):
        np.testing.assert_array_equal(x, y)


# ---------------------------------------------------------- merge formula

def test_merge_special_cases():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((1, 5, 8))
    s = rng.standard_normal((1, 5))
    vo, so = OR.merge_states(v, s)
    np.testing.assert_array_equal(vo, v[0])
    np.testing.assert_array_equal(so, s[0])
    # equal LSEs: plain average, LSE + ln 2
    v2 = rng.standard_normal((2, 4, 8))
    s2 = np.array([[0.5, -3.0, 7.0, 0.0]] * 2)
    vo, so = OR.merge_states(v2, s2)
    close(vo, v2.mean(axis=0), rtol=1e-15, atol=1e-15)
    close(so, s2[0] + math.log(2.0), rtol=1e-15, atol=1e-15)
    # a -inf state carries no weight; all -inf -> 0 and -inf (no NaN)
    s3 = np.array([[1.0, -np.inf], [-np.inf, -np.inf]])
    v3 = rng.standard_normal((2, 2, 3))
    vo, so = OR.merge_states(v3, s3)
    np.testing.assert_array_equal(vo[0], v3[0, 0])
    assert so[0] == 1.0
    assert (vo[1] == 0).all() and np.isneginf(so[1])
    # weights follow exp(LSE): ln(e^2 + e^0) = 2 + ln(1 + e^-2)
    v4 = np.array([[[1.0]], [[0.0]]])
    s4 = np.array([[2.0], [0.0]])
    vo, so = OR.merge_states(v4, s4)
    assert vo[0, 0] == pytest.approx(1.0 / (1.0 + math.exp(-2.0)), rel=1e-15)
    assert so[0] == pytest.approx(2.0 + math.log1p(math.exp(-2.0)), rel=1e-15)


# ------------------------------------------- score jumps and non-positive scales

def _mla_small(seed, heads, q_len, kv_lens, dt=W.DT_BF16, **kw):
    rng = np.random.default_rng(seed)
    return W.build(rng, seed, "mla_small", q_lens=[q_len] * len(kv_lens), kv_lens=kv_lens,
                   num_qo_heads=heads, num_kv_heads=1, head_dim_qk=576, head_dim_vo=512,
                   page_size=16, q_dtype=W.DT_BF16, kv_dtype=dt, shared_kv=True, causal=True,
                   sm_scale=1.0 / math.sqrt(192.0), **kw)


def edge_cases():
    return {
        "jump_gqa": lambda: W.config2(batch=3, min_len=1, max_len=90, k_late_gain=(32.0, 0, 128)),
        "jump_prefill": lambda: W.config3(batch=2, min_q=1, max_q=40, max_prefix=60,
                                          k_late_gain=(32.0, 0, 128)),
        "jump_mla_fp8": lambda: _mla_small(61, 8, 2, [1, 50, 130], dt=W.DT_FP8,
                                           k_late_gain=(32.0, 512, 576)),
        "zero_scale": lambda: dataclasses.replace(W.config2(batch=3, min_len=1, max_len=70),
                                                  sm_scale=0.0),
        "negative_scale": lambda: dataclasses.replace(
            W.config3(batch=2, min_q=1, max_q=30, max_prefix=40), sm_scale=-0.3),
        "zero_k_scale_fp8": lambda: dataclasses.replace(
            _mla_small(62, 4, 2, [2, 70], dt=W.DT_FP8), k_scale=0.0),
        "f16_q_fp8_kv": lambda: W.build(np.random.default_rng(63), 63, "f16xfp8", q_lens=[1, 1],
                                        kv_lens=[9, 40], num_qo_heads=4, num_kv_heads=2,
                                        head_dim_qk=64, head_dim_vo=64, page_size=16,
                                        q_dtype=W.DT_F16, kv_dtype=W.DT_FP8),
    }


@pytest.mark.parametrize("name", list(edge_cases()))
def test_oracle_matches_dense_edge_cases(name):
    """Large late score jumps (scores spanning far beyond +-60), zero and negative
    score scales, a zero fp8 K scale and f16 queries over fp8 KV: the oracle's
    two-pass softmax against the dense torch reference."""
    w = edge_cases()[name]()
    o, lse, mx = OR.attention(w, num_kv_splits=1)
    ro, rl, rm = dense_attention(w)
    close(o, ro)
    close(lse, rl)
    close(mx, rm)
    assert np.isfinite(o).all()


def test_zero_scale_closed_form():
    """sm_scale = 0: every allowed score is 0, so O is the plain mean of V over the
    allowed set, LSE = ln|J| and max = 0."""
    w = edge_cases()["zero_scale"]()
    o, lse, mx = OR.attention(w)
    Hq, G = w.num_qo_heads, w.num_qo_heads // w.num_kv_heads
    v = OR.decode(w.v, w.kv_dtype).reshape(w.num_pool_pages, w.page_size, w.num_kv_heads, -1)
    for b in range(w.batch):
        L = int(w.kv_lens[b])
        pages = w.kv_indices[w.kv_indptr[b]:w.kv_indptr[b + 1]]
        rows = v[pages].reshape(-1, w.num_kv_heads, w.head_dim_vo)[:L]
        for h in range(Hq):
            close(o[b, h], rows[:, h // G].mean(axis=0))
            assert abs(lse[b, h] - math.log(L)) < 1e-12 and mx[b, h] == 0.0
