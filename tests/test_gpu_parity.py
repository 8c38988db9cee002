"""GPU parity: the HIP path through the C ABI vs the CPU oracle, element by
element on the same seeded bytes, at sizes the oracle finishes in seconds that
still span several tiles and ragged tails; plus the invariants and edge cases.
"""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import oracle as OR
from paged_kv_attention_prefill_amd import binding as B
from paged_kv_attention_prefill_amd import runner as R
from paged_kv_attention_prefill_amd import workloads as W
from gpu_check import check_rows, to64, tolerances

pytestmark = pytest.mark.gpu


def small(name):
    return {
        "c1": lambda: W.config1(),
        "c2": lambda: W.config2(batch=6, min_len=1, max_len=1200),
        "c2_hnd": lambda: W.config2(batch=4, min_len=1, max_len=700, k_layout="HND",
                                    v_layout="HND"),
        "c2_mixed": lambda: W.config2(batch=4, min_len=1, max_len=700, k_layout="NHD",
                                      v_layout="HND"),
        "c2_kv2": lambda: W.config2(batch=5, min_len=1, max_len=900, num_qo_heads=16,
                                    num_kv_heads=2),
        "c2_g16": lambda: W.config2(batch=5, min_len=1, max_len=900, num_qo_heads=64,
                                    num_kv_heads=4),
        "c2_q2_causal": lambda: W.build(np.random.default_rng(21), 21, "gqa_q2", q_lens=[2] * 5,
                                        kv_lens=[1, 2, 40, 333, 1000], num_qo_heads=32,
                                        num_kv_heads=4, head_dim_qk=128, head_dim_vo=128,
                                        page_size=16, q_dtype=W.DT_BF16, kv_dtype=W.DT_BF16,
                                        causal=True),
        "c2_d64_f16": lambda: W.build(np.random.default_rng(22), 22, "gqa_d64", q_lens=[1] * 6,
                                      kv_lens=[3, 64, 65, 700, 1500, 2049], num_qo_heads=32,
                                      num_kv_heads=8, head_dim_qk=64, head_dim_vo=64,
                                      page_size=32, q_dtype=W.DT_F16, kv_dtype=W.DT_F16),
        "c2_d256": lambda: W.build(np.random.default_rng(23), 23, "gqa_d256", q_lens=[1] * 4,
                                   kv_lens=[5, 100, 1025, 1800], num_qo_heads=16,
                                   num_kv_heads=4, head_dim_qk=256, head_dim_vo=256,
                                   page_size=16, q_dtype=W.DT_BF16, kv_dtype=W.DT_BF16),
        "c3": lambda: W.config3(batch=3, min_q=1, max_q=300, max_prefix=400),
        "c3_fresh": lambda: W.config3(batch=2, min_q=100, max_q=260, max_prefix=0),
        "c3_p24_g8": lambda: W.build(np.random.default_rng(31), 31, "prefill_p24", q_lens=[1, 70, 200],
                                     kv_lens=[1, 300, 200], num_qo_heads=32, num_kv_heads=4,
                                     head_dim_qk=128, head_dim_vo=128, page_size=24,
                                     q_dtype=W.DT_BF16, kv_dtype=W.DT_BF16, causal=True,
                                     uniform_q_len=False),
        "c3_mha_d64_f16": lambda: W.build(np.random.default_rng(32), 32, "prefill_mha", q_lens=[130, 5],
                                          kv_lens=[900, 5], num_qo_heads=4, num_kv_heads=4,
                                          head_dim_qk=64, head_dim_vo=64, page_size=16,
                                          q_dtype=W.DT_F16, kv_dtype=W.DT_F16, causal=True,
                                          uniform_q_len=False),
        "c3_noncausal_g3": lambda: W.build(np.random.default_rng(33), 33, "prefill_g3", q_lens=[50, 100],
                                           kv_lens=[80, 3000], num_qo_heads=6, num_kv_heads=2,
                                           head_dim_qk=128, head_dim_vo=128, page_size=16,
                                           q_dtype=W.DT_BF16, kv_dtype=W.DT_BF16, causal=False,
                                           uniform_q_len=False),
        "c5_causal_prefill_bcast": lambda: W.build(np.random.default_rng(34), 34, "bcast_prefill",
                                                   q_lens=[3, 40, 1], kv_lens=[500],
                                                   num_qo_heads=32, num_kv_heads=8, head_dim_qk=128,
                                                   head_dim_vo=128, page_size=128, q_dtype=W.DT_F16,
                                                   kv_dtype=W.DT_F16, kv_broadcast=True,
                                                   causal=True, uniform_q_len=False),
        "c5": lambda: W.config5(num_queries=8, kv_len=5000, num_kv_splits=16),
        "c5_long": lambda: W.config5(num_queries=3, kv_len=131072, num_kv_splits=16),
    }[name]()


def c4_small(h, ql, dt):
    return W.config4(num_heads=h, q_len=ql, kv_dtype=dt, batch=3, min_len=1, max_len=900)


def run_and_check(w, label, flags=0, **kw):
    d = R.upload(w)
    res = R.run(d, flags=flags, **kw)
    torch.cuda.synchronize()
    o, lse, mx = OR.attention(w, num_kv_splits=1)
    return check_rows(w, to64(res["o"]), to64(res["lse"]), o, lse,
                      None if res.get("mx") is None else to64(res["mx"]), mx, label=label), res


@pytest.mark.parametrize("name", ["c1", "c2", "c2_hnd", "c2_mixed", "c2_kv2", "c2_g16",
                                  "c2_q2_causal", "c2_d64_f16", "c2_d256", "c3", "c3_fresh",
                                  "c3_p24_g8", "c3_mha_d64_f16", "c3_noncausal_g3",
                                  "c5_causal_prefill_bcast", "c5", "c5_long"])
def test_parity_small(name):
    print(f"case {name}", flush=True)
    run_and_check(small(name), name)


@pytest.mark.parametrize("h", W.C4_HEADS)
@pytest.mark.parametrize("ql", W.C4_QLENS)
@pytest.mark.parametrize("dt", [W.DT_BF16, W.DT_FP8])
def test_parity_mla_small(h, ql, dt):
    label = f"c4 h{h} q{ql} {W.DT_NAMES[dt]}"
    print(label, flush=True)
    run_and_check(c4_small(h, ql, dt), label)


@pytest.mark.parametrize("h", W.C4_HEADS)
@pytest.mark.parametrize("ql", W.C4_QLENS)
def test_parity_mla_fp8_queries(h, ql):
    """fp8 queries over an fp8 cache: Q.K on the fp8 matrix cores for more than
    64 rows per request; the narrow and mid kernels widen the query codes."""
    w = W.config4(num_heads=h, q_len=ql, kv_dtype=W.DT_FP8, q_dtype=W.DT_FP8, batch=3, min_len=1,
                  max_len=900)
    label = f"c4 h{h} q{ql} fp8 KV, fp8 Q"
    print(label, flush=True)
    step = R.prepare(R.upload(w))
    assert step.attention_kernel_name == "mla_decode_mfma_fp8q", step.attention_kernel_name
    run_and_check(w, label)


@pytest.mark.parametrize("heads,q_len,page_size", [(128, 1, 24), (128, 2, 1), (96, 2, 64),
                                                   (144, 1, 7), (128, 4, 96)])
def test_mla_fp8_queries_row_tiles_and_page_sizes(heads, q_len, page_size):
    """The fp8-query many-rows kernel over partial and multiple row tiles and
    page sizes that do not hold whole tiles, with and without internal splits."""
    label = f"MLA fp8 Q h{heads} q{q_len} page {page_size}"
    print(label, flush=True)
    w = mla_build(1100 + heads + page_size + q_len, heads, q_len, [1, 45, 700, 1333, 2100], page_size,
                  dt=W.DT_FP8, q_dtype=W.DT_FP8)
    run_and_check(w, label)
    run_and_check(w, label + " unsplit", flags=B.FLAG_NO_INTERNAL_SPLIT)


@pytest.mark.parametrize("heads,q_len", [(128, 2), (16, 2)])
def test_mla_fp8_queries_explicit_splits(heads, q_len):
    w = mla_build(1191 + heads, heads, q_len, [0, 5, 640, 999], 64, dt=W.DT_FP8, q_dtype=W.DT_FP8)
    d = R.upload(w)
    S = 3
    res = R.run(d, num_kv_splits=S)
    torch.cuda.synchronize()
    po, pl, pm = OR.attention(w, num_kv_splits=S)
    for c in range(S):
        check_rows(w, to64(res["po"][c]), to64(res["plse"][c]), po[c], pl[c],
                   to64(res["pmx"][c]), pm[c], label=f"MLA fp8 Q partial {c}")
    o, lse, _ = OR.attention(w, num_kv_splits=1)
    check_rows(w, to64(res["o"]), to64(res["lse"]), o, lse, label="MLA fp8 Q merged")


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c5"])
def test_parity_generic_kernel(name):
    print(f"generic {name}", flush=True)
    run_and_check(small(name), name + " generic", flags=B.FLAG_FORCE_GENERIC)


def test_split_partials_and_merge():
    w = small("c2")
    d = R.upload(w)
    S = 5
    res = R.run(d, num_kv_splits=S)
    torch.cuda.synchronize()
    po, pl, pm = OR.attention(w, num_kv_splits=S)
    for c in range(S):
        check_rows(w, to64(res["po"][c]), to64(res["plse"][c]), po[c], pl[c],
                   to64(res["pmx"][c]), pm[c], label=f"partial {c}")
    o, lse, _ = OR.attention(w, num_kv_splits=1)
    check_rows(w, to64(res["o"]), to64(res["lse"]), o, lse, label="merged")


def test_merge_states_against_oracle_merge():
    rng = np.random.default_rng(5)
    S, rows, D = 7, 300, 128
    v = rng.standard_normal((S, rows, D)).astype(np.float32)
    s = (rng.standard_normal((S, rows)) * 4).astype(np.float32)
    s[:, 0] = -np.inf          # a row with no state
    s[2:5, 1] = -np.inf        # some empty states
    vo_ref, so_ref = OR.merge_states(v.astype(np.float64), s.astype(np.float64))
    for odt in (torch.float32, torch.bfloat16):
        vo, so = B.merge_states(torch.from_numpy(v).cuda(), torch.from_numpy(s).cuda(),
                                out_dtype=odt)
        torch.cuda.synchronize()
        tol = 1e-5 if odt == torch.float32 else 2e-2
        assert np.abs(to64(vo) - vo_ref).max() <= tol
        so64 = to64(so)
        assert np.isneginf(so64[0]) and (to64(vo)[0] == 0).all()
        assert np.abs(so64[1:] - so_ref[1:]).max() <= 1e-5


def test_page_permutation_bitwise():
    from test_oracle import _permute_pages
    w = small("c2")
    a = R.run(R.upload(w))
    b = R.run(R.upload(_permute_pages(w, 3)))
    torch.cuda.synchronize()
    assert torch.equal(a["o"], b["o"]) and torch.equal(a["lse"], b["lse"])


def test_same_kv_strides_variant_equals_general_bitwise():
    w = small("c2")
    d = R.upload(w)
    a = R.run(d)
    b = R.run(d, flags=B.FLAG_FORCE_GENERAL_STRIDES)
    torch.cuda.synchronize()
    assert torch.equal(a["o"], b["o"]) and torch.equal(a["lse"], b["lse"])


def test_repeat_runs_bitwise_identical():
    w = small("c3")
    d = R.upload(w)
    a = R.run(d)
    for _ in range(3):
        b = R.run(d)
        torch.cuda.synchronize()
        assert torch.equal(a["o"], b["o"]) and torch.equal(a["lse"], b["lse"])


def test_broadcast_equals_replicated():
    w = small("c5")
    a = R.run(R.upload(w))
    r = W.replicate_broadcast(w)
    b = R.run(R.upload(r))
    torch.cuda.synchronize()
    tol_o, tol_l = tolerances(w)
    assert (to64(a["o"]) - to64(b["o"])).__abs__().max() <= tol_o
    assert (to64(a["lse"]) - to64(b["lse"])).__abs__().max() <= tol_l


@pytest.mark.parametrize("kind", ["gqa", "mla_narrow", "mla_mid"])
def test_broadcast_decode_split(kind):
    # one KV batch read by a few query batches, long enough that the decode
    # kernels split it over workgroups (each query batch walks its own copy of
    # the range); checked against the oracle and against replicated page lists
    rng = np.random.default_rng(80 + len(kind))
    if kind == "gqa":
        w = W.build(rng, 81, "bcast gqa", q_lens=[1, 1], kv_lens=[3000], num_qo_heads=16,
                    num_kv_heads=2, head_dim_qk=128, head_dim_vo=128, page_size=16,
                    q_dtype=W.DT_BF16, kv_dtype=W.DT_BF16, kv_broadcast=True)
    else:
        ql = 1 if kind == "mla_narrow" else 2
        w = W.build(rng, 82 + ql, f"bcast {kind}", q_lens=[ql] * 3, kv_lens=[5000], num_qo_heads=16,
                    num_kv_heads=1, head_dim_qk=576, head_dim_vo=512, page_size=64,
                    q_dtype=W.DT_BF16, kv_dtype=W.DT_BF16, shared_kv=True, causal=True,
                    sm_scale=1.0 / np.sqrt(192.0), kv_broadcast=True)
    print(kind, flush=True)
    run_and_check(w, f"broadcast {kind}")
    a = R.run(R.upload(w))
    b = R.run(R.upload(W.replicate_broadcast(w)))
    torch.cuda.synchronize()
    tol_o, tol_l = tolerances(w)
    assert np.abs(to64(a["o"]) - to64(b["o"])).max() <= tol_o
    assert np.abs(to64(a["lse"]) - to64(b["lse"])).max() <= tol_l


def test_prefill_entry_on_decode_shapes():
    # the prefill entry point with uniform q lengths computes what decode computes
    w = c4_small(16, 4, W.DT_BF16)
    d = R.upload(w)
    res = R.run(d, force_prefill=True)
    torch.cuda.synchronize()
    o, lse, _ = OR.attention(w)
    check_rows(w, to64(res["o"]), to64(res["lse"]), o, lse, label="prefill entry, MLA shapes")


def test_edge_lengths_and_empty_batches():
    rng = np.random.default_rng(77)
    # empty KV batch, one token, a partial page, exactly one page, a page + 1
    kv_lens = [0, 1, 7, 16, 17, 33, 0, 250]
    w = W.build(rng, 77, "edges", q_lens=[1] * len(kv_lens), kv_lens=kv_lens, num_qo_heads=64,
                num_kv_heads=8, head_dim_qk=128, head_dim_vo=128, page_size=16,
                q_dtype=W.DT_BF16, kv_dtype=W.DT_BF16, pool_pages=40)
    run_and_check(w, "edge lengths")
    for S in (3, 40):  # more splits than pages: empty partial states
        run_and_check(dataclasses.replace(w, num_kv_splits=S), f"edge lengths S={S}")


def test_balanced_split_ragged_batches():
    # more than 2 x 64 query batches (the workgroups scan the batch 64 at a time),
    # empty and sub-tile KV batches next to long ones: workgroup shares start and
    # end inside items, items span many workgroups, and some workgroups hold
    # several whole items
    rng = np.random.default_rng(78)
    kv_lens = rng.integers(0, 200, size=130)
    kv_lens[[0, 5, 64, 127, 129]] = 0
    kv_lens[[1, 65, 128]] = [1, 31, 33]
    kv_lens[[10, 70, 100]] = [3000, 4097, 2500]
    w = W.build(rng, 78, "balanced", q_lens=[1] * 130, kv_lens=kv_lens, num_qo_heads=16,
                num_kv_heads=2, head_dim_qk=128, head_dim_vo=128, page_size=16,
                q_dtype=W.DT_BF16, kv_dtype=W.DT_BF16)
    run_and_check(w, "balanced ragged")
    run_and_check(w, "balanced ragged, short hint", max_kv_len=300)
    run_and_check(dataclasses.replace(w, causal=True), "balanced ragged causal")


def test_causal_rows_that_see_nothing():
    # q_len 4 against KV lengths 1..3: the first queries see no token
    w = W.config4(num_heads=16, q_len=4, batch=6, min_len=1, max_len=3)
    run_and_check(w, "MLA empty causal rows")
    w2 = W.config4(num_heads=128, q_len=2, kv_dtype=W.DT_FP8, batch=4, min_len=1, max_len=2)
    run_and_check(w2, "MLA fp8 empty causal rows")


def mla_build(seed, heads, q_len, kv_lens, page_size, dt=W.DT_BF16, q_dtype=W.DT_BF16, **kw):
    rng = np.random.default_rng(seed)
    return W.build(rng, seed, f"mla h{heads} q{q_len} p{page_size}", q_lens=[q_len] * len(kv_lens),
                   kv_lens=kv_lens, num_qo_heads=heads, num_kv_heads=1, head_dim_qk=576,
                   head_dim_vo=512, page_size=page_size, q_dtype=q_dtype, kv_dtype=dt,
                   shared_kv=True, causal=True, sm_scale=1.0 / np.sqrt(192.0), **kw)


@pytest.mark.parametrize("heads,q_len,page_size", [(48, 3, 24), (16, 1, 1), (128, 2, 64), (40, 4, 7)])
def test_mla_row_tiles_and_page_sizes(heads, q_len, page_size):
    # q_len x H rows that fill row tiles partly (144 = 128 + 16, 160 = 128 + 32) or
    # cross two tiles, page sizes that are not powers of two, one-token pages
    label = f"MLA h{heads} q{q_len} page {page_size}"
    print(label, flush=True)
    w = mla_build(900 + heads + page_size, heads, q_len, [1, 45, 700, 1333, 64 * 5], page_size)
    run_and_check(w, label)


@pytest.mark.parametrize("heads,q_len,page_size,dt", [(16, 1, 32, W.DT_BF16), (8, 2, 96, W.DT_BF16),
                                                      (16, 1, 32, W.DT_FP8), (4, 3, 96, W.DT_FP8),
                                                      (16, 1, 24, W.DT_FP8),
                                                      (16, 2, 96, W.DT_BF16), (16, 4, 32, W.DT_FP8),
                                                      (12, 3, 24, W.DT_BF16), (10, 3, 64, W.DT_FP8),
                                                      (16, 4, 64, W.DT_BF16)])
def test_mla_narrow_page_sizes(heads, q_len, page_size, dt):
    # up to 16 rows per request (one row block) and 17..64 (two or four row blocks
    # sharing the contraction over waves): page sizes that hold whole 32-token
    # tiles (32, 64, 96: the tile's page offset is uniform) and one that does not
    # (24); long enough that the KV is split over workgroups
    label = f"MLA narrow h{heads} q{q_len} page {page_size} dt {dt}"
    print(label, flush=True)
    w = mla_build(950 + heads + page_size + dt, heads, q_len, [0, 31, 33, 3000, 4500, 96 * 20], page_size,
                  dt=dt)
    run_and_check(w, label)


@pytest.mark.parametrize("heads,q_len,page_size,dt", [(16, 1, 32, W.DT_BF16), (16, 1, 64, W.DT_FP8),
                                                       (16, 4, 32, W.DT_FP8), (16, 2, 64, W.DT_BF16)])
def test_mla_long_range_one_workgroup(heads, q_len, page_size, dt):
    # internal splitting off: one workgroup walks a 20000-token KV, so a range crosses
    # several page-id windows (256 pages each) and the page-aligned tile loads reload
    # their per-wave table of page ids every 64 tiles
    label = f"MLA one-workgroup range h{heads} q{q_len} page {page_size} dt {dt}"
    print(label, flush=True)
    w = mla_build(970 + heads + q_len + page_size + dt, heads, q_len, [20000, 7], page_size, dt=dt)
    run_and_check(w, label, flags=B.FLAG_NO_INTERNAL_SPLIT)


def test_mla_explicit_splits():
    w = mla_build(991, 128, 1, [0, 5, 640, 999], 64)
    d = R.upload(w)
    S = 4
    res = R.run(d, num_kv_splits=S)
    torch.cuda.synchronize()
    po, pl, pm = OR.attention(w, num_kv_splits=S)
    for c in range(S):
        check_rows(w, to64(res["po"][c]), to64(res["plse"][c]), po[c], pl[c],
                   to64(res["pmx"][c]), pm[c], label=f"MLA partial {c}")
    o, lse, _ = OR.attention(w, num_kv_splits=1)
    check_rows(w, to64(res["o"]), to64(res["lse"]), o, lse, label="MLA merged")


def test_output_dtypes():
    w = small("c2")
    d = R.upload(w)
    o, lse, _ = OR.attention(w)
    for odt in (torch.float32, torch.float16, torch.bfloat16):
        res = R.run(d, out_dtype=odt)
        torch.cuda.synchronize()
        assert res["o"].dtype == odt
        check_rows(w, to64(res["o"]), to64(res["lse"]), o, lse, label=f"out {odt}")


def test_decode_takes_mfma_path_with_and_without_internal_chunks():
    w = small("c2")
    step = R.prepare(R.upload(w))
    assert step.attention_kernel_name.startswith("gqa_decode_mfma"), step.attention_kernel_name
    for flags in (0, B.FLAG_NO_INTERNAL_SPLIT, B.FLAG_FORCE_GENERAL_STRIDES,
                  B.FLAG_NO_INTERNAL_SPLIT | B.FLAG_FORCE_GENERAL_STRIDES):
        run_and_check(w, f"c2 flags={flags}", flags=flags)
    # a length hint below the real maximum only changes the chunking, not the result
    run_and_check(w, "c2 short hint", max_kv_len=300)


@pytest.mark.parametrize("name,prefix", [("c3", "flash_attn_mfma"), ("c5", "flash_attn_mfma"),
                                         ("c2", "gqa_decode_mfma"), ("c1", "generic")])
def test_plan_names(name, prefix):
    step = R.prepare(R.upload(small(name)))
    assert step.attention_kernel_name.startswith(prefix), step.attention_kernel_name


def sparse_cases():
    """Sparse-selected KV (page size 1: kv_indices are each query's selected
    token slots in a larger, NaN-poisoned pool), through every decode kernel
    family: MLA narrow (16 rows), mid (64 rows), many-rows (128 rows), GQA."""
    lens = [1, 31, 32, 33, 700, 2048]
    return {
        "mla_h16_bf16": lambda: W.config_sparse(num_heads=16, kv_lens=lens, pool_factor=3),
        "mla_h16_fp8": lambda: W.config_sparse(num_heads=16, kv_dtype=W.DT_FP8, kv_lens=lens,
                                               pool_factor=3),
        "mla_h64_fp8": lambda: W.config_sparse(num_heads=64, kv_dtype=W.DT_FP8,
                                               kv_lens=[17, 500, 1500], pool_factor=2),
        "mla_h128_bf16": lambda: W.config_sparse(num_heads=128, kv_lens=[5, 300, 1000],
                                                 pool_factor=2),
        "gqa": lambda: W.config_sparse(mla=False, kv_lens=[1, 64, 65, 999, 2048], pool_factor=3),
    }


@pytest.mark.parametrize("name", list(sparse_cases()))
def test_sparse_selected_kv(name):
    run_and_check(sparse_cases()[name](), f"sparse {name}")


@pytest.mark.parametrize("name", ["mla_h16_bf16", "gqa"])
def test_sparse_selection_routed_halves_merge_on_gpu(name):
    """Two holders each see an interleaved half of every query's selection: the
    two partial calls (fp32 O and LSE) merged by merge_states match the oracle
    over the whole selection."""
    from test_oracle import select_subset
    w = sparse_cases()[name]()
    o, lse, _ = OR.attention(w)
    parts = [R.run(R.upload(select_subset(w, lambda b, i, r=r: i % 2 == r)), out_dtype=torch.float32)
             for r in (0, 1)]
    mo, ml = B.merge_states(torch.stack([p["o"] for p in parts]).contiguous(),
                            torch.stack([p["lse"] for p in parts]).contiguous(),
                            out_dtype=parts[0]["o"].dtype)
    torch.cuda.synchronize()
    check_rows(w, to64(mo), to64(ml), o, lse, label=f"routed halves {name}")


@pytest.mark.parametrize("name", ["gqa_b1", "gqa_b2_d64_f16", "gqa_b1_d256", "mla_b1_bf16",
                                  "mla_b1_fp8_q2"])
def test_few_long_requests_wide_merge(name):
    """Few long requests: the balanced split gives each row dozens of partial
    states, merged by a workgroup per row (lane groups over fixed shares of the
    states, combined in a fixed order; 16, 8, 4 and 2 lane groups for head dims
    64, 128, 256 and 512): oracle parity and bitwise repeats."""
    w = {
        "gqa_b1": lambda: W.config2(batch=1, min_len=60000, max_len=60000),
        "gqa_b2_d64_f16": lambda: W.build(np.random.default_rng(41), 41, "few_long_d64",
                                          q_lens=[1, 1], kv_lens=[50000, 1], num_qo_heads=16,
                                          num_kv_heads=4, head_dim_qk=64, head_dim_vo=64,
                                          page_size=32, q_dtype=W.DT_F16, kv_dtype=W.DT_F16),
        "gqa_b1_d256": lambda: W.build(np.random.default_rng(42), 42, "few_long_d256", q_lens=[1],
                                       kv_lens=[40000], num_qo_heads=16, num_kv_heads=4,
                                       head_dim_qk=256, head_dim_vo=256, page_size=16,
                                       q_dtype=W.DT_BF16, kv_dtype=W.DT_BF16),
        "mla_b1_bf16": lambda: W.config4(num_heads=16, q_len=1, batch=1, min_len=30000, max_len=30000),
        "mla_b1_fp8_q2": lambda: W.config4(num_heads=16, q_len=2, kv_dtype=W.DT_FP8, batch=1,
                                           min_len=25000, max_len=25000),
    }[name]()
    _, res = run_and_check(w, f"wide merge {name}")
    again = R.run(R.upload(w))
    torch.cuda.synchronize()
    assert torch.equal(again["o"], res["o"]) and torch.equal(again["lse"], res["lse"])


@pytest.mark.parametrize("heads,q_len,dt,qdt", [(128, 2, W.DT_BF16, W.DT_BF16), (128, 3, W.DT_FP8, W.DT_FP8),
                                                (144, 1, W.DT_FP8, W.DT_BF16), (128, 4, W.DT_FP8, W.DT_FP8)])
def test_mla_balanced_split_over_row_tiles(heads, q_len, dt, qdt):
    """More than one 128-row tile per request: the balanced split's items are
    (request, row tile), consecutive shares run on one XCD, and the merge maps
    each row to its row tile's states.  Ragged and empty requests, long ones
    spread over many workgroups; bitwise repeat."""
    kv_lens = [0, 1, 31, 4000, 700, 9000, 2, 5000]
    label = f"MLA balanced row tiles h{heads} q{q_len} {W.DT_NAMES[dt]} q {W.DT_NAMES[qdt]}"
    print(label, flush=True)
    w = mla_build(1300 + heads + q_len + dt + qdt, heads, q_len, kv_lens, 64, dt=dt, q_dtype=qdt)
    _, res = run_and_check(w, label)
    again = R.run(R.upload(w))
    torch.cuda.synchronize()
    assert torch.equal(again["o"], res["o"]) and torch.equal(again["lse"], res["lse"])


def test_mla_one_long_request_many_row_tiles_wide_merge():
    """One request, 512 rows (four row tiles), 40000 tokens: every row tile's
    states are merged by the wide merge."""
    w = mla_build(1350, 128, 4, [40000], 64, dt=W.DT_FP8, q_dtype=W.DT_FP8)
    run_and_check(w, "MLA b1 512 rows wide merge")
