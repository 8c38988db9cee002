"""paged_attn_decode_noalloc (the decode entry point that allocates nothing; its
workspace is the library's own per-GPU scratch array) against paged_attn_decode
(caller workspace) and the CPU oracle, through the C ABI: two calls in a row on
the same GPU, the second with a smaller input, so the second call runs over
scratch memory the first one left behind."""
import numpy as np
import pytest
import torch

from oracle import oracle as OR
from paged_kv_attention_prefill_amd import binding as B
from paged_kv_attention_prefill_amd import runner as R
from paged_kv_attention_prefill_amd import workloads as W
from gpu_check import check_rows, to64

pytestmark = pytest.mark.gpu


def decode_both(w, label):
    print(f"no-alloc case {label}: {w.manifest()}", flush=True)
    d = R.upload(w)
    q4 = d.q.view(w.batch, w.q_len, w.num_qo_heads, w.head_dim_qk)
    common = dict(head_dim_vo=w.head_dim_vo, kv_dtype=w.kv_dtype, k_scale=w.k_scale,
                  v_scale=w.v_scale, q_scale=w.q_scale, max_kv_len=int(w.kv_lens.max()),
                  sm_scale=w.sm_scale,
                  causal=w.causal, kv_broadcast=w.kv_broadcast, return_max=True)
    ref_call = B.prepare_decode(q4, d.k, d.v, d.kv_indptr, d.kv_indices, d.kv_last, **common)
    assert ref_call.ws_bytes > 0, "the case must use a workspace"
    assert ref_call.ws_bytes <= B.NOALLOC_SCRATCH_BYTES
    na_call = B.prepare_decode(q4, d.k, d.v, d.kv_indptr, d.kv_indices, d.kv_last, noalloc=True,
                               **common)
    assert na_call.workspace is None and na_call.plan_name == ref_call.plan_name
    ref = ref_call()
    got = na_call()
    torch.cuda.synchronize()
    # the same plan and kernels over a different workspace: identical bits
    for k in ("o", "lse", "mx"):
        assert torch.equal(got[k], ref[k]), (label, k)
    o, lse, mx = OR.attention(w, num_kv_splits=1)
    check_rows(w, to64(got["o"]), to64(got["lse"]), o, lse, to64(got["mx"]), mx, label=label)


@pytest.mark.parametrize("family", ["gqa", "mla_narrow", "mla_rows", "mla_fp8_queries"])
def test_noalloc_two_calls_second_smaller(family):
    if family == "gqa":
        big = W.config2(batch=16, min_len=1, max_len=6000)
        small = W.config2(batch=3, min_len=1, max_len=1500, sub=1)
    elif family == "mla_narrow":
        big = W.config4(num_heads=16, q_len=1, batch=8, min_len=1, max_len=9000)
        small = W.config4(num_heads=16, q_len=1, batch=2, min_len=1, max_len=3000)
    elif family == "mla_rows":
        big = W.config4(num_heads=128, q_len=2, batch=4, min_len=1, max_len=7000)
        small = W.config4(num_heads=128, q_len=2, batch=2, min_len=1, max_len=2500)
    else:
        # fp8 queries over an fp8 cache (the fp8-MFMA kernel, 128-token units)
        big = W.config4(num_heads=128, q_len=2, kv_dtype=W.DT_FP8, q_dtype=W.DT_FP8, batch=4,
                        min_len=1, max_len=7000)
        small = W.config4(num_heads=16, q_len=4, kv_dtype=W.DT_FP8, q_dtype=W.DT_FP8, batch=2,
                          min_len=1, max_len=2500)
    decode_both(big, f"{family} first call")
    decode_both(small, f"{family} second call, smaller")
