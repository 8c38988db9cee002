"""GPU parity on inputs that drive the kernels into their rarely taken branches,
and on the argument combinations that the host sends to the generic kernel.

* Score jumps: the K rows of the second half of every KV batch get a gain, so a
  row's running maximum jumps by tens of log2 units after its first tiles.  The
  flash and MLA kernels re-base their reference maximum only when a tile's
  maximum exceeds it by more than 8 log2 units (rescaling O and the running
  sum mid-stream); with N(0,1) inputs that branch is rare.  Here it is taken on
  most rows, through every kernel family, with and without internal splits.
  The merged online-softmax state must still equal single-pass attention
  ("Move the Query, Not the Cache" summary, method section), and the LSE and
  max outputs must survive (PyTorch MPS FlexAttention post, experiment section).
* Zero and negative score scales (sm_scale = 0, sm_scale < 0, an fp8 cache with
  k_scale = 0): the flash and MLA kernels order raw scores, which is only right
  for a positive scale, so the host sends these to the generic kernel.
* Page size 8192 for MLA, f16 queries over an fp8 cache, and prefill over an
  fp8 cache: no MFMA kernel takes them; the generic kernel does.
"""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import oracle as OR
from paged_kv_attention_prefill_amd import binding as B
from paged_kv_attention_prefill_amd import runner as R
from paged_kv_attention_prefill_amd import workloads as W
from gpu_check import check_rows, to64

pytestmark = pytest.mark.gpu

MLA_SCALE = 1.0 / np.sqrt(192.0)


def run_and_check(w, label, flags=0, expect_plan=None, **kw):
    print(f"case {label}: {w.manifest()}", flush=True)
    d = R.upload(w)
    if expect_plan is not None:
        step = R.prepare(d, flags=flags)
        assert step.attention_kernel_name.startswith(expect_plan), step.attention_kernel_name
    res = R.run(d, flags=flags, **kw)
    torch.cuda.synchronize()
    o, lse, mx = OR.attention(w, num_kv_splits=1)
    return check_rows(w, to64(res["o"]), to64(res["lse"]), o, lse,
                      None if res.get("mx") is None else to64(res["mx"]), mx, label=label)


def mla(seed, heads, q_len, kv_lens, page_size=64, dt=W.DT_BF16, gain=None, q_dtype=W.DT_BF16,
        **kw):
    rng = np.random.default_rng(seed)
    return W.build(rng, seed, f"mla h{heads} q{q_len} p{page_size}", q_lens=[q_len] * len(kv_lens),
                   kv_lens=kv_lens, num_qo_heads=heads, num_kv_heads=1, head_dim_qk=576,
                   head_dim_vo=512, page_size=page_size, q_dtype=q_dtype, kv_dtype=dt,
                   shared_kv=True, causal=True, sm_scale=MLA_SCALE,
                   k_late_gain=None if gain is None else (gain, 512, 576), **kw)


# ------------------------------------------------------------------ score jumps
# gain 8 on the 64 rope dims (MLA) or on all 128 dims: late scores spread with a
# standard deviation of ~7-12 log2 units; gain 32: late scores span about +-60
# (natural log units) and beyond.

def jump_cases():
    return {
        "flash_c3": lambda g: W.config3(batch=3, min_q=100, max_q=300, max_prefix=900,
                                        k_late_gain=(g, 0, 128)),
        "flash_c5": lambda g: W.config5(num_queries=8, kv_len=6000, num_kv_splits=1,
                                        k_late_gain=(g, 0, 128)),
        "flash_c5_split4": lambda g: W.config5(num_queries=8, kv_len=6000, num_kv_splits=4,
                                               k_late_gain=(g, 0, 128)),
        "gqa_c2": lambda g: W.config2(batch=6, min_len=1, max_len=3000, k_late_gain=(g, 0, 128)),
        "mla_narrow_bf16": lambda g: mla(401, 16, 1, [1, 700, 3000, 4100], gain=g),
        "mla_narrow_fp8": lambda g: mla(402, 16, 1, [1, 700, 3000, 4100], dt=W.DT_FP8, gain=g),
        "mla_mid_bf16": lambda g: mla(403, 16, 4, [2, 900, 3300], gain=g),
        "mla_mid_fp8": lambda g: mla(404, 16, 4, [2, 900, 3300], dt=W.DT_FP8, gain=g),
        "mla_rows_bf16": lambda g: mla(405, 128, 1, [5, 1000, 3000], gain=g),
        "mla_rows_fp8": lambda g: mla(406, 128, 1, [5, 1000, 3000], dt=W.DT_FP8, gain=g),
        "mla_rows2_bf16": lambda g: mla(407, 128, 2, [5, 1500], gain=g),
        "mla_rows2_fp8": lambda g: mla(408, 128, 2, [5, 1500], dt=W.DT_FP8, gain=g),
        "mla_rows_fp8q": lambda g: mla(409, 128, 1, [5, 1000, 3000], dt=W.DT_FP8, gain=g,
                                       q_dtype=W.DT_FP8),
        "mla_rows4_fp8q": lambda g: mla(410, 128, 4, [5, 1500], dt=W.DT_FP8, gain=g,
                                        q_dtype=W.DT_FP8),
        "mla_narrow_fp8q": lambda g: mla(411, 16, 1, [1, 700, 3000, 4100], dt=W.DT_FP8, gain=g,
                                         q_dtype=W.DT_FP8),
        # 64 rows on the fp8-MFMA many-rows kernel (waves 4..7 hold no rows)
        "mla_rows_h16q4_fp8q": lambda g: mla(412, 16, 4, [2, 900, 3300], dt=W.DT_FP8, gain=g,
                                             q_dtype=W.DT_FP8),
    }


PLAN_OF = {"flash": "flash_attn_mfma", "gqa": "gqa_decode_mfma", "mla": "mla_decode_mfma"}


@pytest.mark.parametrize("gain", [8.0, 32.0])
@pytest.mark.parametrize("name", list(jump_cases()))
def test_score_jumps(name, gain):
    w = jump_cases()[name](gain)
    # the rows' maxima really jump: on most rows that see both halves of the KV,
    # the largest score of the second half exceeds that of the first by more
    # than the re-base threshold (8 log2 units; 20 with gain 32)
    _, _, mx2 = OR.attention(w, num_kv_splits=2)
    both = np.isfinite(mx2[0]) & np.isfinite(mx2[1])
    jump = (mx2[1][both] - mx2[0][both]) * np.log2(np.e)
    assert both.any() and (jump > (8 if gain == 8.0 else 20)).mean() > 0.5, np.median(jump)
    stats = [run_and_check(w, f"jump {name} gain {gain}", expect_plan=PLAN_OF[name.split("_")[0]])]
    if name.startswith(("mla", "gqa")):
        # one workgroup walks each row's whole range: the jump lands mid-range
        stats.append(run_and_check(w, f"jump {name} gain {gain} unsplit", flags=B.FLAG_NO_INTERNAL_SPLIT))
    if name.startswith("mla_rows") and name.endswith("fp8q"):
        # the fp8-query many-rows kernel multiplies P.V on the fp8 MFMA with P
        # split into two e4m3 terms (about 8 significant bits, as bf16): its
        # error stays at the level of the bf16-P kernels (about 1.6e-2 here),
        # where P in one e4m3 term (4 significant bits) reaches 5e-2 to 8e-2 on
        # these cases in a CPU emulation of the kernel's arithmetic
        for s in stats:
            assert s["max_err_o"] <= 3e-2, s


def test_score_jumps_split_partials():
    """Explicit split states of a jumping flash case, each against the oracle's
    partial state, then merged by merge_states."""
    w = jump_cases()["flash_c5_split4"](32.0)
    d = R.upload(w)
    res = R.run(d)
    torch.cuda.synchronize()
    po, pl, pm = OR.attention(w)
    for c in range(w.num_kv_splits):
        check_rows(w, to64(res["po"][c]), to64(res["plse"][c]), po[c], pl[c], to64(res["pmx"][c]),
                   pm[c], label=f"jump partial {c}")
    o, lse, _ = OR.attention(w, num_kv_splits=1)
    check_rows(w, to64(res["o"]), to64(res["lse"]), o, lse, label="jump merged")


# ------------------------------------------------------ zero / negative scales

def scale_cases():
    return {
        "flash_c3": lambda: W.config3(batch=2, min_q=50, max_q=200, max_prefix=300),
        "gqa_c2": lambda: W.config2(batch=4, min_len=1, max_len=900),
        "mla_narrow": lambda: mla(411, 16, 1, [3, 700, 2000]),
        "mla_rows": lambda: mla(412, 128, 2, [3, 700]),
        "mla_fp8_mid": lambda: mla(413, 16, 4, [3, 800], dt=W.DT_FP8),
    }


@pytest.mark.parametrize("scale", ["zero", "negative"])
@pytest.mark.parametrize("name", list(scale_cases()))
def test_non_positive_score_scale(name, scale):
    w = scale_cases()[name]()
    w = dataclasses.replace(w, sm_scale=0.0 if scale == "zero" else -w.sm_scale)
    plan = "gqa_decode_mfma" if name.startswith("gqa") else "generic"
    run_and_check(w, f"{name} sm_scale {scale}", expect_plan=plan)


def test_fp8_cache_with_zero_k_scale():
    # real K = 0 * codes: every score is 0, O is the mean of V over the allowed set
    w = dataclasses.replace(mla(414, 16, 2, [4, 1000, 2500], dt=W.DT_FP8), k_scale=0.0)
    run_and_check(w, "fp8 k_scale 0", expect_plan="generic")
    w2 = dataclasses.replace(mla(415, 128, 1, [4, 1200], dt=W.DT_FP8), k_scale=0.0)
    run_and_check(w2, "fp8 k_scale 0, 128 rows", expect_plan="generic")


# -------------------------------------------- combinations the generic kernel takes

@pytest.mark.parametrize("dt", [W.DT_BF16, W.DT_FP8])
@pytest.mark.parametrize("heads,q_len", [(16, 1), (16, 4)])
def test_mla_page_size_8192(heads, q_len, dt):
    w = mla(420 + heads + q_len + dt, heads, q_len, [1, 9000, 17000], page_size=8192, dt=dt)
    run_and_check(w, f"MLA page 8192 h{heads} q{q_len} {W.DT_NAMES[dt]}", expect_plan="generic")


def test_f16_queries_over_fp8_cache():
    rng = np.random.default_rng(431)
    w = W.build(rng, 431, "f16 x fp8 gqa", q_lens=[1] * 4, kv_lens=[1, 90, 700, 1300],
                num_qo_heads=16, num_kv_heads=4, head_dim_qk=128, head_dim_vo=128, page_size=16,
                q_dtype=W.DT_F16, kv_dtype=W.DT_FP8)
    run_and_check(w, "f16 Q x fp8 KV, d128", expect_plan="generic")
    rng = np.random.default_rng(432)
    w2 = W.build(rng, 432, "f16 x fp8 mla", q_lens=[2] * 3, kv_lens=[1, 500, 1800],
                 num_qo_heads=16, num_kv_heads=1, head_dim_qk=576, head_dim_vo=512, page_size=64,
                 q_dtype=W.DT_F16, kv_dtype=W.DT_FP8, shared_kv=True, causal=True,
                 sm_scale=MLA_SCALE)
    run_and_check(w2, "f16 Q x fp8 KV, MLA", expect_plan="generic")


def test_prefill_over_fp8_cache():
    rng = np.random.default_rng(433)
    w = W.build(rng, 433, "prefill fp8", q_lens=[1, 60, 150], kv_lens=[1, 300, 400],
                num_qo_heads=16, num_kv_heads=4, head_dim_qk=128, head_dim_vo=128, page_size=16,
                q_dtype=W.DT_BF16, kv_dtype=W.DT_FP8, causal=True, uniform_q_len=False)
    run_and_check(w, "ragged causal prefill, bf16 Q x fp8 KV", expect_plan="generic")


def test_fp8_queries_generic_kernel():
    """fp8 queries outside the MLA kernels (GQA shape, and MLA forced onto the
    generic kernel): the generic kernel decodes the codes and applies q_scale."""
    rng = np.random.default_rng(435)
    w = W.build(rng, 435, "fp8q gqa", q_lens=[1] * 4, kv_lens=[1, 90, 700, 1300],
                num_qo_heads=16, num_kv_heads=4, head_dim_qk=128, head_dim_vo=128, page_size=16,
                q_dtype=W.DT_FP8, kv_dtype=W.DT_FP8)
    run_and_check(w, "fp8 Q x fp8 KV, d128", expect_plan="generic")
    w2 = mla(436, 128, 2, [1, 333, 900], dt=W.DT_FP8, q_dtype=W.DT_FP8)
    run_and_check(w2, "MLA fp8 Q forced generic", flags=B.FLAG_FORCE_GENERIC, expect_plan="generic")


def test_mla_forced_generic():
    w = mla(434, 16, 2, [1, 333, 1500], dt=W.DT_FP8)
    run_and_check(w, "MLA fp8 forced generic", flags=B.FLAG_FORCE_GENERIC, expect_plan="generic")
