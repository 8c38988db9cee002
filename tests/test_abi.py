"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects every host-checkable bad argument with its status
code before touching the device.  Pointers here are fake (never dereferenced:
validation fails, or only the host-only workspace query runs)."""
import ctypes

import numpy as np
import pytest

from paged_kv_attention_prefill_amd import binding as B

FAKE = 0x100000  # 16-byte aligned, never dereferenced


@pytest.fixture(scope="module")
def lib():
    return B.load_library()


def test_exports_every_header_function(lib):
    names = B.header_functions()
    assert set(names) >= {"paged_attn_decode", "paged_attn_prefill", "merge_states",
                          "paged_attn_decode_workspace_size", "paged_attn_prefill_workspace_size",
                          "pa_abi_version", "pa_status_string", "paged_attn_check_tables"}
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert lib.pa_abi_version() == 2
    for st in range(0, -8, -1):
        assert B.status_string(st) != "unknown status"
    assert B.status_string(-99) == "unknown status"


def good_kv(dqk=128, dvo=128, hkv=8, P=16, dt=B.PA_BF16, nkb=4):
    kv = B.PagedKV()
    kv.k, kv.v = FAKE, FAKE * 2
    st = (P * hkv * dqk, hkv * dqk, dqk)
    for i in range(3):
        kv.k_stride[i] = st[i]
        kv.v_stride[i] = st[i]
    kv.num_kv_heads, kv.page_size, kv.head_dim_qk, kv.head_dim_vo = hkv, P, dqk, dvo
    kv.kv_dtype = dt
    kv.k_scale = kv.v_scale = 1.0
    kv.kv_indptr, kv.kv_indices, kv.kv_last_page_len = FAKE, FAKE, FAKE
    kv.num_kv_batches = nkb
    kv.max_kv_len_hint = 8192
    return kv


def good_decode():
    a = B.DecodeArgs()
    a.q, a.q_dtype, a.batch, a.q_len, a.num_qo_heads = FAKE, B.PA_BF16, 4, 1, 64
    a.kv = good_kv()
    a.kv_broadcast, a.causal, a.sm_scale, a.num_kv_splits = 0, 0, 0.088, 1
    a.o, a.o_dtype, a.lse, a.row_max, a.flags = FAKE, B.PA_BF16, FAKE, None, 0
    return a


def good_prefill():
    a = B.PrefillArgs()
    a.q, a.q_dtype, a.qo_indptr, a.batch, a.total_q, a.max_q_len_hint = FAKE, B.PA_BF16, FAKE, 4, 100, 40
    a.num_qo_heads = 32
    a.kv = good_kv()
    a.kv_broadcast, a.causal, a.sm_scale = 0, 1, 0.088
    a.o, a.o_dtype, a.lse, a.row_max, a.flags = FAKE, B.PA_BF16, FAKE, None, 0
    return a


def dsize(lib, a):
    n = ctypes.c_size_t(12345)
    st = lib.paged_attn_decode_workspace_size(ctypes.byref(a), ctypes.byref(n))
    return st, n.value


def psize(lib, a):
    n = ctypes.c_size_t(12345)
    st = lib.paged_attn_prefill_workspace_size(ctypes.byref(a), ctypes.byref(n))
    return st, n.value


def test_valid_workspace_queries_are_host_only(lib):
    st, n = dsize(lib, good_decode())
    assert st == 0 and n >= 0
    st, n = psize(lib, good_prefill())
    assert st == 0 and n >= 0


def mutate(a, path, value):
    obj = a
    parts = path.split(".")
    for p in parts[:-1]:
        obj = getattr(obj, p)
    last = parts[-1]
    if "[" in last:
        name, idx = last[:-1].split("[")
        getattr(obj, name)[int(idx)] = value
    else:
        setattr(obj, last, value)
    return a


DECODE_BAD = [
    ("q", None, -1), ("o", None, -1), ("kv.k", None, -1), ("kv.v", None, -1),
    ("kv.kv_indptr", None, -1), ("kv.kv_indices", None, -1), ("kv.kv_last_page_len", None, -1),
    ("batch", 0, -2), ("q_len", 0, -2), ("num_qo_heads", 60, -2), ("kv.num_kv_heads", 0, -2),
    ("kv.page_size", 0, -2), ("kv.num_kv_batches", 3, -2), ("num_kv_splits", 0, -2),
    ("num_kv_splits", 2000, -2), ("kv.max_kv_len_hint", -1, -2), ("kv.k_stride[1]", -8, -2),
    ("sm_scale", float("nan"), -2), ("kv.k_scale", float("inf"), -2),
    ("q_dtype", 7, -3), ("kv.kv_dtype", -1, -3), ("o_dtype", B.PA_FP8_E4M3, -3),
    ("q_dtype", B.PA_FP8_E4M3, -5),
    ("kv.head_dim_qk", 96, -5), ("kv.head_dim_vo", 64, -5), ("q_dtype", B.PA_F32, -5),
    ("q", FAKE + 8, -4), ("kv.k", FAKE + 2, -4), ("o", FAKE + 4, -4),
    ("kv.v_stride[2]", 132, -4),
]


@pytest.mark.parametrize("path,value,status", DECODE_BAD)
def test_decode_rejects(lib, path, value, status):
    a = mutate(good_decode(), path, value)
    assert dsize(lib, a)[0] == status
    assert lib.paged_attn_decode(ctypes.byref(a), None, 0, None) == status


def test_decode_rejects_more(lib):
    a = good_decode()
    a.num_kv_splits = 4  # partial states must be fp32 with an LSE buffer
    assert dsize(lib, a)[0] == -3
    a.o_dtype = B.PA_F32
    assert dsize(lib, a)[0] == 0
    a.lse = None
    assert dsize(lib, a)[0] == -1
    a = good_decode()
    a.kv_broadcast = 1  # broadcast needs exactly one KV batch
    assert dsize(lib, a)[0] == -2
    a.kv.num_kv_batches = 1
    assert dsize(lib, a)[0] == 0
    a = good_decode()  # shared latent rows need identical strides and dvo <= dqk
    a.kv.v = a.kv.k
    a.kv.v_stride[0] = 7 * 16
    assert dsize(lib, a)[0] == -2
    assert lib.paged_attn_decode(None, None, 0, None) == -1
    assert lib.paged_attn_decode_workspace_size(ctypes.byref(good_decode()), None) == -1


PREFILL_BAD = [("qo_indptr", None, -1), ("q", None, -1), ("batch", 0, -2), ("total_q", -1, -2),
               ("max_q_len_hint", -3, -2), ("kv.num_kv_batches", 5, -2),
               ("kv.head_dim_qk", 576, -5), ("o", FAKE + 2, -4)]


@pytest.mark.parametrize("path,value,status", PREFILL_BAD)
def test_prefill_rejects(lib, path, value, status):
    a = mutate(good_prefill(), path, value)
    assert psize(lib, a)[0] == status
    assert lib.paged_attn_prefill(ctypes.byref(a), None, 0, None) == status


def test_merge_rejects(lib):
    m = lib.merge_states
    assert m(None, 0, FAKE, 2, 10, 128, FAKE, 0, None, None) == -1
    assert m(FAKE, 0, None, 2, 10, 128, FAKE, 0, None, None) == -1
    assert m(FAKE, 0, FAKE, 2, 10, 128, None, 0, None, None) == -1
    assert m(FAKE, 3, FAKE, 2, 10, 128, FAKE, 0, None, None) == -3
    assert m(FAKE, 0, FAKE, 2, 10, 128, FAKE, 9, None, None) == -3
    assert m(FAKE, 0, FAKE, 0, 10, 128, FAKE, 0, None, None) == -2
    assert m(FAKE, 0, FAKE, 1025, 10, 128, FAKE, 0, None, None) == -2
    assert m(FAKE, 0, FAKE, 2, -1, 128, FAKE, 0, None, None) == -2
    assert m(FAKE, 0, FAKE, 2, 10, 126, FAKE, 0, None, None) == -2
    assert m(FAKE, 0, FAKE, 2, 10, 2048, FAKE, 0, None, None) == -2
    assert m(FAKE + 4, 0, FAKE, 2, 10, 128, FAKE, 0, None, None) == -4
    assert m(FAKE, 0, FAKE, 2, 0, 128, FAKE, 0, None, None) == 0  # no rows: nothing to do


def test_check_tables(lib):
    def run(indptr, indices, last, pool, P):
        ip = np.asarray(indptr, np.int32)
        ix = np.asarray(indices, np.int32)
        la = np.asarray(last, np.int32)
        return lib.paged_attn_check_tables(ip.ctypes.data, ix.ctypes.data, la.ctypes.data,
                                           len(ip) - 1, pool, P)
    assert run([0, 2, 3], [4, 1, 0], [16, 5], 5, 16) == 0
    assert run([0, 2, 2], [4, 1], [16, 0], 5, 16) == 0      # empty batch: last ignored
    assert run([1, 2, 3], [4, 1, 0], [16, 5], 5, 16) == -2  # indptr[0] != 0
    assert run([0, 2, 1], [4, 1], [16, 5], 5, 16) == -2     # decreasing
    assert run([0, 2, 3], [4, 1, 5], [16, 5], 5, 16) == -2  # index out of pool
    assert run([0, 2, 3], [4, 1, 0], [17, 5], 5, 16) == -2  # last > page_size
    assert run([0, 2, 3], [4, 1, 0], [16, 0], 5, 16) == -2  # last < 1


def test_workloads_pass_table_check(lib):
    from paged_kv_attention_prefill_amd import workloads as W
    for w in (W.config1(), W.config2(batch=4, max_len=600), W.config5(num_queries=2, kv_len=1000)):
        assert lib.paged_attn_check_tables(w.kv_indptr.ctypes.data, w.kv_indices.ctypes.data,
                                           w.kv_last_page_len.ctypes.data, w.num_kv_batches,
                                           w.num_pool_pages, w.page_size) == 0


@pytest.mark.parametrize("which", ["decode", "prefill"])
def test_overflowing_score_scale_rejected(lib, which):
    # sm_scale * k_scale * log2(e) must be finite in fp32
    for sm, ks in ((3e38, 1.0), (1e10, 1e30), (-3e38, 1.0)):
        a = good_decode() if which == "decode" else good_prefill()
        a.sm_scale, a.kv.k_scale = sm, ks
        st = dsize(lib, a)[0] if which == "decode" else psize(lib, a)[0]
        assert st == -2, (sm, ks, st)


def mla_decode_args(sm=0.072, dt=B.PA_BF16, P=64, k_scale=1.0, heads=16):
    a = good_decode()
    a.num_qo_heads = heads
    a.kv = good_kv(dqk=576, dvo=512, hkv=1, P=P, dt=dt)
    a.kv.v = a.kv.k  # shared latent rows
    a.kv.k_scale = k_scale
    a.sm_scale = sm
    return a


def plan(lib, a):
    fn = lib.paged_attn_decode_plan_name if isinstance(a, B.DecodeArgs) else \
        lib.paged_attn_prefill_plan_name
    name = fn(ctypes.byref(a))
    return name.decode() if name else None


def test_plans_for_non_positive_scales(lib):
    # the flash and MLA kernels order raw scores, valid for a positive scale only
    assert plan(lib, mla_decode_args()).startswith("mla_decode_mfma")
    assert plan(lib, mla_decode_args(heads=128)).startswith("mla_decode_mfma")
    assert plan(lib, mla_decode_args(sm=0.0)) == "generic"
    assert plan(lib, mla_decode_args(sm=-0.072)) == "generic"
    assert plan(lib, mla_decode_args(dt=B.PA_FP8_E4M3)) == "mla_decode_mfma_fp8"
    assert plan(lib, mla_decode_args(dt=B.PA_FP8_E4M3, k_scale=0.0)) == "generic"
    p = good_prefill()
    assert plan(lib, p).startswith("flash_attn_mfma")
    for sm in (0.0, -0.088):
        p.sm_scale = sm
        assert plan(lib, p) == "generic"
    d = good_decode()  # the GQA decode scales every score before it is compared
    for sm in (0.088, 0.0, -0.088):
        d.sm_scale = sm
        assert plan(lib, d).startswith("gqa_decode_mfma")


def test_plans_for_generic_only_combinations(lib):
    assert plan(lib, mla_decode_args(P=8192)) == "generic"
    assert plan(lib, mla_decode_args(P=4096)).startswith("mla_decode_mfma")
    a = mla_decode_args(dt=B.PA_FP8_E4M3)
    a.q_dtype = B.PA_F16
    assert plan(lib, a) == "generic"
    p = good_prefill()
    p.kv.kv_dtype = B.PA_FP8_E4M3
    for i in range(3):
        p.kv.k_stride[i] //= 2
        p.kv.v_stride[i] //= 2
    assert plan(lib, p) == "generic"


def test_noalloc_rejects_oversized_workspace(lib):
    """paged_attn_decode_noalloc: a call whose workspace exceeds the library's
    scratch array (PA_NOALLOC_SCRATCH_BYTES) is refused before any GPU work;
    argument errors come back as for paged_attn_decode."""
    text = open(B.HEADER).read()
    assert "#define PA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)" in text
    assert B.NOALLOC_SCRATCH_BYTES == 128 << 20
    # GQA decode of 20000 requests x 8 KV heads, KV up to 8192 tokens: the
    # balanced split's partial-state slots (items + workgroups) x 16 rows x 128
    # fp32 dims exceed 1 GB
    a = good_decode()
    a.batch = 20000
    a.kv.num_kv_batches = 20000
    st, n = dsize(lib, a)
    assert st == 0 and n > B.NOALLOC_SCRATCH_BYTES
    assert lib.paged_attn_decode_noalloc(ctypes.byref(a), None) == -6
    for path, value, status in DECODE_BAD[:4]:
        bad = mutate(good_decode(), path, value)
        assert lib.paged_attn_decode_noalloc(ctypes.byref(bad), None) == status
    assert lib.paged_attn_decode_noalloc(None, None) == -1
