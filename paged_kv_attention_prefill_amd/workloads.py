"""Seeded synthetic inputs for batched attention over a paged KV cache.

This module is shared by the HIP path's tests/bench and by the CPU oracle's
tests.  It holds none of the attention arithmetic: only shapes, random draws,
the rounding of those draws to the storage dtype (the bytes both sides read),
the page-table layout and NaN poisoning of bytes that no result may depend on.

Page-table convention (the paged KV cache of the FlashInfer PR #4736 analysis,
introduction and the ``paged_kv_t`` constructor in its code section 1): KV
batch b owns ``n_b = kv_indptr[b+1] - kv_indptr[b]`` pages whose physical ids
are ``kv_indices[kv_indptr[b]:kv_indptr[b+1]]``; the last page holds
``kv_last_page_len[b]`` tokens (1..page_size), so ``L_b = (n_b-1)*P + last``.

Draw order for every workload: lengths -> page permutation -> Q -> K -> V, from
``np.random.default_rng(seed)``; values ~ N(0,1) in fp32, then rounded to the
storage dtype with round-to-nearest-even (torch's CPU casts).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np
import torch

# numeric codes shared with the C ABI's pa_dtype enum
DT_F32, DT_F16, DT_BF16, DT_FP8 = 0, 1, 2, 3
DT_NAMES = {DT_F32: "f32", DT_F16: "f16", DT_BF16: "bf16", DT_FP8: "fp8_e4m3"}
DT_BYTES = {DT_F32: 4, DT_F16: 2, DT_BF16: 2, DT_FP8: 1}
_NP_STORAGE = {DT_F32: np.float32, DT_F16: np.uint16, DT_BF16: np.uint16, DT_FP8: np.uint8}
_TORCH_VIEW = {DT_F32: torch.float32, DT_F16: torch.float16, DT_BF16: torch.bfloat16,
               DT_FP8: torch.float8_e4m3fn}
# a NaN code of each storage dtype (OCP e4m3fn: S.1111.111 is its only NaN)
_NAN_CODE = {DT_F16: 0x7E00, DT_BF16: 0x7FC0, DT_FP8: 0x7F}
FP8_MAX = 448.0


def round_to_storage(x: np.ndarray, dtype: int) -> np.ndarray:
    """fp32 array -> raw storage codes of ``dtype`` (RNE), as a numpy array."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == DT_F32:
        return x
    t = torch.from_numpy(x)
    if dtype == DT_F16:
        return t.to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    if dtype == DT_BF16:
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if dtype == DT_FP8:
        # torch's cast yields NaN above 448, so clamp first
        return t.clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    raise ValueError(dtype)


def as_torch(raw: np.ndarray, dtype: int) -> torch.Tensor:
    """Raw storage codes -> CPU torch tensor of the storage dtype (no copy)."""
    t = torch.from_numpy(np.ascontiguousarray(raw))
    if dtype == DT_F32:
        return t
    return t.view(_TORCH_VIEW[dtype])


@dataclass
class Workload:
    name: str
    seed: int
    # queries: [total_q, Hq, Dqk] raw codes; query batch b owns rows qo_indptr[b]..qo_indptr[b+1]
    q: np.ndarray
    q_dtype: int
    qo_indptr: np.ndarray
    q_len: Optional[int]          # uniform query length (decode form), else None
    num_qo_heads: int
    num_kv_heads: int
    head_dim_qk: int
    head_dim_vo: int
    page_size: int
    # caches: raw codes; the logical element (page, slot, head, d) sits at
    # page*stride[0] + slot*stride[1] + head*stride[2] + d of the flat array
    k: np.ndarray
    v: Optional[np.ndarray]       # None: V is the first head_dim_vo dims of K's rows (shared latent cache)
    kv_dtype: int
    k_stride: tuple
    v_stride: tuple
    k_scale: float
    v_scale: float
    kv_indptr: np.ndarray
    kv_indices: np.ndarray
    kv_last_page_len: np.ndarray
    kv_lens: np.ndarray
    num_pool_pages: int
    kv_broadcast: bool
    causal: bool
    sm_scale: float
    num_kv_splits: int = 1
    k_layout: str = "NHD"
    v_layout: str = "NHD"
    q_scale: float = 1.0          # real Q = q_scale * stored Q (fp8 queries; 1 otherwise)
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return len(self.qo_indptr) - 1

    @property
    def total_q(self) -> int:
        return int(self.qo_indptr[-1])

    @property
    def num_kv_batches(self) -> int:
        return len(self.kv_indptr) - 1

    @property
    def shared_kv(self) -> bool:
        return self.v is None

    def q_lens(self) -> np.ndarray:
        return np.diff(self.qo_indptr)

    def kv_len_of_query_batch(self) -> np.ndarray:
        if self.kv_broadcast:
            return np.repeat(self.kv_lens[:1], self.batch)
        return self.kv_lens

    def manifest(self) -> dict:
        return dict(name=self.name, seed=self.seed, batch=self.batch, total_q=self.total_q,
                    q_len=self.q_len, Hq=self.num_qo_heads, Hkv=self.num_kv_heads,
                    Dqk=self.head_dim_qk, Dvo=self.head_dim_vo, P=self.page_size,
                    q_dtype=DT_NAMES[self.q_dtype], kv_dtype=DT_NAMES[self.kv_dtype],
                    kv_batches=self.num_kv_batches, sum_kv_len=int(self.kv_lens.sum()),
                    pages=int(self.kv_indptr[-1]), pool_pages=self.num_pool_pages,
                    broadcast=self.kv_broadcast, causal=self.causal, splits=self.num_kv_splits,
                    k_scale=self.k_scale, v_scale=self.v_scale, q_scale=self.q_scale,
                    sm_scale=self.sm_scale)


def _layout_array(x: np.ndarray, layout: str):
    """x logical [pool, P, H, D] -> (physical contiguous array, element strides (page, slot, head))."""
    pool, P, H, D = x.shape
    if layout == "NHD":
        return np.ascontiguousarray(x), (P * H * D, H * D, D)
    if layout == "HND":
        return np.ascontiguousarray(x.transpose(0, 2, 1, 3)), (H * P * D, D, P * D)
    raise ValueError(layout)


def build(rng: np.random.Generator, seed: int, name: str, *, q_lens: Sequence[int],
          kv_lens: Sequence[int], num_qo_heads: int, num_kv_heads: int, head_dim_qk: int,
          head_dim_vo: int, page_size: int, q_dtype: int, kv_dtype: int,
          shared_kv: bool = False, kv_broadcast: bool = False, causal: bool = False,
          sm_scale: Optional[float] = None, num_kv_splits: int = 1,
          pool_pages: Optional[int] = None, poison: bool = True, k_layout: str = "NHD",
          v_layout: str = "NHD", uniform_q_len: bool = True,
          k_late_gain: Optional[tuple] = None) -> Workload:
    """Lay out one paged workload.  ``rng`` has already drawn the lengths; this
    draws, in order, the page permutation, Q, K and V.

    ``k_late_gain = (gain, d0, d1)`` multiplies dims [d0, d1) of the K rows of
    the second half of every KV batch (tokens j >= ceil(L/2)) by ``gain`` before
    any fp8 scale is taken, so the scores of those tokens spread ``gain`` times
    wider: a row's running maximum then jumps far above its first tiles' maximum
    part-way through the KV (for a shared latent cache, dims past head_dim_vo
    leave V untouched)."""
    q_lens = np.asarray(q_lens, dtype=np.int64)
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    P = page_size
    n_pages = (kv_lens + P - 1) // P
    kv_indptr = np.zeros(len(kv_lens) + 1, dtype=np.int32)
    kv_indptr[1:] = np.cumsum(n_pages)
    total_pages = int(kv_indptr[-1])
    pool = total_pages if pool_pages is None else int(pool_pages)
    assert pool >= total_pages
    last = np.where(n_pages > 0, kv_lens - (n_pages - 1) * P, 0).astype(np.int32)

    perm = rng.permutation(pool).astype(np.int32)
    kv_indices = perm[:total_pages].copy()

    qo_indptr = np.zeros(len(q_lens) + 1, dtype=np.int32)
    qo_indptr[1:] = np.cumsum(q_lens)
    total_q = int(qo_indptr[-1])

    q32 = rng.standard_normal((total_q, num_qo_heads, head_dim_qk), dtype=np.float32)
    k32 = rng.standard_normal((pool, P, num_kv_heads, head_dim_qk), dtype=np.float32)
    v32 = None
    if not shared_kv:
        v32 = rng.standard_normal((pool, P, num_kv_heads, head_dim_vo), dtype=np.float32)

    if k_late_gain is not None:
        gain, d0, d1 = k_late_gain
        for b in range(len(kv_lens)):
            L = int(kv_lens[b])
            js = np.arange((L + 1) // 2, L)
            pages = kv_indices[kv_indptr[b] + js // P]
            k32[pages, js % P, :, d0:d1] *= np.float32(gain)

    k_scale = v_scale = 1.0
    if kv_dtype == DT_FP8:
        # one per-tensor scale per cache: s = amax/448 (computed in fp32)
        k_scale = float(np.float32(np.abs(k32).max()) / np.float32(FP8_MAX))
        k32 = k32 / np.float32(k_scale)
        if shared_kv:
            v_scale = k_scale
        else:
            v_scale = float(np.float32(np.abs(v32).max()) / np.float32(FP8_MAX))
            v32 = v32 / np.float32(v_scale)

    q_scale = 1.0
    if q_dtype == DT_FP8:
        # fp8 queries: one per-tensor scale, s = amax/448 (as for the caches)
        q_scale = float(np.float32(np.abs(q32).max()) / np.float32(FP8_MAX))
        q32 = q32 / np.float32(q_scale)
    q = round_to_storage(q32, q_dtype)
    del q32
    k = round_to_storage(k32, kv_dtype).reshape(k32.shape)
    del k32
    v = None
    if v32 is not None:
        v = round_to_storage(v32, kv_dtype).reshape(v32.shape)
        del v32

    if poison:
        used = np.zeros(pool, dtype=bool)
        used[kv_indices] = True
        for arr in (k, v):
            if arr is None:
                continue
            nan = np.float32("nan") if kv_dtype == DT_F32 else _NAN_CODE[kv_dtype]
            arr[~used] = nan
            for b in range(len(kv_lens)):
                if n_pages[b] > 0 and last[b] < P:
                    arr[kv_indices[kv_indptr[b + 1] - 1], last[b]:] = nan

    k_phys, k_stride = _layout_array(k, k_layout)
    del k
    if v is not None:
        v_phys, v_stride = _layout_array(v, v_layout)
        del v
    else:
        v_phys, v_stride = None, k_stride

    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(head_dim_qk)
    uq = int(q_lens[0]) if (uniform_q_len and len(set(q_lens.tolist())) == 1) else None
    return Workload(name=name, seed=seed, q=q, q_dtype=q_dtype, qo_indptr=qo_indptr, q_len=uq,
                    num_qo_heads=num_qo_heads, num_kv_heads=num_kv_heads,
                    head_dim_qk=head_dim_qk, head_dim_vo=head_dim_vo, page_size=P,
                    k=k_phys, v=v_phys, kv_dtype=kv_dtype, k_stride=tuple(int(s) for s in k_stride),
                    v_stride=tuple(int(s) for s in v_stride), k_scale=k_scale, v_scale=v_scale,
                    kv_indptr=kv_indptr, kv_indices=kv_indices, kv_last_page_len=last,
                    kv_lens=kv_lens, num_pool_pages=pool, kv_broadcast=kv_broadcast,
                    causal=causal, sm_scale=float(sm_scale), num_kv_splits=num_kv_splits,
                    k_layout=k_layout, v_layout=v_layout, q_scale=q_scale)


# ---------------------------------------------------------------------------
# The five workloads.  Seeds are 1000*config + sub-index.  Keyword overrides
# shrink a workload (fewer batches, shorter lengths) while keeping its shape
# family; the defaults are the full sizes.
# ---------------------------------------------------------------------------

def config1(poison: bool = True, **kw) -> Workload:
    """Tiny paged decode: 4 requests, q_len 1, 8 query / 2 KV heads, head_dim 64,
    page 16, KV lengths {37, 64, 100, 5}, pool of 32 pages, fp32, scale 1/8."""
    seed = 1000
    rng = np.random.default_rng(seed)
    kv_lens = kw.pop("kv_lens", [37, 64, 100, 5])
    return build(rng, seed, "c1_tiny_decode_f32", q_lens=[1] * len(kv_lens), kv_lens=kv_lens,
                 num_qo_heads=8, num_kv_heads=2, head_dim_qk=64, head_dim_vo=64, page_size=16,
                 q_dtype=DT_F32, kv_dtype=DT_F32, sm_scale=1.0 / 8.0,
                 pool_pages=kw.pop("pool_pages", 32), poison=poison, **kw)


def config2(batch: int = 64, min_len: int = 512, max_len: int = 8192, poison: bool = True,
            sub: int = 0, **kw) -> Workload:
    """Llama-70B-like GQA decode: q_len 1, 64 query / 8 KV heads, head_dim 128,
    bf16, page 16, KV lengths uniform in [512, 8192], separate K and V caches
    with identical strides."""
    seed = 2000 + sub
    rng = np.random.default_rng(seed)
    kv_lens = rng.integers(min_len, max_len, endpoint=True, size=batch)
    dt = kw.pop("dtype", DT_BF16)
    return build(rng, seed, "c2_gqa_decode", q_lens=[1] * batch, kv_lens=kv_lens,
                 num_qo_heads=kw.pop("num_qo_heads", 64), num_kv_heads=kw.pop("num_kv_heads", 8),
                 head_dim_qk=128, head_dim_vo=128, page_size=kw.pop("page_size", 16),
                 q_dtype=dt, kv_dtype=dt, poison=poison, **kw)


def config3(batch: int = 8, min_q: int = 512, max_q: int = 2048, max_prefix: int = 4096,
            poison: bool = True, sub: int = 0, **kw) -> Workload:
    """GPT-OSS-like batched causal prefill: new q_len uniform in [512, 2048]
    appended to an existing paged KV of length uniform in [0, 4096]; 32 query /
    8 KV heads, head_dim 128, bf16, page 16, causal over the total position."""
    seed = 3000 + sub
    rng = np.random.default_rng(seed)
    q_lens = rng.integers(min_q, max_q, endpoint=True, size=batch)
    prefix = rng.integers(0, max_prefix, endpoint=True, size=batch)
    dt = kw.pop("dtype", DT_BF16)
    return build(rng, seed, "c3_causal_prefill", q_lens=q_lens, kv_lens=prefix + q_lens,
                 num_qo_heads=kw.pop("num_qo_heads", 32), num_kv_heads=kw.pop("num_kv_heads", 8),
                 head_dim_qk=128, head_dim_vo=128, page_size=16, q_dtype=dt, kv_dtype=dt,
                 causal=kw.pop("causal", True), poison=poison, uniform_q_len=False, **kw)


C4_HEADS = (16, 128)
C4_QLENS = (1, 2, 4)


def config4(num_heads: int = 16, q_len: int = 1, kv_dtype: int = DT_BF16, batch: int = 32,
            min_len: int = 4096, max_len: int = 32768, poison: bool = True,
            q_dtype: int = DT_BF16, **kw) -> Workload:
    """MLA latent decode: q_len in {1,2,4} folded into heads, 16 or 128 query
    heads, one shared KV head of 576 dims (V = first 512), page 64, KV lengths
    uniform in [4096, 32768], bf16 or fp8-e4m3 KV with a per-tensor scale,
    scale 1/sqrt(192).  One draw per (heads, q_len); the fp8 variant is
    quantised from the same fp32 values.  ``q_dtype=DT_FP8`` (with fp8 KV):
    the queries are fp8-e4m3 codes with their own per-tensor scale too."""
    sub = C4_HEADS.index(num_heads) * len(C4_QLENS) + C4_QLENS.index(q_len)
    seed = 4000 + sub
    rng = np.random.default_rng(seed)
    kv_lens = rng.integers(min_len, max_len, endpoint=True, size=batch)
    qtag = "_fp8q" if q_dtype == DT_FP8 else ""
    return build(rng, seed, f"c4_mla_decode_h{num_heads}_q{q_len}_{DT_NAMES[kv_dtype]}{qtag}",
                 q_lens=[q_len] * batch, kv_lens=kv_lens, num_qo_heads=num_heads,
                 num_kv_heads=1, head_dim_qk=576, head_dim_vo=512, page_size=64,
                 q_dtype=q_dtype, kv_dtype=kv_dtype, shared_kv=True,
                 causal=kw.pop("causal", True), sm_scale=1.0 / math.sqrt(192.0),
                 poison=poison, **kw)


def config_sparse(num_heads: int = 16, kv_dtype: int = DT_BF16, batch: int = 128,
                  topk: int = 2048, pool_factor: int = 4, mla: bool = True,
                  poison: bool = True, sub: int = 0, **kw) -> Workload:
    """Sparse-selected KV decode: every query (q_len 1, one request each) attends
    only the ``topk`` token rows a sparse indexer picked for it, given as an
    index list into a token pool (page size 1, so kv_indices are token slots).
    The pool holds ``pool_factor`` times the selected rows; the selection of
    each query is a uniformly random set of distinct slots, in ascending slot
    order; rows nobody selected are poisoned (NaN) unless ``poison`` is off.
    MLA shape by default (576/512 shared latent rows, one KV head, scale
    1/sqrt(192), bf16 or fp8-e4m3 KV); ``mla=False`` gives a GQA shape (32 query
    / 8 KV heads, head_dim 128, bf16)."""
    seed = 6000 + sub
    rng = np.random.default_rng(seed)
    kv_lens = np.full(batch, topk, dtype=np.int64)
    if "kv_lens" in kw:
        kv_lens = np.asarray(kw.pop("kv_lens"), dtype=np.int64)
    pool = max(1, int(kv_lens.sum()) * pool_factor)
    if mla:
        w = build(rng, seed, f"sparse_mla_h{num_heads}_{DT_NAMES[kv_dtype]}", q_lens=[1] * len(kv_lens),
                  kv_lens=kv_lens, num_qo_heads=num_heads, num_kv_heads=1, head_dim_qk=576,
                  head_dim_vo=512, page_size=1, q_dtype=DT_BF16, kv_dtype=kv_dtype, shared_kv=True,
                  sm_scale=1.0 / math.sqrt(192.0), pool_pages=pool, poison=poison, **kw)
    else:
        w = build(rng, seed, "sparse_gqa", q_lens=[1] * len(kv_lens), kv_lens=kv_lens,
                  num_qo_heads=kw.pop("num_qo_heads", 32), num_kv_heads=kw.pop("num_kv_heads", 8),
                  head_dim_qk=128, head_dim_vo=128, page_size=1, q_dtype=kv_dtype,
                  kv_dtype=kv_dtype, pool_pages=pool, poison=poison, **kw)
    # an indexer emits its picks in position order
    for b in range(len(kv_lens)):
        seg = slice(int(w.kv_indptr[b]), int(w.kv_indptr[b + 1]))
        w.kv_indices[seg] = np.sort(w.kv_indices[seg])
    return w


def config5(num_queries: int = 128, kv_len: int = 131072, num_kv_splits: int = 16,
            poison: bool = True, **kw) -> Workload:
    """Shared-prefix split-KV decode with KV broadcast: 128 query batches
    (q_len 1) attend one KV batch of 131072 tokens; 32 query / 8 KV heads,
    head_dim 128, fp16, page 128, 16 split chunks merged by their LSE."""
    seed = 5000
    rng = np.random.default_rng(seed)
    return build(rng, seed, "c5_broadcast_split_decode", q_lens=[1] * num_queries,
                 kv_lens=[kv_len], num_qo_heads=32, num_kv_heads=8, head_dim_qk=128,
                 head_dim_vo=128, page_size=128, q_dtype=DT_F16, kv_dtype=DT_F16,
                 kv_broadcast=True, num_kv_splits=num_kv_splits, poison=poison, **kw)


def replicate_broadcast(w: Workload) -> Workload:
    """The same workload with the one shared KV batch's page list repeated for
    every query batch (zero-copy replication through the page table)."""
    assert w.kv_broadcast
    nb = w.batch
    n0 = int(w.kv_indptr[1])
    indptr = (np.arange(nb + 1, dtype=np.int32) * n0).astype(np.int32)
    indices = np.tile(w.kv_indices[:n0], nb).astype(np.int32)
    last = np.repeat(w.kv_last_page_len[:1], nb).astype(np.int32)
    lens = np.repeat(w.kv_lens[:1], nb)
    import dataclasses
    return dataclasses.replace(w, name=w.name + "_replicated", kv_indptr=indptr,
                               kv_indices=indices, kv_last_page_len=last, kv_lens=lens,
                               kv_broadcast=False)
