"""Upload a seeded workload to the GPU and run it through the C ABI.

Marshalling only: tensors are created with torch (host -> device copies of the
workload's raw bytes), and every computation is a call into libpaged_attn.so
through ``binding``.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import binding as B
from . import workloads as W


@dataclass
class DeviceWorkload:
    w: W.Workload
    q: torch.Tensor
    k: torch.Tensor          # logical [pool, P, Hkv, Dqk] view (strides per layout)
    v: Optional[torch.Tensor]
    kv_indptr: torch.Tensor
    kv_indices: torch.Tensor
    kv_last: torch.Tensor
    qo_indptr: torch.Tensor

    @property
    def is_decode(self) -> bool:
        return self.w.q_len is not None


def _cache_view(flat: torch.Tensor, stride, pool, P, H, D) -> torch.Tensor:
    return torch.as_strided(flat, (pool, P, H, D), (stride[0], stride[1], stride[2], 1))


def upload(w: W.Workload, device: str = "cuda") -> DeviceWorkload:
    q = W.as_torch(w.q, w.q_dtype).to(device)
    kflat = W.as_torch(w.k.reshape(-1), w.kv_dtype).to(device)
    k = _cache_view(kflat, w.k_stride, w.num_pool_pages, w.page_size, w.num_kv_heads,
                    w.head_dim_qk)
    v = None
    if w.v is not None:
        vflat = W.as_torch(w.v.reshape(-1), w.kv_dtype).to(device)
        v = _cache_view(vflat, w.v_stride, w.num_pool_pages, w.page_size, w.num_kv_heads,
                        w.head_dim_vo)
    ix = w.kv_indices if w.kv_indices.size else np.zeros(1, np.int32)
    return DeviceWorkload(
        w=w, q=q, k=k, v=v,
        kv_indptr=torch.from_numpy(w.kv_indptr.astype(np.int32)).to(device),
        kv_indices=torch.from_numpy(ix.astype(np.int32)).to(device),
        kv_last=torch.from_numpy(w.kv_last_page_len.astype(np.int32)).to(device),
        qo_indptr=torch.from_numpy(w.qo_indptr.astype(np.int32)).to(device))


def run(d: DeviceWorkload, *, num_kv_splits: Optional[int] = None, merge: bool = True,
        flags: int = 0, out_dtype=None, return_max: bool = True, stream=None,
        max_kv_len: Optional[int] = None, force_prefill: bool = False):
    """One call of the hot path on the device workload.

    Decode-shaped workloads go through paged_attn_decode (with S split states
    then merge_states when S > 1 and ``merge``), the ragged ones through
    paged_attn_prefill.  Returns a dict of device tensors: o, lse, mx and, for
    split runs, the partial states po, plse.
    """
    w = d.w
    S = w.num_kv_splits if num_kv_splits is None else num_kv_splits
    kvdt = w.kv_dtype
    hint = int(w.kv_lens.max()) if max_kv_len is None else max_kv_len
    common = dict(head_dim_vo=w.head_dim_vo, kv_dtype=kvdt, k_scale=w.k_scale,
                  v_scale=w.v_scale, q_scale=w.q_scale, max_kv_len=hint, flags=flags, stream=stream,
                  sm_scale=w.sm_scale, causal=w.causal, kv_broadcast=w.kv_broadcast)
    res = {}
    if d.is_decode and not force_prefill:
        q4 = d.q.view(w.batch, w.q_len, w.num_qo_heads, w.head_dim_qk)
        o, lse, mx = B.decode(q4, d.k, d.v, d.kv_indptr, d.kv_indices, d.kv_last,
                              num_kv_splits=S, return_max=True,
                              out_dtype=out_dtype if S == 1 else None, **common)
        if S > 1:
            res["po"], res["plse"], res["pmx"] = o, lse, mx
            if merge:
                odt = out_dtype or (d.q.dtype if d.q.dtype in (torch.float16, torch.bfloat16)
                                    else torch.bfloat16 if d.q.dtype != torch.float32
                                    else torch.float32)
                o, lse = B.merge_states(o, lse, out_dtype=odt, stream=stream)
                mx = None
        res["o"], res["lse"], res["mx"] = o, lse, mx
        return res
    o, lse, mx = B.prefill(d.q, d.qo_indptr, d.k, d.v, d.kv_indptr, d.kv_indices, d.kv_last,
                           return_max=True, out_dtype=out_dtype,
                           max_q_len=int(w.q_lens().max()), **common)
    res["o"], res["lse"], res["mx"] = o, lse, mx
    return res


def as_rows(t: torch.Tensor, w: W.Workload) -> np.ndarray:
    """Device output -> float64 numpy with rows (t*Hq + h) flattened on axis 0 (or 1
    for split states)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


class Step:
    """One step of the hot path on a device workload, marshalled once.

    Decode-shaped workloads: one paged_attn_decode call (with the workload's
    explicit split count S; S > 1 adds one merge_states call).  Ragged ones:
    one paged_attn_prefill call.
    """

    def __init__(self, d: DeviceWorkload, flags: int = 0, stream=None):
        import torch
        w = d.w
        self.w = w
        self.stream = stream or torch.cuda.current_stream()
        S = w.num_kv_splits
        self.num_states = S
        common = dict(head_dim_vo=w.head_dim_vo, kv_dtype=w.kv_dtype, k_scale=w.k_scale,
                      v_scale=w.v_scale, q_scale=w.q_scale, max_kv_len=int(w.kv_lens.max()),
                      flags=flags,
                      stream=self.stream, sm_scale=w.sm_scale, causal=w.causal,
                      kv_broadcast=w.kv_broadcast)
        self.merge = None
        if d.is_decode:
            q4 = d.q.view(w.batch, w.q_len, w.num_qo_heads, w.head_dim_qk)
            self.attn = B.prepare_decode(q4, d.k, d.v, d.kv_indptr, d.kv_indices, d.kv_last,
                                         num_kv_splits=S, **common)
            if S > 1:
                po, pl = self.attn.outputs["o"], self.attn.outputs["lse"]
                odt = d.q.dtype if d.q.dtype != torch.float8_e4m3fn else torch.bfloat16
                self.final_o = torch.empty(po.shape[1:], dtype=odt, device=po.device)
                self.final_lse = torch.empty(pl.shape[1:], dtype=torch.float32, device=po.device)
                lib = B.load_library()
                rows = pl[0].numel()
                args = (po.data_ptr(), B.PA_F32, pl.data_ptr(), S, rows, w.head_dim_vo,
                        self.final_o.data_ptr(), B._pa_dtype(self.final_o),
                        self.final_lse.data_ptr(), B._stream_handle(self.stream))
                self.merge = lambda: B._check("merge_states", lib.merge_states(*args))
        else:
            self.attn = B.prepare_prefill(d.q, d.qo_indptr, d.k, d.v, d.kv_indptr, d.kv_indices,
                                          d.kv_last, max_q_len=int(w.q_lens().max()), **common)
        self.attention_kernel_name = self.attn.plan_name

    def __call__(self):
        self.attn()
        if self.merge is not None:
            self.merge()

    def time_attention_kernel(self, steps: int) -> float:
        """Average ms of the attention kernel alone over ``steps`` full steps: the
        library records a HIP event pair around that launch on its stream (any
        merge launch of the step falls outside the pair)."""
        import torch
        hip = _hip()
        pairs = []
        for _ in range(steps):
            e0, e1 = ctypes.c_void_p(), ctypes.c_void_p()
            if hip.hipEventCreate(ctypes.byref(e0)) or hip.hipEventCreate(ctypes.byref(e1)):
                raise RuntimeError("hipEventCreate failed")
            pairs.append((e0, e1))
        torch.cuda.synchronize()
        for e0, e1 in pairs:
            self.attn.args.timing_events[0] = e0.value
            self.attn.args.timing_events[1] = e1.value
            self()
        self.attn.args.timing_events[0] = None
        self.attn.args.timing_events[1] = None
        torch.cuda.synchronize()
        total = 0.0
        for e0, e1 in pairs:
            ms = ctypes.c_float()
            if hip.hipEventElapsedTime(ctypes.byref(ms), e0, e1):
                raise RuntimeError("hipEventElapsedTime failed")
            total += ms.value
            hip.hipEventDestroy(e0)
            hip.hipEventDestroy(e1)
        return total / steps


_HIP = None


def _hip():
    """The HIP runtime, for event handles only."""
    global _HIP
    if _HIP is None:
        lib = ctypes.CDLL("libamdhip64.so")
        lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                            ctypes.c_void_p]
        lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _HIP = lib
    return _HIP


def prepare(d: DeviceWorkload, flags: int = 0, stream=None) -> Step:
    return Step(d, flags=flags, stream=stream)
