"""Thin ctypes binding of libpaged_attn.so (declarations in include/paged_attn.h).

Argument marshalling only: torch tensors supply device pointers, strides and
the current HIP stream; every step of the computation runs in the library's
kernels.  The only torch calls on device memory are allocations of outputs
and workspace (``torch.empty``).  There is no fallback: if the library is not
built, every entry point raises.
"""
from __future__ import annotations

import ctypes
import math
import os
import re
from typing import Optional

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpaged_attn.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "paged_attn.h")

PA_F32, PA_F16, PA_BF16, PA_FP8_E4M3 = 0, 1, 2, 3
FLAG_FORCE_GENERAL_STRIDES = 0x1
FLAG_FORCE_GENERIC = 0x2
FLAG_NO_INTERNAL_SPLIT = 0x4
NOALLOC_SCRATCH_BYTES = 128 << 20  # PA_NOALLOC_SCRATCH_BYTES

_TORCH_TO_PA = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16,
                torch.float8_e4m3fn: PA_FP8_E4M3}
_PA_TO_TORCH = {PA_F32: torch.float32, PA_F16: torch.float16, PA_BF16: torch.bfloat16}

c_i32, c_i64, c_f32, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p


class PagedKV(ctypes.Structure):
    _fields_ = [("k", c_vp), ("v", c_vp), ("k_stride", c_i64 * 3), ("v_stride", c_i64 * 3),
                ("num_kv_heads", c_i32), ("page_size", c_i32), ("head_dim_qk", c_i32),
                ("head_dim_vo", c_i32), ("kv_dtype", ctypes.c_int), ("k_scale", c_f32),
                ("v_scale", c_f32), ("kv_indptr", c_vp), ("kv_indices", c_vp),
                ("kv_last_page_len", c_vp), ("num_kv_batches", c_i32),
                ("max_kv_len_hint", c_i32)]


class DecodeArgs(ctypes.Structure):
    _fields_ = [("q", c_vp), ("q_dtype", ctypes.c_int), ("batch", c_i32), ("q_len", c_i32),
                ("num_qo_heads", c_i32), ("kv", PagedKV), ("kv_broadcast", c_i32),
                ("causal", c_i32), ("sm_scale", c_f32), ("num_kv_splits", c_i32), ("o", c_vp),
                ("o_dtype", ctypes.c_int), ("lse", c_vp), ("row_max", c_vp),
                ("flags", ctypes.c_uint32), ("timing_events", c_vp * 2), ("q_scale", c_f32)]


class PrefillArgs(ctypes.Structure):
    _fields_ = [("q", c_vp), ("q_dtype", ctypes.c_int), ("qo_indptr", c_vp), ("batch", c_i32),
                ("total_q", c_i32), ("max_q_len_hint", c_i32), ("num_qo_heads", c_i32),
                ("kv", PagedKV), ("kv_broadcast", c_i32), ("causal", c_i32),
                ("sm_scale", c_f32), ("o", c_vp), ("o_dtype", ctypes.c_int), ("lse", c_vp),
                ("row_max", c_vp), ("flags", ctypes.c_uint32), ("timing_events", c_vp * 2),
                ("q_scale", c_f32)]


class PagedAttnError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: status {status} ({msg})")
        self.status = status


_lib = None


def header_functions():
    """Names of the functions include/paged_attn.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


def load_library(path: str = LIB_PATH):
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; build it with `python -m paged_kv_attention_prefill_amd.build`")
    lib = ctypes.CDLL(path)
    lib.pa_abi_version.restype = ctypes.c_int
    lib.pa_abi_version.argtypes = []
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_status_string.argtypes = [ctypes.c_int]
    lib.paged_attn_decode_workspace_size.restype = ctypes.c_int
    lib.paged_attn_decode_workspace_size.argtypes = [ctypes.POINTER(DecodeArgs),
                                                     ctypes.POINTER(ctypes.c_size_t)]
    lib.paged_attn_prefill_workspace_size.restype = ctypes.c_int
    lib.paged_attn_prefill_workspace_size.argtypes = [ctypes.POINTER(PrefillArgs),
                                                      ctypes.POINTER(ctypes.c_size_t)]
    lib.paged_attn_decode.restype = ctypes.c_int
    lib.paged_attn_decode.argtypes = [ctypes.POINTER(DecodeArgs), c_vp, ctypes.c_size_t, c_vp]
    lib.paged_attn_prefill.restype = ctypes.c_int
    lib.paged_attn_prefill.argtypes = [ctypes.POINTER(PrefillArgs), c_vp, ctypes.c_size_t, c_vp]
    lib.paged_attn_decode_noalloc.restype = ctypes.c_int
    lib.paged_attn_decode_noalloc.argtypes = [ctypes.POINTER(DecodeArgs), c_vp]
    lib.merge_states.restype = ctypes.c_int
    lib.merge_states.argtypes = [c_vp, ctypes.c_int, c_vp, c_i32, c_i64, c_i32, c_vp,
                                 ctypes.c_int, c_vp, c_vp]
    for nm, st in (("paged_attn_decode_plan_name", DecodeArgs),
                   ("paged_attn_prefill_plan_name", PrefillArgs)):
        getattr(lib, nm).restype = ctypes.c_char_p
        getattr(lib, nm).argtypes = [ctypes.POINTER(st)]
    lib.paged_attn_check_tables.restype = ctypes.c_int
    lib.paged_attn_check_tables.argtypes = [c_vp, c_vp, c_vp, c_i32, c_i32, c_i32]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().pa_status_string(status).decode()


def _check(fn: str, status: int):
    if status != 0:
        raise PagedAttnError(fn, status, status_string(status))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _pa_dtype(t: torch.Tensor, explicit: Optional[int] = None) -> int:
    if explicit is not None:
        return explicit
    if t.dtype not in _TORCH_TO_PA:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _TORCH_TO_PA[t.dtype]


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def make_paged_kv(k_cache: torch.Tensor, v_cache: Optional[torch.Tensor], kv_indptr, kv_indices,
                  kv_last_page_len, *, head_dim_vo: Optional[int] = None, kv_dtype=None,
                  k_scale: float = 1.0, v_scale: float = 1.0, max_kv_len: int = 0) -> PagedKV:
    """k_cache / v_cache: logical [pages, page_size, num_kv_heads, head_dim] views of any
    strides with a unit innermost stride.  v_cache None: shared latent rows (V = first
    head_dim_vo dims of K)."""
    if k_cache.dim() != 4:
        raise ValueError("k_cache must be a [pages, page_size, kv_heads, head_dim] view")
    shared = v_cache is None
    vc = k_cache if shared else v_cache
    kv = PagedKV()
    kv.k = k_cache.data_ptr()
    kv.v = vc.data_ptr()
    for i in range(3):
        kv.k_stride[i] = k_cache.stride(i)
        kv.v_stride[i] = vc.stride(i)
    kv.num_kv_heads = k_cache.shape[2]
    kv.page_size = k_cache.shape[1]
    kv.head_dim_qk = k_cache.shape[3]
    kv.head_dim_vo = head_dim_vo if head_dim_vo is not None else vc.shape[3]
    kv.kv_dtype = _pa_dtype(k_cache, kv_dtype)
    kv.k_scale = k_scale
    kv.v_scale = v_scale
    kv.kv_indptr = kv_indptr.data_ptr()
    kv.kv_indices = kv_indices.data_ptr()
    kv.kv_last_page_len = kv_last_page_len.data_ptr()
    kv.num_kv_batches = kv_indptr.numel() - 1
    kv.max_kv_len_hint = int(max_kv_len)
    return kv


class PreparedCall:
    """A validated argument struct with its outputs and workspace allocated once;
    calling it enqueues the entry point again on the stream (no re-marshalling)."""

    def __init__(self, fn_name: str, args, outputs: dict, workspace: Optional[torch.Tensor],
                 ws_bytes: int, stream):
        self.lib = load_library()
        self.fn_name = fn_name
        self.fn = getattr(self.lib, fn_name)
        self.args = args
        self.outputs = outputs
        self.workspace = workspace
        self.ws_bytes = ws_bytes
        self.stream = _stream_handle(stream)
        self._ref = ctypes.byref(args)
        self._ws = _ptr(workspace) if ws_bytes else None
        plan = "paged_attn_prefill_plan_name" if fn_name == "paged_attn_prefill" \
            else "paged_attn_decode_plan_name"
        name = getattr(self.lib, plan)(self._ref)
        self.plan_name = name.decode() if name else None

    def __call__(self):
        if self.fn_name == "paged_attn_decode_noalloc":
            _check(self.fn_name, self.fn(self._ref, self.stream))
        else:
            _check(self.fn_name, self.fn(self._ref, self._ws, self.ws_bytes, self.stream))
        return self.outputs


def _workspace(lib, size_fn, args, device, workspace):
    ws_bytes = ctypes.c_size_t(0)
    _check(size_fn, getattr(lib, size_fn)(ctypes.byref(args), ctypes.byref(ws_bytes)))
    n = ws_bytes.value
    if n > 0 and (workspace is None or workspace.numel() < n):
        # every workspace byte a kernel reads was written earlier in the same
        # call, so the buffer needs no initial contents
        workspace = torch.empty(n, dtype=torch.uint8, device=device)
    return workspace, n


def prepare_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: Optional[torch.Tensor],
                   kv_indptr: torch.Tensor, kv_indices: torch.Tensor,
                   kv_last_page_len: torch.Tensor, *, causal: bool = False,
                   sm_scale: Optional[float] = None, kv_broadcast: bool = False,
                   num_kv_splits: int = 1, out_dtype: Optional[torch.dtype] = None,
                   head_dim_vo: Optional[int] = None, kv_dtype: Optional[int] = None,
                   k_scale: float = 1.0, v_scale: float = 1.0, q_scale: float = 1.0,
                   return_max: bool = False,
                   max_kv_len: int = 0, flags: int = 0, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                   stream=None, noalloc: bool = False) -> PreparedCall:
    """Validate and marshal one paged decode; see ``decode``.  ``noalloc``: call
    paged_attn_decode_noalloc (the library's own scratch array is the workspace)."""
    lib = load_library()
    if q.dim() != 4 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [batch, q_len, heads, head_dim] tensor")
    batch, q_len, hq, dqk = q.shape
    kv = make_paged_kv(k_cache, v_cache, kv_indptr, kv_indices, kv_last_page_len,
                       head_dim_vo=head_dim_vo, kv_dtype=kv_dtype, k_scale=k_scale,
                       v_scale=v_scale, max_kv_len=max_kv_len)
    dvo = kv.head_dim_vo
    S = int(num_kv_splits)
    if out_dtype is None:
        out_dtype = torch.float32 if S > 1 else (q.dtype if q.dtype in _PA_TO_TORCH.values()
                                                 else torch.bfloat16)
    lead = (S,) if S > 1 else ()
    if out is None:
        out = torch.empty(lead + (batch, q_len, hq, dvo), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty(lead + (batch, q_len, hq), dtype=torch.float32, device=q.device)
    mx = torch.empty_like(lse) if return_max else None
    a = DecodeArgs()
    a.q = q.data_ptr()
    a.q_dtype = _pa_dtype(q)
    a.batch, a.q_len, a.num_qo_heads = batch, q_len, hq
    a.kv = kv
    a.kv_broadcast = int(kv_broadcast)
    a.causal = int(causal)
    a.sm_scale = float(sm_scale if sm_scale is not None else 1.0 / math.sqrt(dqk))
    a.num_kv_splits = S
    a.o = out.data_ptr()
    a.o_dtype = _pa_dtype(out)
    a.lse = _ptr(lse)
    a.row_max = _ptr(mx)
    a.flags = flags
    a.q_scale = q_scale
    keep = dict(o=out, lse=lse, mx=mx, _q=q, _k=k_cache, _v=v_cache, _ip=kv_indptr,
                _ix=kv_indices, _lp=kv_last_page_len)
    if noalloc:
        return PreparedCall("paged_attn_decode_noalloc", a, keep, None, 0, stream)
    workspace, n = _workspace(lib, "paged_attn_decode_workspace_size", a, q.device, workspace)
    return PreparedCall("paged_attn_decode", a, keep, workspace, n, stream)


def decode(*args, return_max: bool = False, **kw):
    """Paged decode.  q: [batch, q_len, num_qo_heads, head_dim_qk].
    Returns (o, lse[, max]); with num_kv_splits = S > 1 the outputs carry a leading
    S axis of fp32 partial states (merge them with ``merge_states``)."""
    out = prepare_decode(*args, return_max=return_max, **kw)()
    return (out["o"], out["lse"], out["mx"]) if return_max else (out["o"], out["lse"])


def prepare_prefill(q: torch.Tensor, qo_indptr: torch.Tensor, k_cache: torch.Tensor,
                    v_cache: Optional[torch.Tensor], kv_indptr: torch.Tensor,
                    kv_indices: torch.Tensor, kv_last_page_len: torch.Tensor, *,
                    causal: bool = True, sm_scale: Optional[float] = None,
                    kv_broadcast: bool = False, out_dtype: Optional[torch.dtype] = None,
                    head_dim_vo: Optional[int] = None, kv_dtype: Optional[int] = None,
                    k_scale: float = 1.0, v_scale: float = 1.0, q_scale: float = 1.0,
                    return_max: bool = False,
                    max_q_len: int = 0, max_kv_len: int = 0, flags: int = 0,
                    workspace: Optional[torch.Tensor] = None, stream=None) -> PreparedCall:
    """Validate and marshal one paged prefill; see ``prefill``."""
    lib = load_library()
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [total_q, heads, head_dim] tensor")
    total_q, hq, dqk = q.shape
    kv = make_paged_kv(k_cache, v_cache, kv_indptr, kv_indices, kv_last_page_len,
                       head_dim_vo=head_dim_vo, kv_dtype=kv_dtype, k_scale=k_scale,
                       v_scale=v_scale, max_kv_len=max_kv_len)
    dvo = kv.head_dim_vo
    if out_dtype is None:
        out_dtype = q.dtype if q.dtype in _PA_TO_TORCH.values() else torch.bfloat16
    out = torch.empty((total_q, hq, dvo), dtype=out_dtype, device=q.device)
    lse = torch.empty((total_q, hq), dtype=torch.float32, device=q.device)
    mx = torch.empty_like(lse) if return_max else None
    a = PrefillArgs()
    a.q = q.data_ptr()
    a.q_dtype = _pa_dtype(q)
    a.qo_indptr = qo_indptr.data_ptr()
    a.batch = qo_indptr.numel() - 1
    a.total_q = total_q
    a.max_q_len_hint = int(max_q_len)
    a.num_qo_heads = hq
    a.kv = kv
    a.kv_broadcast = int(kv_broadcast)
    a.causal = int(causal)
    a.sm_scale = float(sm_scale if sm_scale is not None else 1.0 / math.sqrt(dqk))
    a.o = out.data_ptr()
    a.o_dtype = _pa_dtype(out)
    a.lse = lse.data_ptr()
    a.row_max = _ptr(mx)
    a.flags = flags
    a.q_scale = q_scale
    workspace, n = _workspace(lib, "paged_attn_prefill_workspace_size", a, q.device, workspace)
    keep = dict(o=out, lse=lse, mx=mx, _q=q, _qo=qo_indptr, _k=k_cache, _v=v_cache,
                _ip=kv_indptr, _ix=kv_indices, _lp=kv_last_page_len)
    return PreparedCall("paged_attn_prefill", a, keep, workspace, n, stream)


def prefill(*args, return_max: bool = False, **kw):
    """Paged prefill.  q: [total_q, num_qo_heads, head_dim_qk] ragged by qo_indptr.
    Returns (o, lse[, max])."""
    out = prepare_prefill(*args, return_max=return_max, **kw)()
    return (out["o"], out["lse"], out["mx"]) if return_max else (out["o"], out["lse"])


def merge_states(v_states: torch.Tensor, s_states: torch.Tensor, *,
                 out_dtype: Optional[torch.dtype] = None, stream=None):
    """v_states [S, rows..., D] (fp32/f16/bf16), s_states [S, rows...] fp32 LSE ->
    (v [rows..., D], s [rows...])."""
    lib = load_library()
    if not (v_states.is_contiguous() and s_states.is_contiguous()):
        raise ValueError("merge_states needs contiguous inputs")
    S = v_states.shape[0]
    D = v_states.shape[-1]
    rows = s_states[0].numel()
    out_dtype = out_dtype or v_states.dtype
    out = torch.empty(v_states.shape[1:], dtype=out_dtype, device=v_states.device)
    s_out = torch.empty(s_states.shape[1:], dtype=torch.float32, device=v_states.device)
    _check("merge_states", lib.merge_states(v_states.data_ptr(), _pa_dtype(v_states),
                                            s_states.data_ptr(), S, rows, D, out.data_ptr(),
                                            _pa_dtype(out), s_out.data_ptr(),
                                            _stream_handle(stream)))
    return out, s_out
